// fa_bwd.hip — backward kernels of exact tiled attention for gfx950.
//
// Recomputation ([ODP] "FlashAttention: Fast and Memory-Efficient Exact
// Attention with IO-Awareness", section "The key idea"; [DEC]
// "FlashAttention, Decoded", "The Hardware Picture: Why Tiling Wins"): the
// probabilities are never stored.  Each tile pair rebuilds
// P = exp(scale * q.k - lse) on-chip from Q, K and the forward's per-row
// log-sum-exp, so the backward reads O(N d) from HBM per pass and writes
// only dQ, dK, dV.
//
// Gradients (chain rule through the row softmax; the pages do not print
// them): dV = P^T dO, dP = dO V^T, dS = P * (dP - D) with
// D_i = sum_c dO_ic O_ic (= sum_j P_ij dP_ij), dQ = scale dS K,
// dK = scale dS^T Q.
//
// Stages (deterministic: no atomics):
//   bwd_pre   per query row: D and the base-2 softmax shift lse*log2(e)
//             (+inf for rows without keys), into the workspace, and each
//             workgroup's maxima of |Q|, |K|, |V|, |dO|; bwd_convert
//             reduces those to per-(b, h) maxima and writes the scaled
//             fp16 copies of Q, K, dO and the scaled row terms described
//             below;
//   bwd_dkdv  one workgroup per 128 keys (32 per wave); query tiles of 64
//             rows (Q, dO, row terms) are double buffered in LDS.  With
//             v_mfma_f32_32x32x16, S = Q K^T and dP = dO V^T come out with
//             the key in the lane's column, so P and dS rounded to 16 bits
//             are directly the k-operands of dV^T += dO^T P and
//             dK^T += Q^T dS (dO^T and Q^T via the LDS transpose read);
//   bwd_dq    one workgroup per 128 queries (32 per wave); key tiles of 64
//             rows (K, V) double buffered in LDS: S^T = K Q^T and
//             dP^T = V dO^T keep the query in the lane's column, and
//             dQ^T += K^T dS^T.
// LDS tiles are XOR-swizzled (conflict-free row and transpose reads) and
// filled by direct global->LDS copies one tile ahead of the compute.
//
// The products run on fp16 operands for both input types.  Rounding
// P and dS to bf16 (8 significant bits) before dV = P^T dO and dK = dS^T Q
// costs up to ~0.01 absolute in the gradients, next to the output
// rounding; fp16 keeps 11 bits.  The D pass also finds max |Q|, |K|, |V|,
// |dO| per (b, h); a convert pass writes c Q * 2^-eq (c = scale * log2 e)
// and dO * 2^-eo as fp16, and -shift * 2^-f, -D * 2^-(eo+ev) per row; the
// dK/dV kernel converts its K and V rows the same way (* 2^-ek, * 2^-ev).
// The power-of-two exponents keep every operand in fp16 range (max |dO'|
// in [2^3, 2^4), |V'| in [2^2, 2^3), so |dP'|, |D'| < 2^14 and |dS'| < 2^15
// for d <= 128; |c Q'|, |K'| <= 2^14) and fold back exactly into the output
// scaling.  The dQ kernel forms dP from the unscaled dO and V and gives P
// the same factor 2^-(eo+ev) through its row term, so the dS it rounds to
// fp16 is the same scaled dS' with the same bound.  eq and ek are split so that f = eq + ek = 0 whenever the
// geometric mean of max |c Q| and max |K| lies in [2^-4, 2^13]: then the
// score accumulator, started at -shift, is exactly the exponent of P, and
// the dP accumulator, started at -D, is exactly dP - D, so P costs one
// exponential and dS one multiply.  Heads whose maxima allow large logits
// (c max|Q| max|K| sqrt(d) > 64) leave c out of the Q copy, which rounding
// c Q to fp16 would make inexact by ~2^-11 |c q.k| in the exponent, and
// multiply the score accumulator by c 2^f in fp32 instead (see Scales).
// fp16 inputs need no Q and K copies: their products are exact as given,
// so those kernels use Q and K themselves in that exact mode, and the D
// pass copies only dO (see use_raw).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace bwd {

#ifndef FA_BWD_SNAKE
#define FA_BWD_SNAKE 0  // snake workgroup order in the causal dK/dV and dQ kernels
#endif

constexpr int kBKV = 128;      // keys per dK/dV workgroup (= block-sparse block)
constexpr int kBQ = 64;        // query rows per LDS tile in the dK/dV kernel
constexpr int kBR = 128;       // queries per dQ workgroup (= block-sparse block)
constexpr int kBC = 64;        // key rows per LDS tile in the dQ kernel
constexpr int kListMax = 1024; // block-sparse: active blocks listed per pass

template <typename T> constexpr bool kIsBf16 = false;
template <> constexpr bool kIsBf16<__bf16> = true;

template <typename T> __device__ __forceinline__ float to_f32(uint32_t bits16);
template <> __device__ __forceinline__ float to_f32<__bf16>(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}
template <> __device__ __forceinline__ float to_f32<_Float16>(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

__device__ __forceinline__ int valid_keys(const int32_t* key_len, int b, int N) {
  if (!key_len) return N;
  int kl = key_len[b];
  return kl < 0 ? 0 : (kl > N ? N : kl);
}

// Exponent e with max * 2^-e in [2^t, 2^(t+1)) for the float bit pattern
// `maxbits` of a non-negative maximum; 0 for a zero tensor; clamped so that
// every scale stays a normal float.
__device__ __forceinline__ int scale_exp(uint32_t maxbits, int t) {
  if (maxbits == 0u) return 0;
  const int e = (int)((maxbits >> 23) & 0xffu) - 127 - t;
  return e < -60 ? -60 : (e > 60 ? 60 : e);
}
constexpr int kTq = 13, kTk = 13, kTo = 3, kTv = 2;  // targets: max' in [2^t, 2^(t+1))

__device__ __forceinline__ int exp_of(uint32_t bits) { return (int)((bits >> 23) & 0xffu) - 127; }
__device__ __forceinline__ int clamp60(int e) { return e < -60 ? -60 : (e > 60 ? 60 : e); }

// Per-(b, h) exponents of the fp16 operands of the products:
// Q'' = c Q 2^-eq (exact: Q 2^-eq), K' = K 2^-ek, V' = V 2^-ev,
// dO' = dO 2^-eo, and c S = m S'' with m = 2^f (exact: c 2^f), f = eq + ek.
// Folding c into the fp16 copy of Q rounds c Q to 11 bits, which moves a
// score by about 2^-11 |c q.k| / sqrt(d) in base-2 units: nothing for
// ordinary logits, but percent-level errors in P once |c q.k| reaches the
// hundreds.  A head whose maxima allow that (c max|Q| max|K| sqrt(d) > 64)
// is "exact": its Q copy is only scaled by a power of two (exact), and the
// score accumulator is multiplied by m in fp32 (one multiply per score).
struct Scales {
  int eq, ek, ev, eo, f;
  bool exact;  // c not folded into the Q copy
  bool mul;    // the score accumulator needs the factor m (m != 1)
  float m;     // c S = m S''
};

// mx: max |Q|, |K|, |V|, |dO| of the (b, h) as float bit patterns
template <int D>
__device__ __forceinline__ Scales bwd_scales_of(uint32_t mxq, uint32_t mxk, uint32_t mxv,
                                                uint32_t mxo, float c) {
  Scales s;
  const float qmax = __builtin_bit_cast(float, mxq);
  const float kmax = __builtin_bit_cast(float, mxk);
  const float bound = c * qmax * kmax;
  s.exact = bound * bound * (float)D > 4096.f;
  const uint32_t mq = __builtin_bit_cast(uint32_t, s.exact ? qmax : c * qmax);
  const uint32_t mk = mxk;
  s.ev = scale_exp(mxv, kTv);
  s.eo = scale_exp(mxo, kTo);
  if (mq == 0u || mk == 0u) {
    s.eq = s.ek = 0;
  } else {
    const int Eq = exp_of(mq), Ek = exp_of(mk), g = Eq + Ek;
    if (g >= -8 && g <= 26) {  // balanced: both maxima near 2^(g/2), eq + ek = 0
      const int d = Eq - Ek;
      s.eq = clamp60(d >= 0 ? d / 2 : -((-d + 1) / 2));  // floor(d / 2)
      s.ek = -s.eq;
    } else {
      s.eq = clamp60(Eq - kTq);
      s.ek = clamp60(Ek - kTk);
    }
  }
  s.f = s.eq + s.ek;
  s.m = s.exact ? ldexpf(c, s.f) : ldexpf(1.f, s.f);
  s.mul = s.exact || s.f != 0;
  return s;
}


// The raw path's scales: Q and K enter the products unscaled (in the
// input type, exactly), so c multiplies the score accumulator in fp32
// (exact mode, m = c, f = 0); dO and V keep their power-of-two scales (the
// fp16 copy of dO, V converted in registers), from their maxima alone.
__device__ __forceinline__ Scales raw_scales_of(uint32_t mxv, uint32_t mxo, float c) {
  Scales s;
  s.eq = s.ek = s.f = 0;
  s.ev = scale_exp(mxv, kTv);
  s.eo = scale_exp(mxo, kTo);
  s.exact = true;
  s.mul = true;
  s.m = c;
  return s;
}

// largest |x| of the 8 16-bit values in a 16-byte chunk, as float bits
// (magnitude bit patterns of both formats order like the values)
template <typename T>
__device__ __forceinline__ uint32_t absmax8(u32x4 a) {
  uint32_t m = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = a[j] & 0x7fffu, hi = (a[j] >> 16) & 0x7fffu;
    m = m > lo ? m : lo;
    m = m > hi ? m : hi;
  }
  return __builtin_bit_cast(uint32_t, to_f32<T>(m));
}

// ---------------------------------------------------------------------------
// Per row: D_i = sum_c dO_ic O_ic and shift_i = lse_i * log2(e) (+inf when
// the row saw no key, so that exp2(c s - shift) = 0 there).  STATS: also
// max |Q|, |K|, |V|, |dO| of the workgroup's rows, stored as its partial
// maxima part[4][BH][kPreChunks] (no atomics, so nothing has to be cleared
// first: the convert pass reduces exactly the gridDim.y partials that this
// launch wrote).  Grid (B*H, chunks of `iters` row groups): a workgroup
// stays inside one (b, h).
// ---------------------------------------------------------------------------

// threads per row in the D pass: one per 8 elements (16 bytes), rounded up
// to a power of two for the shuffle reduction (d = 96: 16, the last 4 idle)
template <int D>
constexpr int pre_tpr() {
  return D / 8 <= 4 ? 4 : D / 8 <= 8 ? 8 : 16;
}

template <typename T, int D, bool STATS, bool RAW>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* o, const uint16_t* dO,
                                                      const float* lse, const uint16_t* q,
                                                      const uint16_t* k, const uint16_t* v,
                                                      float* Dbuf, float* shift,
                                                      uint32_t* part, int N, int BH,
                                                      int iters, int H, Layout lay) {
  constexpr int TPR = pre_tpr<D>();  // threads per row, 8 elements (16 B) each
  constexpr int RPB = 256 / TPR;      // rows per pass of the workgroup
  const int bh = blockIdx.x;
  const int b = bh / H, hd = bh - b * H;
  o += b * lay.o.b + hd * lay.o.h;
  dO += b * lay.dO.b + hd * lay.dO.h;
  q += b * lay.q.b + hd * lay.q.h;
  k += b * lay.k.b + hd * lay.k.h;
  v += b * lay.v.b + hd * lay.v.h;
  const int c = (int)(threadIdx.x % TPR) * 8;
  const bool col_ok = c < D;
  uint32_t mx[4] = {0u, 0u, 0u, 0u};
  const int r_begin = blockIdx.y * RPB * iters;
#pragma unroll 4
  for (int it = 0; it < iters; ++it) {
    const int r = r_begin + it * RPB + (int)(threadIdx.x / TPR);  // row inside this (b, h)
    const bool ok = r < N;
    const int64_t row = (int64_t)bh * N + r;
    float s = 0.f;
    if (ok && col_ok) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(o + r * lay.o.n + c);
      const u32x4 g = *reinterpret_cast<const u32x4*>(dO + r * lay.dO.n + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s = fmaf(to_f32<T>(a[j] & 0xffffu), to_f32<T>(g[j] & 0xffffu), s);
        s = fmaf(to_f32<T>(a[j] >> 16), to_f32<T>(g[j] >> 16), s);
      }
      if (STATS) {
        // the raw path scales neither Q nor K: their maxima stay 0
        const uint32_t m0 =
            RAW ? 0u : absmax8<T>(*reinterpret_cast<const u32x4*>(q + r * lay.q.n + c));
        const uint32_t m1 =
            RAW ? 0u : absmax8<T>(*reinterpret_cast<const u32x4*>(k + r * lay.k.n + c));
        const uint32_t m2 = absmax8<T>(*reinterpret_cast<const u32x4*>(v + r * lay.v.n + c));
        const uint32_t m3 = absmax8<T>(g);
        mx[0] = mx[0] > m0 ? mx[0] : m0;
        mx[1] = mx[1] > m1 ? mx[1] : m1;
        mx[2] = mx[2] > m2 ? mx[2] : m2;
        mx[3] = mx[3] > m3 ? mx[3] : m3;
      }
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (ok && c == 0) {
      Dbuf[row] = s;
      const float l = lse[row];
      shift[row] = l == neg_inf() ? pos_inf() : l * kLog2e;
    }
  }
  if (STATS) {
    __shared__ uint32_t red[4][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t o2 = (uint32_t)__shfl_xor((int)mx[t], off);
        mx[t] = mx[t] > o2 ? mx[t] : o2;
      }
    if (lane == 0)
#pragma unroll
      for (int t = 0; t < 4; ++t) red[t][wave] = mx[t];
    __syncthreads();
    if (threadIdx.x < 4) {
      uint32_t m = red[threadIdx.x][0];
#pragma unroll
      for (int w = 1; w < 4; ++w) m = m > red[threadIdx.x][w] ? m : red[threadIdx.x][w];
      part[((size_t)threadIdx.x * BH + bh) * kPreChunks + blockIdx.y] = m;
    }
  }
}

// c Q * 2^-eq, K * 2^-ek and dO * 2^-eo as fp16; -(shift + rexp) * 2^-f and
// -D * 2^-(eo+ev) per row (the initial values of the dK/dV kernel's score and
// dP accumulators; rexp = 0 without dropout).  Workgroup (b, h) =
// blockIdx.x / rbph, `iters` blocks of
// RPB rows from row (blockIdx.x % rbph) * iters * RPB.  Every wave reduces
// the head's nchunk partial maxima from the D pass itself (iters > 1 on
// large grids spreads that over more rows); the head's first workgroup
// also stores them in maxes[4][BH] for the dK/dV and dQ kernels.
template <typename T, int D, bool RAW>
__global__ __launch_bounds__(256) void bwd_convert_kernel(const uint16_t* q, const uint16_t* k,
                                                          const uint16_t* dO, const float* Dbuf,
                                                          const float* shift,
                                                          const uint32_t* part, int nchunk,
                                                          uint32_t* maxes, float c,
                                                          uint16_t* q16, uint16_t* k16,
                                                          uint16_t* do16, float* nDs, float* nsh,
                                                          int N, int BH, int rbph, int iters,
                                                          int rexp, int H, Layout lay) {
  constexpr int TPR = D / 8;       // threads per row, 16 bytes each
  constexpr int RPB = 256 / TPR;   // rows per workgroup (d = 96: 21, 4 threads idle)
  const int bh = (int)(blockIdx.x / (unsigned)rbph), rb = (int)(blockIdx.x % (unsigned)rbph);
  {
    const int b = bh / H, hd = bh - b * H;
    q += b * lay.q.b + hd * lay.q.h;
    k += b * lay.k.b + hd * lay.k.h;
    dO += b * lay.dO.b + hd * lay.dO.h;
  }
  const int lane = threadIdx.x & 63;
  uint32_t mx[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t* pt = part + ((size_t)t * BH + bh) * kPreChunks;
    uint32_t m = 0u;
    for (int j = lane; j < nchunk; j += 64) m = m > pt[j] ? m : pt[j];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t o2 = (uint32_t)__shfl_xor((int)m, off);
      m = m > o2 ? m : o2;
    }
    mx[t] = m;
  }
  if (rb == 0 && threadIdx.x == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) maxes[(size_t)t * BH + bh] = mx[t];
  }
  const Scales sc = RAW ? raw_scales_of(mx[2], mx[3], c)
                        : bwd_scales_of<D>(mx[0], mx[1], mx[2], mx[3], c);
  if ((int)threadIdx.x >= RPB * TPR) return;
  const int col = (int)(threadIdx.x % TPR) * 8;
  const float cq = ldexpf(sc.exact ? 1.f : c, -sc.eq);
  for (int it = 0; it < iters; ++it) {
    const int r = (rb * iters + it) * RPB + (int)(threadIdx.x / TPR);
    if (r >= N) return;
    const int64_t row = (int64_t)bh * N + r;
    const u32x4 g = *reinterpret_cast<const u32x4*>(dO + r * lay.dO.n + col);
    u32x4 rg;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      rg[j] = Elt<_Float16>::pack2(ldexpf(to_f32<T>(g[j] & 0xffffu), -sc.eo),
                                   ldexpf(to_f32<T>(g[j] >> 16), -sc.eo));
    *reinterpret_cast<u32x4*>(do16 + row * D + col) = rg;
    if constexpr (!RAW) {  // the raw path reads Q and K themselves
      const u32x4 a = *reinterpret_cast<const u32x4*>(q + r * lay.q.n + col);
      const u32x4 kk = *reinterpret_cast<const u32x4*>(k + r * lay.k.n + col);
      u32x4 ra, rk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ra[j] = Elt<_Float16>::pack2(cq * to_f32<T>(a[j] & 0xffffu),
                                     cq * to_f32<T>(a[j] >> 16));
        rk[j] = Elt<_Float16>::pack2(ldexpf(to_f32<T>(kk[j] & 0xffffu), -sc.ek),
                                     ldexpf(to_f32<T>(kk[j] >> 16), -sc.ek));
      }
      *reinterpret_cast<u32x4*>(q16 + row * D + col) = ra;
      *reinterpret_cast<u32x4*>(k16 + row * D + col) = rk;
    }
    if (col == 0) {
      nDs[row] = -ldexpf(Dbuf[row], -(sc.eo + sc.ev));
      // with dropout the exponent also carries -rexp: P 2^-rexp (see Dropout)
      const float sh = shift[row] + (float)rexp;
      nsh[row] = sc.exact ? -sh / sc.m : -ldexpf(sh, -sc.f);
    }
  }
}

// The D pass of one (b, h) in one workgroup of 1024 threads, for grids of
// many short heads: the maxima need no second launch (the workgroup
// reduces them itself), and the second read of Q, K and dO, for the fp16
// copies, finds them in L2 or the MALL.  Writes exactly what
// bwd_pre_kernel and bwd_convert_kernel write (the same per-row thread
// mapping and sum order for D; maxima are order-free), except the partial
// maxima, which nothing reads on this path.  Rows are staged in LDS only
// as D and shift (2 N floats, N <= kHeadPrepMaxN).
constexpr int kHeadPrepMaxN = 2048;
template <typename T, int D, bool RAW>
__global__ __launch_bounds__(1024) void bwd_prep_head_kernel(
    const uint16_t* o, const uint16_t* dO, const float* lse, const uint16_t* q,
    const uint16_t* k, const uint16_t* v, float* Dbuf, float* shift, uint32_t* maxes, float c,
    uint16_t* q16, uint16_t* k16, uint16_t* do16, float* nDs, float* nsh, int N, int BH,
    int rexp, int H, Layout lay) {
  constexpr int TPR = pre_tpr<D>();  // threads per row for D, as bwd_pre_kernel
  constexpr int RPB = 1024 / TPR;
  __shared__ float sD[kHeadPrepMaxN], sS[kHeadPrepMaxN];
  __shared__ uint32_t red[4][16];
  const int bh = blockIdx.x;
  const int b = bh / H, hd = bh - b * H;
  o += b * lay.o.b + hd * lay.o.h;
  dO += b * lay.dO.b + hd * lay.dO.h;
  q += b * lay.q.b + hd * lay.q.h;
  k += b * lay.k.b + hd * lay.k.h;
  v += b * lay.v.b + hd * lay.v.h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  {
    const int c8 = (tid % TPR) * 8;
    const bool col_ok = c8 < D;
    uint32_t mx[4] = {0u, 0u, 0u, 0u};
    for (int r0 = 0; r0 < N; r0 += RPB) {
      const int r = r0 + tid / TPR;
      const bool ok = r < N;
      float s = 0.f;
      if (ok && col_ok) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(o + r * lay.o.n + c8);
        const u32x4 g = *reinterpret_cast<const u32x4*>(dO + r * lay.dO.n + c8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s = fmaf(to_f32<T>(a[j] & 0xffffu), to_f32<T>(g[j] & 0xffffu), s);
          s = fmaf(to_f32<T>(a[j] >> 16), to_f32<T>(g[j] >> 16), s);
        }
        const uint32_t m0 =
            RAW ? 0u : absmax8<T>(*reinterpret_cast<const u32x4*>(q + r * lay.q.n + c8));
        const uint32_t m1 =
            RAW ? 0u : absmax8<T>(*reinterpret_cast<const u32x4*>(k + r * lay.k.n + c8));
        const uint32_t m2 = absmax8<T>(*reinterpret_cast<const u32x4*>(v + r * lay.v.n + c8));
        const uint32_t m3 = absmax8<T>(g);
        mx[0] = mx[0] > m0 ? mx[0] : m0;
        mx[1] = mx[1] > m1 ? mx[1] : m1;
        mx[2] = mx[2] > m2 ? mx[2] : m2;
        mx[3] = mx[3] > m3 ? mx[3] : m3;
      }
#pragma unroll
      for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
      if (ok && c8 == 0) {
        const int64_t row = (int64_t)bh * N + r;
        const float l = lse[row];
        const float sh = l == neg_inf() ? pos_inf() : l * kLog2e;
        Dbuf[row] = s;
        shift[row] = sh;
        sD[r] = s;
        sS[r] = sh;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t o2 = (uint32_t)__shfl_xor((int)mx[t], off);
        mx[t] = mx[t] > o2 ? mx[t] : o2;
      }
    if (lane == 0)
#pragma unroll
      for (int t = 0; t < 4; ++t) red[t][wave] = mx[t];
  }
  __syncthreads();
  uint32_t mx[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint32_t m = red[t][0];
#pragma unroll
    for (int w = 1; w < 16; ++w) m = m > red[t][w] ? m : red[t][w];
    mx[t] = m;
  }
  if (tid == 0)
#pragma unroll
    for (int t = 0; t < 4; ++t) maxes[(size_t)t * BH + bh] = mx[t];
  const Scales sc = RAW ? raw_scales_of(mx[2], mx[3], c)
                        : bwd_scales_of<D>(mx[0], mx[1], mx[2], mx[3], c);
  // the fp16 copies and row terms, as bwd_convert_kernel
  constexpr int CT = D / 8;      // threads per row, 16 bytes each
  constexpr int CR = 1024 / CT;  // rows per pass (d = 96: 85, 4 threads idle)
  if (tid >= CR * CT) return;
  const int col = (tid % CT) * 8;
  const float cq = ldexpf(sc.exact ? 1.f : c, -sc.eq);
  for (int r = tid / CT; r < N; r += CR) {
    const int64_t row = (int64_t)bh * N + r;
    const u32x4 g = *reinterpret_cast<const u32x4*>(dO + r * lay.dO.n + col);
    u32x4 rg;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      rg[j] = Elt<_Float16>::pack2(ldexpf(to_f32<T>(g[j] & 0xffffu), -sc.eo),
                                   ldexpf(to_f32<T>(g[j] >> 16), -sc.eo));
    *reinterpret_cast<u32x4*>(do16 + row * D + col) = rg;
    if constexpr (!RAW) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(q + r * lay.q.n + col);
      const u32x4 kk = *reinterpret_cast<const u32x4*>(k + r * lay.k.n + col);
      u32x4 ra, rk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ra[j] = Elt<_Float16>::pack2(cq * to_f32<T>(a[j] & 0xffffu),
                                     cq * to_f32<T>(a[j] >> 16));
        rk[j] = Elt<_Float16>::pack2(ldexpf(to_f32<T>(kk[j] & 0xffffu), -sc.ek),
                                     ldexpf(to_f32<T>(kk[j] >> 16), -sc.ek));
      }
      *reinterpret_cast<u32x4*>(q16 + row * D + col) = ra;
      *reinterpret_cast<u32x4*>(k16 + row * D + col) = rk;
    }
    if (col == 0) {
      nDs[row] = -ldexpf(sD[r], -(sc.eo + sc.ev));
      const float sh = sS[r] + (float)rexp;
      nsh[row] = sc.exact ? -sh / sc.m : -ldexpf(sh, -sc.f);
    }
  }
}

template <bool R, typename A, typename B> struct Pick { typedef B type; };
template <typename A, typename B> struct Pick<true, A, B> { typedef A type; };

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dO;
  const float* shift;  // lse * log2(e), +inf for rows without keys
  const float* Dbuf;
  // dK/dV kernel: fp16 copies, negated scaled D and shift, the maxima
  const uint16_t* q16;
  const uint16_t* do16;
  const uint16_t* k16;
  const float* nDs;
  const float* nsh;
  const uint32_t* maxes;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int H, N, BH, ntiles;
  int period;  // snake period of map_workgroup (0: plain order)
  Dropout drop;  // used by the DROP kernels only
  float c;      // scale * log2(e)
  float scale;
  const int32_t* key_len;
  const uint8_t* block_mask;
  int nblk;
  // element strides of the caller's k, v, dO, dq, dk, dv and q (q and o are
  // read only by the D pass, except by the raw path; the workspace copies
  // are packed [BH][N][d])
  Strides sk, sv, sdO, sdq, sdk, sdv;
  Strides sq;  // the raw path reads Q in the gradient kernels too
};

// B operand (P or dS, 16 keys or queries of chunk a) from a 32x32
// accumulator: chunk a covers accumulator elements 8(a%2) .. 8(a%2)+7 of
// block a/2, i.e. rows 16a + 4h + 0..3 and 16a + 8 + 4h + 0..3.
template <typename T>
__device__ __forceinline__ typename Elt<T>::vec8 pack_chunk(const f32x16& x, int half) {
  u32x4 r;
  r.x = Elt<T>::pack2(x[8 * half + 0], x[8 * half + 1]);
  r.y = Elt<T>::pack2(x[8 * half + 2], x[8 * half + 3]);
  r.z = Elt<T>::pack2(x[8 * half + 4], x[8 * half + 5]);
  r.w = Elt<T>::pack2(x[8 * half + 6], x[8 * half + 7]);
  return as_vec8<T>(r);
}

// Copy of 64 consecutive fp32 values (one per lane) into LDS, by wave 0.
__device__ __forceinline__ void copy_row_stat(const float* g, int row0, int nrows, float* lds,
                                              int lane) {
  int row = row0 + lane;
  row = row < nrows ? row : nrows - 1;
  __builtin_amdgcn_global_load_lds(g + row, lds, 4, 0, 0);
}

// Active 128-blocks of one mask row (stride 1) or column (stride nblk),
// window [w0, wend), gathered into lst by wave 0; every wave gets the count.
__device__ __forceinline__ int list_blocks(const uint8_t* m, int stride, int w0, int wend,
                                           int* lst, int wave, int lane) {
  int cnt = 0;
  for (int j0 = w0; j0 < wend; j0 += 64) {
    const int j = j0 + lane;
    const bool on = j < wend && m[(size_t)j * stride] != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
    if (wave == 0 && on) lst[cnt + __builtin_popcountll(bal & ((1ull << lane) - 1))] = j;
    cnt += __builtin_popcountll(bal);
  }
  return cnt;
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 128 keys, 32 per wave
// ---------------------------------------------------------------------------
// T is the input/output type; the products run on the scaled fp16 operands
// described at the top of this file.
// DROP: dropout on P (dV uses P M / (1 - p), dS = P (dP M / (1 - p) - D))
// LDS of one dK/dV workgroup: double-buffered Q and dO tiles and their row
// terms, and the block-sparse list
template <int D, bool SPARSE>
struct DkdvLds {
  __attribute__((aligned(16))) uint16_t q0[kBQ * D], q1[kBQ * D], o0[kBQ * D], o1[kBQ * D];
  __attribute__((aligned(16))) float l0[kBQ], l1[kBQ], d0[kBQ], d1[kBQ];
  int list[SPARSE ? kListMax : 1];
};

// workgroup `wg` of the dK/dV grid
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP, bool RAW>
__device__ __forceinline__ void bwd_dkdv_body(BwdParams p, int wg, DkdvLds<D, SPARSE>& lds) {
  constexpr int KS = D / 16, DB = D / 32, TILE = kBQ * D, NW = 4;
  // operand types: TQ for Q, K and dS (S = Q K^T, dK = dS^T Q), fp16 for dO,
  // V and P (dP = dO V^T, dV = P^T dO)
  typedef typename Pick<RAW, T, _Float16>::type TQ;
  typedef _Float16 TI;
  typedef typename Elt<TQ>::vec8 qvec8;
  typedef typename Elt<TI>::vec8 vec8;
  uint16_t* const sQ0 = lds.q0;
  uint16_t* const sQ1 = lds.q1;
  uint16_t* const sO0 = lds.o0;
  uint16_t* const sO1 = lds.o1;
  float* const sL0 = lds.l0;
  float* const sL1 = lds.l1;
  float* const sD0 = lds.d0;
  float* const sD1 = lds.d1;
  int* const sList = lds.list;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5, sub = lane & 15, g4 = lane >> 4;
  int rank, bh;
  map_workgroup(wg, p.ntiles, p.BH, p.period, &rank, &bh);
  const int kt = rank;  // causal: the lowest key tiles see the most queries, so go first
  const int b = bh / p.H, hd = bh - b * p.H, N = p.N;
  const size_t base = (size_t)bh * N * D;  // the packed workspace copies
  // Q (raw) or c Q 2^-eq (fp16 copy); dO 2^-eo (fp16 copy)
  const uint16_t* Q = RAW ? p.q + b * p.sq.b + hd * p.sq.h : p.q16 + base;
  const uint16_t* dO = p.do16 + base;
  const int64_t qrs = RAW ? p.sq.n : D;  // Q's row stride (the copies are packed)
  const float* nsh = p.nsh + (size_t)bh * N;
  const float* nD = p.nDs + (size_t)bh * N;
  const int L = valid_keys(p.key_len, b, N);
  const int k0 = kt * kBKV, kw = k0 + wave * 32, key = kw + l32;
  // The prologue issues every load (the head's maxima, the first query
  // tile's copies, this wave's keys and values) before it uses any, so that
  // their global latencies overlap instead of adding up.
  const uint32_t mxq = RAW ? 0u : p.maxes[bh], mxk = RAW ? 0u : p.maxes[p.BH + bh];
  const uint32_t mxv = p.maxes[2 * p.BH + bh], mxo = p.maxes[3 * p.BH + bh];

  const TileCopy<D, kBQ, NW> copy(wave, lane, qrs);  // Q; dO's tiles adjust to its stride
  // copies of the query tile at row r0 (Q, dO and the two row terms)
  auto load = [&](int r0, uint16_t* dq_, uint16_t* do_, float* dl, float* dd)
      __attribute__((always_inline)) {
    copy(Q, r0, N, dq_);
    copy.copy_rs(dO, D, r0, N, do_);
    if (wave == 0) copy_row_stat(nsh, r0, N, dl, lane);
    if (wave == 1) copy_row_stat(nD, r0, N, dd, lane);
  };
  // Dense masks: the query tiles t0 .. nqt-1 (causal: the queries before k0
  // see none of these keys); the first one's copies go out here.
  const int nqt = (N + kBQ - 1) / kBQ;
  const int t0 = CAUSAL ? k0 / kBQ : 0;
  const bool primed = !SPARSE && k0 < L && nqt > t0;
  if (primed) load(t0 * kBQ, sQ0, sO0, sL0, sD0);

  // this wave's keys (K, or K 2^-ek in fp16) and values (V 2^-ev, fp16) as
  // B operands (lane = key, k = d values)
  u32x4 kraw[KS], vraw[KS];
  const uint16_t* const Kin = p.k + b * p.sk.b + hd * p.sk.h;
  const uint16_t* const Vin = p.v + b * p.sv.b + hd * p.sv.h;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kraw[ks] = ldg16_row(Kin, key, p.sk.n, ks * 16 + h * 8, N);
    vraw[ks] = ldg16_row(Vin, key, p.sv.n, ks * 16 + h * 8, N);
  }
  const Scales sc =
      RAW ? raw_scales_of(mxv, mxo, p.c) : bwd_scales_of<D>(mxq, mxk, mxv, mxo, p.c);
  const int ek = sc.ek, ev = sc.ev;
  qvec8 kf[KS];
  vec8 vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 kr = kraw[ks], vr = vraw[ks];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (!RAW)
        kr[j] = Elt<TI>::pack2(ldexpf(to_f32<T>(kr[j] & 0xffffu), -ek),
                               ldexpf(to_f32<T>(kr[j] >> 16), -ek));
      vr[j] = Elt<TI>::pack2(ldexpf(to_f32<T>(vr[j] & 0xffffu), -ev),
                             ldexpf(to_f32<T>(vr[j] >> 16), -ev));
    }
    kf[ks] = as_vec8<TQ>(kr);
    vf[ks] = as_vec8<TI>(vr);
  }
  f32x16 dk[DB], dv[DB];  // dK^T, dV^T: rows d = 32db + 8i + 4h + j, column = key
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[db][e] = dv[db][e] = 0.f;

  int roff[KS];  // Q / dO rows as A operands: row l32, d chunk 2 ks + h
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = tile_off<D>(l32, ks * 16 + h * 8);
  int toff[2][DB];  // dO^T / Q^T transpose reads (rows = queries 16a + 4h + sub/4 [+8])
#pragma unroll
  for (int sec = 0; sec < 2; ++sec)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      toff[sec][db] = tile_off<D>(4 * h + (sub >> 2) + 8 * sec, db * 32 + 16 * (g4 & 1) + 4 * (sub & 3));

  const bool any_key = kw < L;  // every key of this wave padded away -> zero gradients

  auto compute = [&](const uint16_t* tq, const uint16_t* to, const float* tl, const float* td,
                     int q0) __attribute__((always_inline)) {
    if (!any_key) return;
    if (CAUSAL && q0 + kBQ - 1 < kw) return;  // every query of the tile precedes the keys
    // rows = queries 32 qb + 8i + 4h + j, column = key.  The score
    // accumulator starts at -shift 2^-f and the dP accumulator at
    // -D 2^-(eo+ev) (the row's values, read in accumulator order), so they
    // end as 2^-f (c s - shift) and 2^-(eo+ev) (dP - D).
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(tl + qb * 32 + 8 * i + 4 * h);
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(td + qb * 32 + 8 * i + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[qb][4 * i + j] = a4[j];
          dp[qb][4 * i + j] = DROP ? 0.f : b4[j];  // with dropout -D enters after the mask
        }
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const qvec8 aq = as_vec8<TQ>(lds16(tq + roff[ks] + qb * 32 * D));
        const vec8 ao = as_vec8<TI>(lds16(to + roff[ks] + qb * 32 * D));
        s[qb] = Elt<TQ>::mfma32(aq, kf[ks], s[qb]);
        dp[qb] = Elt<TI>::mfma32(ao, vf[ks], dp[qb]);
      }
    // P = exp2(c s - shift_row), dS' = P (dP - D_row) 2^-(eo+ev)
    const bool need_mask = (kw + 32 > L) || (q0 + kBQ > N) || (CAUSAL && q0 < kw + 31);
    if (sc.mul) {  // exact head or unbalanced operand scales (large or extreme ranges)
      const float sf = sc.m;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[qb] *= sf;
    }
    // The visibility test is hoisted out of the element loop and done with
    // selects: query q0 + 32qb + 4h + o, o = 8(e/4) + e%4, sees this lane's
    // key iff lo <= o < hi.
    if constexpr (DROP) {
      // Element e is query q0 + 32qb + 8(e/4) + 4h + e%4 of this lane's key.
      // One generator call covers 8 keys at one query: the keys of this
      // lane's call group are held by the 8 lanes that differ from it in
      // lane bits 0, 1, 3, and this lane's key is draw t8 of the call.  For
      // the 8 queries of a pair of element rows (e/4 = 2c, 2c+1), the lane at
      // position t8 draws the call of query t8 and turns its 8 draws into
      // a byte of keep bits (bit t: the key of draw t); the 8 lanes gather
      // the bytes into 64 bits (byte u: query u), and each lane reads bit
      // t8 of every byte.  One call per 8 elements.
      const int t8 = (lane & 3) | ((lane >> 1) & 4);
      const uint32_t gk = (uint32_t)drop_call(key), th = p.drop.thresh;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qbase = q0 + qb * 32 + 4 * h;
        const int hi = key < L ? N - qbase : -64;
        const int lo = CAUSAL ? key - qbase : -64;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          uint32_t w[4];
          philox4x32_10(gk, (uint32_t)(qbase + 8 * (2 * c2 + (t8 >> 2)) + (t8 & 3)),
                        (uint32_t)bh, p.drop.offset, p.drop.k0, p.drop.k1, w);
          uint32_t byte = 0u;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            byte |= (((w[u] & 0xFFFFu) >= th ? 1u : 0u) | (w[u] >= (th << 16) ? 2u : 0u))
                    << (2 * u);
          const uint32_t xlo = or8_bits013(t8 < 4 ? byte << (8 * t8) : 0u) >> t8;
          const uint32_t xhi = or8_bits013(t8 >= 4 ? byte << (8 * (t8 - 4)) : 0u) >> t8;
#pragma unroll
          for (int il = 0; il < 2; ++il) {
            const int i = 2 * c2 + il;
            const f32x4 nd4 = *reinterpret_cast<const f32x4*>(td + qb * 32 + 8 * i + 4 * h);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int o = 8 * i + j, e = 4 * i + j;
              const float pv = ((o >= lo) & (o < hi)) ? fast_exp2(s[qb][e]) : 0.f;
              const float mk = ((il ? xhi : xlo) >> (8 * j)) & 1u ? p.drop.rinv : 0.f;
              dp[qb][e] = pv * fmaf(mk, dp[qb][e], nd4[j]);
              s[qb][e] = pv * mk;
            }
          }
        }
      }
    } else if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qbase = q0 + qb * 32 + 4 * h;
        const int hi = key < L ? N - qbase : -64;     // past N, or the key is padded
        const int lo = CAUSAL ? key - qbase : -64;    // queries before the key
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int o = 8 * (e >> 2) + (e & 3);
          const float pv = ((o >= lo) & (o < hi)) ? fast_exp2(s[qb][e]) : 0.f;
          s[qb][e] = pv;
          dp[qb][e] *= pv;
        }
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pv = fast_exp2(s[qb][e]);
          s[qb][e] = pv;
          dp[qb][e] *= pv;
        }
    }
    // dV^T += dO^T P, dK^T += Q^T dS, 16 queries (chunk a) per MFMA
#pragma unroll
    for (int a = 0; a < kBQ / 16; ++a) {
      const vec8 pb = pack_chunk<TI>(s[a >> 1], a & 1);
      const qvec8 sb = pack_chunk<TQ>(dp[a >> 1], a & 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const vec8 ao = join8<TI>(lds_tr4(to + toff[0][db] + a * 16 * D),
                                  lds_tr4(to + toff[1][db] + a * 16 * D));
        const qvec8 aq = join8<TQ>(lds_tr4(tq + toff[0][db] + a * 16 * D),
                                   lds_tr4(tq + toff[1][db] + a * 16 * D));
        dv[db] = Elt<TI>::mfma32(ao, pb, dv[db]);
        dk[db] = Elt<TQ>::mfma32(aq, sb, dk[db]);
      }
    }
  };

  // query tiles t -> first row row0(t); copies one tile ahead, one barrier
  // per tile (`primed`: the first tile's copies are already in flight)
  auto walk = [&](int ntiles, auto row0, bool primed_) __attribute__((always_inline)) {
    if (ntiles <= 0) return;
    if (!primed_) load(row0(0), sQ0, sO0, sL0, sD0);
    auto step = [&](int t, const uint16_t* cq, const uint16_t* co, const float* cl,
                    const float* cd, uint16_t* nq, uint16_t* no, float* nl, float* nd)
        __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of tile t landed
      __syncthreads();                     // ... and every wave's; tile t-1 fully read
      if (t + 1 < ntiles) load(row0(t + 1), nq, no, nl, nd);
      compute(cq, co, cl, cd, row0(t));
    };
    for (int t = 0; t < ntiles; t += 2) {
      step(t, sQ0, sO0, sL0, sD0, sQ1, sO1, sL1, sD1);
      if (t + 1 < ntiles) step(t + 1, sQ1, sO1, sL1, sD1, sQ0, sO0, sL0, sD0);
    }
    __syncthreads();
  };

  if (k0 < L) {
    if (SPARSE) {
      const uint8_t* mcol = p.block_mask + kt;  // column kt, stride nblk
      for (int w0 = 0; w0 < p.nblk; w0 += kListMax) {
        const int wend = w0 + kListMax < p.nblk ? w0 + kListMax : p.nblk;
        const int cnt = list_blocks(mcol, p.nblk, w0, wend, sList, wave, lane);
        __syncthreads();
        walk(2 * cnt, [&](int t) { return sList[t >> 1] * 128 + (t & 1) * kBQ; }, false);
      }
    } else {
      walk(nqt - t0, [&](int t) { return (t0 + t) * kBQ; }, primed);
    }
  }

  // store dK = scale/c 2^(eq+eo+ev) dK'^T^T (scale/c = ln 2; an exact head's
  // Q copy carries no c: scale) and dV = 2^eo dV' (4 consecutive d per store);
  // with dropout both also undo the 2^-rexp that P carried
  if (key < N) {
    const int rx = DROP ? p.drop.rexp : 0;
    const int ekk = sc.eq + sc.eo + sc.ev + rx;
    const float kmul = sc.exact ? p.scale : kLn2;
    uint16_t* const dKo = p.dk + b * p.sdk.b + hd * p.sdk.h + (int64_t)key * p.sdk.n;
    uint16_t* const dVo = p.dv + b * p.sdv.b + hd * p.sdv.h + (int64_t)key * p.sdv.n;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int off = db * 32 + 8 * i + 4 * h;
        f32x4 k4, v4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          k4[j] = ldexpf(dk[db][4 * i + j] * kmul, ekk);
          v4[j] = ldexpf(dv[db][4 * i + j], sc.eo + rx);
        }
        *reinterpret_cast<u32x2*>(dKo + off) = pack4<T>(k4);
        *reinterpret_cast<u32x2*>(dVo + off) = pack4<T>(v4);
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 128 queries, 32 per wave
//
// Scores run on fp16 operands (c Q 2^-eq against K 2^-ek, the fp16 copies
// of the convert pass; for fp16 inputs Q and K themselves) and dP on the
// input type.  The first k-step of each
// product starts from the query's -shift 2^-f (scores) or -D (dP) as its C
// operand, so the accumulators end as the exponent of P and as dP - D: P is
// one exponential and dS one multiply.
// ---------------------------------------------------------------------------
// DROP: dS = P (dP M / (1 - p) - D); dP starts from 0 and D enters after
// the mask
// LDS of one dQ workgroup: double-buffered K and V tiles and the
// block-sparse list
template <int D, bool SPARSE>
struct DqLds {
  __attribute__((aligned(16))) uint16_t k0[kBC * D], k1[kBC * D], v0[kBC * D], v1[kBC * D];
  int list[SPARSE ? kListMax : 1];
};

// workgroup `wg` of the dQ grid
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP, bool RAW>
__device__ __forceinline__ void bwd_dq_body(BwdParams p, int wg, DqLds<D, SPARSE>& lds) {
  constexpr int KS = D / 16, DB = D / 32, TILE = kBC * D, NW = 4;
  typedef typename Pick<RAW, T, _Float16>::type TI;  // the score and dQ operand type
  typedef typename Elt<TI>::vec8 hvec8;
  typedef typename Elt<T>::vec8 vec8;
  uint16_t* const sK0 = lds.k0;
  uint16_t* const sK1 = lds.k1;
  uint16_t* const sV0 = lds.v0;
  uint16_t* const sV1 = lds.v1;
  int* const sList = lds.list;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5, sub = lane & 15, g4 = lane >> 4;
  int rank, bh;
  map_workgroup(wg, p.ntiles, p.BH, p.period, &rank, &bh);
  const int qt = CAUSAL ? p.ntiles - 1 - rank : rank;  // longest rows first
  const int b = bh / p.H, hd = bh - b * p.H, N = p.N;
  const size_t base = (size_t)bh * N * D;  // the packed workspace copies
  // K 2^-ek (fp16 copy) or K itself (raw)
  const uint16_t* K = RAW ? p.k + b * p.sk.b + hd * p.sk.h : p.k16 + base;
  const int64_t krs = RAW ? p.sk.n : D;  // its row stride
  const uint16_t* V = p.v + b * p.sv.b + hd * p.sv.h;
  const int L = valid_keys(p.key_len, b, N);
  const int q0 = qt * kBR, qw = q0 + wave * 32, query = qw + l32;
  // The prologue issues every load (the head's maxima, the first key tile's
  // copies, this wave's queries, output gradients and row terms) before it
  // uses any, so that their global latencies overlap instead of adding up.
  const uint32_t mxq = RAW ? 0u : p.maxes[bh], mxk = RAW ? 0u : p.maxes[p.BH + bh];
  const uint32_t mxv = p.maxes[2 * p.BH + bh], mxo = p.maxes[3 * p.BH + bh];

  // chunk offsets for K's tiles; V's tiles adjust them when its row stride
  // differs
  const TileCopy<D, kBC, NW> copy(wave, lane, krs);
  // Dense masks: key tiles 0 .. nkt-1 (causal: up to the last query's
  // diagonal); the first one's copies go out here.
  int nkt = (L + kBC - 1) / kBC;
  if (CAUSAL) {
    const int last = (q0 + kBR < N ? q0 + kBR : N) - 1;
    nkt = nkt < last / kBC + 1 ? nkt : last / kBC + 1;
  }
  const bool primed = !SPARSE && nkt > 0;
  if (primed) {
    copy(K, 0, N, sK0);
    copy.copy_rs(V, p.sv.n, 0, N, sV0);
  }
  // this wave's queries (c Q 2^-eq, fp16) and output gradients as B
  // operands (lane = query, k = d values)
  hvec8 qf[KS];
  vec8 of[KS];
  const bool qok = query < N;
  const uint16_t* const dOin = p.dO + b * p.sdO.b + hd * p.sdO.h;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = as_vec8<TI>(RAW ? ldg16_row(p.q + b * p.sq.b + hd * p.sq.h, query, p.sq.n,
                                         ks * 16 + h * 8, N)
                             : ldg16_row(p.q16 + base, query, D, ks * 16 + h * 8, N));
    of[ks] = as_vec8<T>(ldg16_row(dOin, query, p.sdO.n, ks * 16 + h * 8, N));
  }
  // the row values of this lane's query: -shift 2^-f and D
  const float nsh_q = ldg_f32(p.nsh + (size_t)bh * N, query, N, neg_inf());
  const float D_q = ldg_f32(p.Dbuf + (size_t)bh * N, query, N, 0.f);
  const float dq_D = DROP ? D_q : 0.f;  // dropout: D is subtracted after the mask
  const Scales sc =
      RAW ? raw_scales_of(mxv, mxo, p.c) : bwd_scales_of<D>(mxq, mxk, mxv, mxo, p.c);
  // dS is rounded to fp16 (raw path: the input type) for dQ = dS K.  dP and D here are unscaled (raw
  // dO against raw V), so P carries the power of two 2^kq, kq = -(eo + ev),
  // that the dK/dV kernel's dS gets from its scaled dO and V copies: then
  // |dS'| = |P 2^kq (dP - D)| <= 2 d max|dO'| max|V'| < 2^15 for d <= 128,
  // whatever the magnitudes of dO and V, and entries of ordinary size stay
  // clear of fp16's subnormal range.  kq enters the exponent through the
  // row term (no instruction per score) and is undone exactly in the
  // epilogue.  With dropout P also carries 2^-rexp, from the row term the
  // convert pass wrote.
  const int kq = -(sc.eo + sc.ev);
  // the row terms of this lane's query (-shift 2^-f for the scores, -D for
  // dP; dropout subtracts D after the mask instead), replicated: every
  // element of a lane's 32 x 32 accumulator block belongs to its query, so
  // the first k-step of each product takes them as its C operand and the
  // fp32 accumulator starts from them exactly
  f32x16 s_init, dp_init;
  {
    // the exponent is m (nsh + S'') when the accumulator is rescaled by m
    // (m = 2^f, or c 2^f in exact mode), else nsh + S''
    const float kqm = sc.mul ? (float)kq / sc.m : (float)kq;
    const float ns = nsh_q + kqm;
    const float nd = DROP ? 0.f : -D_q;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s_init[e] = ns;
      dp_init[e] = nd;
    }
  }
  f32x16 acc[DB];  // dQ^T: rows d = 32db + 8i + 4h + j, column = query
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;

  int roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = tile_off<D>(l32, ks * 16 + h * 8);
  int toff[2][DB];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      toff[sec][db] = tile_off<D>(4 * h + (sub >> 2) + 8 * sec, db * 32 + 16 * (g4 & 1) + 4 * (sub & 3));

  // `prefetch` starts the copies of the next tile; it runs inside the
  // compute, after the score products are issued, so that the copies (which
  // can stall issue while the CU's vector-memory path is busy) overlap
  // matrix-core work instead of delaying it
  auto compute = [&](const uint16_t* tk, const uint16_t* tv, int kt0, auto prefetch)
      __attribute__((always_inline)) {
    if (qw >= N || (CAUSAL && kt0 > qw + 31)) {  // no rows / tile above the diagonal
      prefetch();
      return;
    }
    f32x16 s[2], dp[2];  // rows = keys 32 kb + 8i + 4h + j, column = query
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const hvec8 ak = as_vec8<TI>(lds16(tk + roff[ks] + kb * 32 * D));
        const vec8 av = as_vec8<T>(lds16(tv + roff[ks] + kb * 32 * D));
        s[kb] = Elt<TI>::mfma32(ak, qf[ks], ks == 0 ? s_init : s[kb]);
        dp[kb] = Elt<T>::mfma32(av, of[ks], ks == 0 ? dp_init : dp[kb]);
      }
    prefetch();
    const bool need_mask = (kt0 + kBC > L) || (CAUSAL && kt0 + kBC - 1 > qw);
    if (sc.mul) {  // exact head or unbalanced operand scales (large or extreme ranges)
      const float sf = sc.m;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] *= sf;
    }
    // key kt0 + 32kb + 4h + o, o = 8(e/4) + e%4, is visible to this lane's
    // query iff o <= thr (the test hoisted out of the element loop, selects)
    if constexpr (DROP) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kbase = kt0 + kb * 32 + 4 * h;
        int thr = L - 1 - kbase;
        if (CAUSAL) thr = min(thr, query - kbase);
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // elements 8c .. 8c+7 (i = 2c, 2c+1): keys kbase + 16c + {0..3,
          // 8..11}, one generator call; element 4i + j takes the low (j
          // even) or high half of word 2 (i % 2) + j / 2
          if ((i & 1) == 0)
            philox4x32_10((uint32_t)drop_call(kbase + 8 * i), (uint32_t)query, (uint32_t)bh,
                          p.drop.offset, p.drop.k0, p.drop.k1, w);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = 4 * i + j;
            const uint32_t wd = w[2 * (i & 1) + (j >> 1)];
            const bool keep = (j & 1) ? wd >= (p.drop.thresh << 16)
                                      : (wd & 0xFFFFu) >= p.drop.thresh;
            const float pv = 8 * i + j <= thr ? fast_exp2(s[kb][e]) : 0.f;
            const float mk = keep ? p.drop.rinv : 0.f;
            dp[kb][e] = pv * fmaf(mk, dp[kb][e], -dq_D);
          }
        }
      }
    } else if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kbase = kt0 + kb * 32 + 4 * h;
        int thr = L - 1 - kbase;
        if (CAUSAL) thr = min(thr, query - kbase);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int o = 8 * (e >> 2) + (e & 3);
          dp[kb][e] *= o <= thr ? fast_exp2(s[kb][e]) : 0.f;
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) dp[kb][e] *= fast_exp2(s[kb][e]);
    }
    // dQ^T += K^T dS^T  (k = 16 keys per MFMA; K 2^-ek)
#pragma unroll
    for (int a = 0; a < kBC / 16; ++a) {
      const hvec8 sb = pack_chunk<TI>(dp[a >> 1], a & 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const hvec8 ak = join8<TI>(lds_tr4(tk + toff[0][db] + a * 16 * D),
                                   lds_tr4(tk + toff[1][db] + a * 16 * D));
        acc[db] = Elt<TI>::mfma32(ak, sb, acc[db]);
      }
    }
  };

  // `primed`: the first tile's copies are already in flight
  auto walk = [&](int ntiles, auto key0, bool primed_) __attribute__((always_inline)) {
    if (ntiles <= 0) return;
    if (!primed_) {
      copy(K, key0(0), N, sK0);
      copy.copy_rs(V, p.sv.n, key0(0), N, sV0);
    }
    auto step = [&](int t, const uint16_t* ck, const uint16_t* cv, uint16_t* nk, uint16_t* nv)
        __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      auto prefetch = [&]() __attribute__((always_inline)) {
        if (t + 1 < ntiles) {
          const int k1 = key0(t + 1);
          copy(K, k1, N, nk);
          copy.copy_rs(V, p.sv.n, k1, N, nv);
        }
      };
      compute(ck, cv, key0(t), prefetch);
    };
    for (int t = 0; t < ntiles; t += 2) {
      step(t, sK0, sV0, sK1, sV1);
      if (t + 1 < ntiles) step(t + 1, sK1, sV1, sK0, sV0);
    }
    __syncthreads();
  };

  if (SPARSE) {
    const uint8_t* mrow = p.block_mask + (size_t)qt * p.nblk;
    for (int w0 = 0; w0 < p.nblk; w0 += kListMax) {
      const int wend = w0 + kListMax < p.nblk ? w0 + kListMax : p.nblk;
      const int cnt = list_blocks(mrow, 1, w0, wend, sList, wave, lane);
      __syncthreads();
      walk(2 * cnt, [&](int t) { return sList[t >> 1] * 128 + (t & 1) * kBC; }, false);
    }
  } else {
    walk(nkt, [](int t) { return t * kBC; }, primed);
  }

  if (qok) {  // dQ = scale 2^(ek - kq + rexp) (dS' K')
    const int eqo = sc.ek - kq + (DROP ? p.drop.rexp : 0);
    uint16_t* const dQo = p.dq + b * p.sdq.b + hd * p.sdq.h + (int64_t)query * p.sdq.n;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 q4;
#pragma unroll
        for (int j = 0; j < 4; ++j) q4[j] = ldexpf(acc[db][4 * i + j] * p.scale, eqo);
        *reinterpret_cast<u32x2*>(dQo + db * 32 + 8 * i + 4 * h) = pack4<T>(q4);
      }
  }
}

// The two gradient kernels as separate launches (fa_bwd_stage) ...
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP, bool RAW>
__global__ __launch_bounds__(256, D <= 64 ? 2 : 1) void bwd_dkdv_kernel(BwdParams p) {
  __shared__ DkdvLds<D, SPARSE> lds;
  bwd_dkdv_body<T, D, CAUSAL, SPARSE, DROP, RAW>(p, (int)blockIdx.x, lds);
}

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP, bool RAW>
__global__ __launch_bounds__(256, D <= 64 ? 2 : 1) void bwd_dq_kernel(BwdParams p) {
  __shared__ DqLds<D, SPARSE> lds;
  bwd_dq_body<T, D, CAUSAL, SPARSE, DROP, RAW>(p, (int)blockIdx.x, lds);
}

// ... and as one launch (fa_bwd): the dK/dV and dQ kernels need only what
// the D pass wrote, not each other, so the first ntiles * BH workgroups
// take dK/dV and the rest dQ, and dQ workgroups start while the last,
// longest dK/dV workgroups still run (short sequences leave most compute
// units idle in each kernel's tail).  The two LDS layouts share one buffer.
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP, bool RAW>
__global__ __launch_bounds__(256, D <= 64 ? 2 : 1) void bwd_fused_kernel(BwdParams p) {
  static_assert(kBKV == kBR, "one tile count for both parts of the grid");
  __shared__ union {
    DkdvLds<D, SPARSE> kv;
    DqLds<D, SPARSE> q;
  } lds;
  const int n = p.ntiles * p.BH;
  if ((int)blockIdx.x < n)
    bwd_dkdv_body<T, D, CAUSAL, SPARSE, DROP, RAW>(p, (int)blockIdx.x, lds.kv);
  else
    bwd_dq_body<T, D, CAUSAL, SPARSE, DROP, RAW>(p, (int)blockIdx.x - n, lds.q);
}

// fp16 inputs take the raw path: Q and K enter the gradient products as
// they are (exact fp16 products, c applied to the score accumulator in
// fp32), so the D pass needs neither their maxima nor their copies (about
// half its bytes); dS stays fp16 with its power-of-two scale, as on the
// scaled path.  bf16 inputs keep the scaled fp16 copies: their raw
// products would need dS in bf16 for dK = dS^T Q, whose 8 bits cost dK
// up to 2.4e-2 against the oracle on a head with 17 unpadded keys
// (1.4e-2 with fp16 dS), past the bf16 gate.
template <typename T>
constexpr bool use_raw() {
  return !kIsBf16<T>;
}

// Every kernel the launcher below can select (the host pass of this compiler
// otherwise leaves some kernel-template launch stubs undefined).
#define FA_BWD_INSTANTIATE_DP(T, D, RAW)                                              \
  template __global__ void bwd_pre_kernel<T, D, true, RAW>(                         \
      const uint16_t*, const uint16_t*, const float*, const uint16_t*, const uint16_t*, \
      const uint16_t*, float*, float*, uint32_t*, int, int, int, int, Layout);      \
  template __global__ void bwd_prep_head_kernel<T, D, RAW>(                         \
      const uint16_t*, const uint16_t*, const float*, const uint16_t*, const uint16_t*, \
      const uint16_t*, float*, float*, uint32_t*, float, uint16_t*, uint16_t*, uint16_t*, \
      float*, float*, int, int, int, int, Layout);                                 \
  template __global__ void bwd_convert_kernel<T, D, RAW>(                           \
      const uint16_t*, const uint16_t*, const uint16_t*, const float*, const float*,   \
      const uint32_t*, int, uint32_t*, float,                                        \
      uint16_t*, uint16_t*, uint16_t*, float*, float*, int, int, int, int, int, int, Layout);
#define FA_BWD_INSTANTIATE_GR(T, D, RAW)                                              \
  template __global__ void bwd_dkdv_kernel<T, D, true, false, false, RAW>(BwdParams);   \
  template __global__ void bwd_dkdv_kernel<T, D, false, false, false, RAW>(BwdParams);  \
  template __global__ void bwd_dkdv_kernel<T, D, false, true, false, RAW>(BwdParams);   \
  template __global__ void bwd_dkdv_kernel<T, D, true, false, true, RAW>(BwdParams);    \
  template __global__ void bwd_dkdv_kernel<T, D, false, false, true, RAW>(BwdParams);   \
  template __global__ void bwd_dq_kernel<T, D, true, false, false, RAW>(BwdParams);     \
  template __global__ void bwd_dq_kernel<T, D, false, false, false, RAW>(BwdParams);    \
  template __global__ void bwd_dq_kernel<T, D, true, false, true, RAW>(BwdParams);      \
  template __global__ void bwd_dq_kernel<T, D, false, false, true, RAW>(BwdParams);     \
  template __global__ void bwd_dq_kernel<T, D, false, true, false, RAW>(BwdParams);     \
  template __global__ void bwd_fused_kernel<T, D, true, false, false, RAW>(BwdParams);  \
  template __global__ void bwd_fused_kernel<T, D, false, false, false, RAW>(BwdParams); \
  template __global__ void bwd_fused_kernel<T, D, true, false, true, RAW>(BwdParams);   \
  template __global__ void bwd_fused_kernel<T, D, false, false, true, RAW>(BwdParams);  \
  template __global__ void bwd_fused_kernel<T, D, false, true, false, RAW>(BwdParams);
#define FA_BWD_INSTANTIATE(T, D)                                                  \
  FA_BWD_INSTANTIATE_DP(T, D, use_raw<T>())                                       \
  FA_BWD_INSTANTIATE_GR(T, D, use_raw<T>())
FA_BWD_INSTANTIATE(__bf16, 32)
FA_BWD_INSTANTIATE(__bf16, 64)
FA_BWD_INSTANTIATE(__bf16, 96)
FA_BWD_INSTANTIATE(__bf16, 128)
FA_BWD_INSTANTIATE(_Float16, 32)
FA_BWD_INSTANTIATE(_Float16, 64)
FA_BWD_INSTANTIATE(_Float16, 96)
FA_BWD_INSTANTIATE(_Float16, 128)
#undef FA_BWD_INSTANTIATE
#undef FA_BWD_INSTANTIATE_DP
#undef FA_BWD_INSTANTIATE_GR

// The D pass in one launch (one workgroup per head) when there are enough
// heads to spread over the GPU and each is short; otherwise the two
// launches whose grids split every head over many workgroups.  Measured
// (stage D alone, bf16): 61 -> 56 us at B = 16, H = 16, N = 1024; 29 -> 26 us
// at 8 x 12 x 1024; 67 -> 63 us at 8 x 16 x 2048; 26 -> 25 us at 2 x 16 x 1024;
// but 60 -> 94 us at 4 x 16 x 4096 (too few workgroups for the bytes).
inline bool head_prep(int N, int BH) { return N <= kHeadPrepMaxN && BH >= 32; }

// The gradient launches of stage 0 or 4 (one grid of dK/dV and dQ
// workgroups), 2 (dK/dV) or 3 (dQ).
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP, bool RAW>
hipError_t launch_grads(BwdParams p, hipStream_t stream, int stage) {
  p.ntiles = (p.N + kBKV - 1) / kBKV;  // = (N + kBR - 1) / kBR
  if (stage == 0 || stage == 4)
    hipLaunchKernelGGL((bwd_fused_kernel<T, D, CAUSAL, SPARSE, DROP, RAW>),
                       dim3(2 * p.ntiles * p.BH), dim3(256), 0, stream, p);
  else if (stage == 2)
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, SPARSE, DROP, RAW>),
                       dim3(p.ntiles * p.BH), dim3(256), 0, stream, p);
  else if (stage == 3)
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, SPARSE, DROP, RAW>), dim3(p.ntiles * p.BH),
                       dim3(256), 0, stream, p);
  return hipGetLastError();
}


// The D pass: D, shift, maxima, the fp16 copies and the row terms, in one
// launch (one workgroup per head) or two (maxima per chunk of rows, then the
// copies); the raw path copies dO only.
template <typename T, int D, bool RAW>
hipError_t launch_dpass(const BwdArgs& a, char* ws, const BwdWorkspace& w) {
  const int BH = a.B * a.H;
  float* Dbuf = reinterpret_cast<float*>(ws + w.D);
  float* shift = reinterpret_cast<float*>(ws + w.shift);
  float* nDs = reinterpret_cast<float*>(ws + w.nDs);
  float* nsh = reinterpret_cast<float*>(ws + w.nsh);
  const float c = a.scale * kLog2e;
  uint32_t* maxes = reinterpret_cast<uint32_t*>(ws + w.maxes);
  uint32_t* part = reinterpret_cast<uint32_t*>(ws + w.part);
  uint16_t* q16 = reinterpret_cast<uint16_t*>(ws + w.q16);
  uint16_t* do16 = reinterpret_cast<uint16_t*>(ws + w.do16);
  uint16_t* k16 = reinterpret_cast<uint16_t*>(ws + w.k16);
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* dO = static_cast<const uint16_t*>(a.dO);
  const int rexp = a.drop.on ? a.drop.rexp : 0;
  if (head_prep(a.N, BH)) {
    hipLaunchKernelGGL((bwd_prep_head_kernel<T, D, RAW>), dim3(BH), dim3(1024), 0, a.stream,
                       static_cast<const uint16_t*>(a.o), dO, a.lse, q,
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), Dbuf,
                       shift, maxes, c, q16, k16, do16, nDs, nsh, a.N, BH, rexp, a.H, a.lay);
    return hipGetLastError();
  }
  // row groups per workgroup of the D pass: enough for a grid of about
  // 2048 workgroups, and at least enough that a head has at most
  // kPreChunks workgroups (one partial maximum each)
  constexpr int rpb = 256 / pre_tpr<D>();  // rows per group
  const int64_t groups = (a.N + rpb - 1) / rpb;
  const int64_t by_head = (groups + kPreChunks - 1) / kPreChunks;
  const int64_t by_grid = (groups * BH + 2047) / 2048;
  int iters = (int)(by_head > by_grid ? by_head : by_grid);
  iters = iters < 1 ? 1 : iters;
  const int pre_rows = rpb * iters;  // rows per workgroup
  const int nchunk = (a.N + pre_rows - 1) / pre_rows;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D, true, RAW>), dim3(BH, nchunk), dim3(256), 0, a.stream,
                     static_cast<const uint16_t*>(a.o), dO, a.lse, q,
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), Dbuf,
                     shift, part, a.N, BH, iters, a.H, a.lay);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // convert: row blocks per workgroup so that the grid stays near 4096
  // workgroups (each reduces the partial maxima once)
  constexpr int crpb = 256 / (D / 8);  // rows per block
  const int64_t cblocks = (a.N + crpb - 1) / crpb;
  int citers = (int)((cblocks * BH) / 4096);
  citers = citers < 1 ? 1 : (citers > 16 ? 16 : citers);
  const int rbph = (int)((cblocks + citers - 1) / citers);  // convert workgroups per head
  hipLaunchKernelGGL((bwd_convert_kernel<T, D, RAW>), dim3((unsigned)((int64_t)BH * rbph)),
                     dim3(256), 0, a.stream, q, static_cast<const uint16_t*>(a.k), dO, Dbuf,
                     shift, part, nchunk, maxes, c, q16, k16, do16, nDs, nsh, a.N, BH, rbph,
                     citers, rexp, a.H, a.lay);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
hipError_t run_bwd(const BwdArgs& a, int stage) {
  hipError_t e = hipSuccess;
  const int BH = a.B * a.H;
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.H, a.N, a.d);
  char* ws = static_cast<char*>(a.workspace);
  float* Dbuf = reinterpret_cast<float*>(ws + w.D);
  float* shift = reinterpret_cast<float*>(ws + w.shift);
  float* nDs = reinterpret_cast<float*>(ws + w.nDs);
  float* nsh = reinterpret_cast<float*>(ws + w.nsh);
  const float c = a.scale * kLog2e;
  uint32_t* maxes = reinterpret_cast<uint32_t*>(ws + w.maxes);
  uint32_t* part = reinterpret_cast<uint32_t*>(ws + w.part);
  uint16_t* q16 = reinterpret_cast<uint16_t*>(ws + w.q16);
  uint16_t* do16 = reinterpret_cast<uint16_t*>(ws + w.do16);
  uint16_t* k16 = reinterpret_cast<uint16_t*>(ws + w.k16);
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* dO = static_cast<const uint16_t*>(a.dO);
  constexpr bool raw = use_raw<T>();
  if (stage == 0 || stage == 1) {
    e = launch_dpass<T, D, raw>(a, ws, w);
    if (e != hipSuccess || stage == 1) return e;
  }

  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.dO = static_cast<const uint16_t*>(a.dO);
  p.shift = shift;
  p.Dbuf = Dbuf;
  p.q16 = q16;
  p.do16 = do16;
  p.k16 = k16;
  p.nDs = nDs;
  p.nsh = nsh;
  p.maxes = maxes;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.H = a.H;
  p.N = a.N;
  p.BH = a.B * a.H;
  p.c = c;
  p.scale = a.scale;
  p.key_len = a.key_len;
  p.block_mask = a.block_mask;
  p.nblk = (a.N + 127) / 128;
  p.period = (FA_BWD_SNAKE && CAUSAL) ? snake_period(p.BH) : 0;
  p.drop = a.drop;
  p.sq = a.lay.q;
  p.sk = a.lay.k;
  p.sv = a.lay.v;
  p.sdO = a.lay.dO;
  p.sdq = a.lay.dq;
  p.sdk = a.lay.dk;
  p.sdv = a.lay.dv;

  return launch_grads<T, D, CAUSAL, SPARSE, DROP, raw>(p, a.stream, stage);
}

template <typename T, int D>
hipError_t dispatch_mask(const BwdArgs& a, int stage) {
  if (a.block_mask) return run_bwd<T, D, false, true, false>(a, stage);
  if (a.drop.on)
    return a.causal ? run_bwd<T, D, true, false, true>(a, stage)
                    : run_bwd<T, D, false, false, true>(a, stage);
  return a.causal ? run_bwd<T, D, true, false, false>(a, stage)
                  : run_bwd<T, D, false, false, false>(a, stage);
}

}  // namespace bwd

namespace bwd {
template <typename T>
hipError_t dispatch_dim(const BwdArgs& a, int stage) {
  switch (a.d) {
    case 32: return dispatch_mask<T, 32>(a, stage);
    case 64: return dispatch_mask<T, 64>(a, stage);
    case 96: return dispatch_mask<T, 96>(a, stage);
    default: return dispatch_mask<T, 128>(a, stage);
  }
}
}  // namespace bwd

hipError_t launch_bwd(const BwdArgs& a, int stage) {
  if (a.dtype == 0) return launch_bwd_f32(a, stage);
  if (a.dtype == 1) return bwd::dispatch_dim<_Float16>(a, stage);
  return bwd::dispatch_dim<__bf16>(a, stage);
}

}  // namespace fa
