// fa_fwd.hip — forward kernels of exact tiled attention for gfx950.
//
// Method ([ODP] "FlashAttention: Fast and Memory-Efficient Exact Attention
// with IO-Awareness", section "The key idea"; [DEC] "FlashAttention,
// Decoded", "Decoding the Abstract", Sentence 4; [HFL] "FlashAttention: A
// Novel Attention Algorithm with IO Awareness", section "FlashAttention"):
// a workgroup owns a tile of query rows, streams the key/value tiles of its
// head through LDS, and keeps per query a running maximum m and running sum
// l of the exponentiated scores; when m grows the partial output is rescaled
// by exp(m_old - m_new).  Q is read from HBM once, O and the row statistic
// are written once, and no score ever leaves the chip.
//
// Work split (16-bit path): 256 threads = 4 waves per workgroup.  A wave
// owns QW query rows (64 at d <= 64; 32 at d >= 96, with dropout, and for
// block-sparse masks, whose workgroup covers one 128-query mask row) held
// in registers as the
// B operand of the transposed score tile S^T = K Q^T, computed with
// v_mfma_f32_32x32x16: a lane holds 16 keys of one query column, so the
// per-query reductions are in-lane plus one exchange with lane ^ 32, and
// the scores rounded to 16 bits are already laid out as the k-operand of
// O^T += V^T P^T (V^T comes from the row-major V tile through the LDS
// transpose read).  Key/value tiles of 64 rows are double buffered in LDS
// and filled with direct global->LDS loads one tile ahead of the compute.
//
// Softmax runs in base 2 (scale*log2(e) folded into one FMA per score).  The
// reference maximum m is only moved when a tile could push an
// exponentiated score above 2^8: each lane sums its 32 probabilities of the
// tile (v_dot2c over the packed 16-bit values, which also gives the row sum
// l of exactly the values the P V product uses) and the wave takes the
// rescaling path only if some partial sum exceeds 256 (or is inf/NaN, which
// is how the first tile of every row enters it).  Between rescalings the
// output, l and m stay consistent, so the result is the same softmax up to
// rounding; per-tile maxima are not needed on the common path.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace fwd {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int H, N, BH, nqt;
  int period;  // snake period of map_workgroup (0: plain order)
  float c;  // scale * log2(e)
  const int32_t* key_len;
  const uint8_t* block_mask;
  int nblk;
  Dropout drop;  // used by the DROP kernels only
  Strides sq, sk, sv, so;  // element strides of q, k, v, o (lse is packed [B][H][N])
};

// Compile-time tuning knobs (defaults are the measured best).
#ifndef FA_FWD_WAVES_PER_SIMD
#define FA_FWD_WAVES_PER_SIMD 2
#endif

constexpr int kBC = 64;              // key rows per LDS tile
constexpr int kBR = 128;             // queries per workgroup of the fp32 kernel
constexpr int kListMax = 1024;       // block-sparse: active blocks listed per pass
constexpr float kRescaleAt = 256.f;  // largest probability allowed between rescalings

__device__ __forceinline__ int valid_keys(const int32_t* key_len, int b, int N) {
  if (!key_len) return N;
  int kl = key_len[b];
  return kl < 0 ? 0 : (kl > N ? N : kl);
}

template <int D>
struct FwdShape {
  static constexpr int QW = D <= 64 ? 64 : 32;  // default queries per wave
  static constexpr int NQB = QW / 32;           // 32-query MFMA blocks per wave
  static constexpr int KS = D / 16;             // k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;             // 32-row blocks of O^T
  static constexpr int TILE = kBC * D;          // elements per K or V tile
};

// NW waves per workgroup of QW (32 or 64) queries each; a workgroup covers
// NW * QW queries.
// DROP: dropout on P before the product with V (P kept with probability
// 1 - p and scaled by 1 / (1 - p); the row sum l and lse use P itself).
template <typename T, int D, int NW, int QW, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(64 * NW, FA_FWD_WAVES_PER_SIMD) void fwd_kernel(FwdParams p) {
  typedef FwdShape<D> Sh;
  static_assert(QW == 32 || QW == 64, "a wave holds one or two 32-query blocks");
  constexpr int NQB = QW / 32, KS = Sh::KS, DB = Sh::DB;
  constexpr int TILE = Sh::TILE;
  constexpr int BR = NW * QW;
  typedef typename Elt<T>::vec8 vec8;
  // two K and two V tile buffers, separate arrays so that the compiler can
  // tell the buffer being filled from the one being read
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[TILE];
  __shared__ int sList[SPARSE ? kListMax : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  int rank, bh;
  // One query tile per workgroup; causal grids take the longest tiles (the
  // most keys) first, so that the dispatcher fills the compute units that
  // finish early with the short tiles at the end.
  map_workgroup(blockIdx.x, p.nqt, p.BH, p.period, &rank, &bh);
  const int qt = CAUSAL ? p.nqt - 1 - rank : rank;
  const int b = bh / p.H, hd = bh - b * p.H, N = p.N;
  const uint16_t* Q = p.q + b * p.sq.b + hd * p.sq.h;
  const uint16_t* K = p.k + b * p.sk.b + hd * p.sk.h;
  const uint16_t* V = p.v + b * p.sv.b + hd * p.sv.h;
  const int L = valid_keys(p.key_len, b, N);
  const int q0 = qt * BR, qw = q0 + wave * QW;
  const float c = p.c;

  // one set of chunk offsets for K's row stride; V (normally the same
  // stride) adjusts them when its stride differs
  const TileCopy<D, kBC, NW> copy(wave, lane, p.sk.n);
  // Dense masks: key tiles 0 .. nkt-1 (causal: up to the diagonal of the
  // last query).  The first tile's copies are issued before the loads of
  // this wave's queries below, so that the two global latencies overlap.
  int nkt = (L + kBC - 1) / kBC;
  if (CAUSAL) {
    const int last = (q0 + BR < N ? q0 + BR : N) - 1;
    nkt = nkt < last / kBC + 1 ? nkt : last / kBC + 1;
  }
  const bool primed = !SPARSE && nkt > 0;
  if (primed) {
    copy(K, 0, N, sK0);
    copy.copy_rs(V, p.sv.n, 0, N, sV0);
  }

  // This wave's queries as B operands of S^T = K Q^T: lane = query column
  // l32 of block qb, k = d values 16 ks + 8 h .. +7.
  vec8 qf[NQB][KS];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = qw + qb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[qb][ks] = as_vec8<T>(ldg16_clamp(Q, row, p.sq.n, ks * 16 + h * 8, N));
  }

  float m[NQB], mc[NQB], l[NQB];  // reference max (raw score), m * c, partial row sum
  f32x16 acc[DB][NQB];            // O^T, relative to the reference
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m[qb] = neg_inf();
    mc[qb] = neg_inf();  // "no reference yet": forces the rescaling path
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[db][qb][e] = 0.f;
  }

  // per-lane LDS element offsets (tile-invariant)
  // K reads: row kb*32 + l32, chunk 2 ks + h  -> kb adds 32*D
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = tile_off<D>(l32, ks * 16 + h * 8);
  // V^T transpose reads: 16-lane group g4 = lane / 16; lanes of a group
  // address rows 16a + 4h + sub/4 (+8 for the second read), columns
  // db*32 + 16*(g4&1) + 4*(sub%4) .. +3.  a adds 16*D.
  const int sub = lane & 15, g4 = lane >> 4;
  int voff[2][DB];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      voff[sec][db] = tile_off<D>(4 * h + (sub >> 2) + 8 * sec,
                                  db * 32 + 16 * (g4 & 1) + 4 * (sub & 3));

  // one 64-key tile from LDS buffer `buf` (key rows kt0 ..)
  auto compute = [&](const uint16_t* kt, const uint16_t* vt, int kt0) {
    if (qw >= N) return;                        // wave has no query rows
    if (CAUSAL && kt0 > qw + QW - 1) return;    // tile above the diagonal

    // S^T for 64 keys (2 blocks of 32) x QW queries
    f32x16 s[2][NQB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kb][qb][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const vec8 a = as_vec8<T>(lds16(kt + koff[ks] + kb * 32 * D));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = Elt<T>::mfma32(a, qf[qb][ks], s[kb][qb]);
      }

    // -inf on keys past key_len / above the diagonal (boundary tiles only);
    // accumulator element 4i+j of block kb is key kt0 + 32kb + 8i + 4h + j
    const bool need_mask = (kt0 + kBC > L) || (CAUSAL && kt0 + kBC - 1 > qw);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kt0 + kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            const int query = qw + qb * 32 + l32;
            if (key >= L || (CAUSAL && key > query)) s[kb][qb][e] = neg_inf();
          }
    }

    // P = exp2(c s - m c), packed to 16 bits; rs = this lane's part of the
    // tile's row sum (of the rounded values)
    uint32_t pk[2][NQB][8];
    float rs[NQB];
    auto exp_pack = [&](int qb, float msc) {
      float r[4] = {0.f, 0.f, 0.f, 0.f};  // four independent sum chains
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};  // dropout draws of the current 8 keys
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float x0 = fast_exp2(fmaf(s[kb][qb][2 * e], c, -msc));
          float x1 = fast_exp2(fmaf(s[kb][qb][2 * e + 1], c, -msc));
          if constexpr (DROP) {
            // elements 8c .. 8c+7 (pairs e = 4c .. 4c+3) are keys
            // kt0 + 32 kb + 16 c + 4 h + {0..3, 8..11}: one generator call;
            // pair e takes word e % 4, low half for x0 and high for x1
            if ((e & 3) == 0)
              philox4x32_10((uint32_t)drop_call(kt0 + kb * 32 + 16 * (e >> 2) + 4 * h),
                            (uint32_t)(qw + qb * 32 + l32), (uint32_t)bh, p.drop.offset,
                            p.drop.k0, p.drop.k1, w);
            r[(2 * e) & 3] += x0;
            r[(2 * e + 1) & 3] += x1;
            const uint32_t wd = w[e & 3];
            x0 = (wd & 0xFFFFu) >= p.drop.thresh ? x0 * p.drop.rinv : 0.f;
            x1 = wd >= (p.drop.thresh << 16) ? x1 * p.drop.rinv : 0.f;
            pk[kb][qb][e] = Elt<T>::pack2(x0, x1);
          } else {
            pk[kb][qb][e] = Elt<T>::pack2(x0, x1);
            r[e & 3] = Elt<T>::sum2(pk[kb][qb][e], r[e & 3]);
          }
        }
      }
      rs[qb] = (r[0] + r[1]) + (r[2] + r[3]);
    };
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      exp_pack(qb, mc[qb]);
      over |= !(rs[qb] <= kRescaleAt);
    }
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
      // move the reference to the running maximum and rescale
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float mx = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][qb][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m[qb], mx);
        const float msc = mn == neg_inf() ? 0.f : mn * c;
        const float alpha = fast_exp2(m[qb] * c - msc);  // 0 while m = -inf
        m[qb] = mn;
        mc[qb] = mn == neg_inf() ? neg_inf() : msc;
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
        exp_pack(qb, msc);
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) l[qb] += rs[qb];

    // O^T += V^T P^T, 16 keys per MFMA k-step (a = 16-key chunk of the tile)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const vec8 va = join8<T>(lds_tr4(vt + voff[0][db] + a * 16 * D),
                                 lds_tr4(vt + voff[1][db] + a * 16 * D));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const uint32_t* pp = &pk[a >> 1][qb][(a & 1) * 4];
          const u32x4 pb = {pp[0], pp[1], pp[2], pp[3]};
          acc[db][qb] = Elt<T>::mfma32(va, as_vec8<T>(pb), acc[db][qb]);
        }
      }
    }
  };

  // Walk `ntiles` tiles (first key of tile t = key0(t)) with the copy of
  // tile t+1 in flight while tile t is computed.  One barrier per tile.
  // `primed`: the first tile's copies are already in flight.
  auto walk = [&](int ntiles, auto key0, bool primed_) {
    if (ntiles <= 0) return;
    if (!primed_) {
      copy(K, key0(0), N, sK0);
      copy.copy_rs(V, p.sv.n, key0(0), N, sV0);
    }
    auto step = [&](int t, const uint16_t* kc, const uint16_t* vc, uint16_t* kn, uint16_t* vn) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of tile t landed
      __syncthreads();                     // ... and every wave's; tile t-1 fully read
      if (t + 1 < ntiles) {
        const int nk = key0(t + 1);
        copy(K, nk, N, kn);
        copy.copy_rs(V, p.sv.n, nk, N, vn);
      }
      compute(kc, vc, key0(t));
    };
    for (int t = 0; t < ntiles; t += 2) {
      step(t, sK0, sV0, sK1, sV1);
      if (t + 1 < ntiles) step(t + 1, sK1, sV1, sK0, sV0);
    }
    __syncthreads();  // LDS free for the caller
  };

  if (SPARSE) {
    // Active 128-key blocks of this 128-query block row, two tiles each,
    // gathered into LDS a window of kListMax blocks at a time.
    const uint8_t* mrow = p.block_mask + (size_t)qt * p.nblk;
    for (int w0 = 0; w0 < p.nblk; w0 += kListMax) {
      const int wend = w0 + kListMax < p.nblk ? w0 + kListMax : p.nblk;
      int cnt = 0;
      for (int j0 = w0; j0 < wend; j0 += 64) {
        const int jb = j0 + lane;
        const bool on = jb < wend && mrow[jb] != 0;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
        if (wave == 0 && on) sList[cnt + __builtin_popcountll(bal & ((1ull << lane) - 1))] = jb;
        cnt += __builtin_popcountll(bal);
      }
      __syncthreads();
      walk(2 * cnt, [&](int t) { return sList[t >> 1] * 128 + (t & 1) * kBC; }, false);
    }
  } else {
    walk(nkt, [](int t) { return t * kBC; }, primed);
  }

  // epilogue: O = O^T / l, lse = (m c + log2 l) ln 2
  uint16_t* O = p.o + b * p.so.b + hd * p.so.h;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    const int query = qw + qb * 32 + l32;
    if (query < N) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 o4 = {acc[db][qb][4 * i] * inv, acc[db][qb][4 * i + 1] * inv,
                            acc[db][qb][4 * i + 2] * inv, acc[db][qb][4 * i + 3] * inv};
          *reinterpret_cast<u32x2*>(O + (int64_t)query * p.so.n + db * 32 + 8 * i + 4 * h) =
              pack4<T>(o4);
        }
      if (h == 0)
        p.lse[(size_t)bh * N + query] = lt > 0.f ? (mc[qb] + fast_log2(lt)) * kLn2 : neg_inf();
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 forward: same tiling and softmax, fp32 products through
// v_mfma_f32_16x16x4_f32 (A: row n, k = g; B: col n, k = g).  P stays fp32.
// ---------------------------------------------------------------------------
struct FwdParamsF32 {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int H, N, BH, nqt;
  int period;
  float c;
  const int32_t* key_len;
  Strides sq, sk, sv, so;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdParamsF32 p) {
  constexpr int S = D + 1;  // LDS row stride (floats)
  constexpr int DB = D / 16;
  __shared__ float sK[kBC * S];
  __shared__ float sV[kBC * S];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  int rank, bh;
  map_workgroup(blockIdx.x, p.nqt, p.BH, p.period, &rank, &bh);
  const int qt = CAUSAL ? p.nqt - 1 - rank : rank;
  const int b = bh / p.H, hd = bh - b * p.H, N = p.N;
  const float* Q = p.q + b * p.sq.b + hd * p.sq.h;
  const float* K = p.k + b * p.sk.b + hd * p.sk.h;
  const float* V = p.v + b * p.sv.b + hd * p.sv.h;
  const int L = valid_keys(p.key_len, b, N);
  const int q0 = qt * kBR, qw = q0 + wave * 32;

  float qf[2][D / 4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qw + qb * 16 + n;
#pragma unroll
    for (int ks = 0; ks < D / 4; ++ks)
      qf[qb][ks] = row < N ? Q[(int64_t)row * p.sq.n + ks * 4 + g] : 0.f;
  }
  float m[2] = {neg_inf(), neg_inf()}, l[2] = {0.f, 0.f};
  f32x4 acc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) acc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  int nkt = (L + kBC - 1) / kBC;
  if (CAUSAL) {
    const int last = (q0 + kBR < N ? q0 + kBR : N) - 1;
    nkt = nkt < last / kBC + 1 ? nkt : last / kBC + 1;
  }
  for (int t = 0; t < nkt; ++t) {
    const int kt0 = t * kBC;
    __syncthreads();
    for (int c = tid; c < kBC * D; c += 256) {
      const int r = c / D, col = c % D, key = kt0 + r;
      sK[r * S + col] = key < N ? K[(int64_t)key * p.sk.n + col] : 0.f;
      sV[r * S + col] = key < N ? V[(int64_t)key * p.sv.n + col] : 0.f;
    }
    __syncthreads();
    if (qw >= N || (CAUSAL && kt0 > qw + 31)) continue;
    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 4; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float a = sK[(kb * 16 + n) * S + ks * 4 + g];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qf[qb][ks], s[kb][qb], 0, 0, 0);
      }
    const bool need_mask = (kt0 + kBC > L) || (CAUSAL && kt0 + kBC - 1 > qw);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kt0 + kb * 16 + g * 4 + i, query = qw + qb * 16 + n;
            if (key >= L || (CAUSAL && key > query)) s[kb][qb][i] = neg_inf();
          }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][qb][i]);
      mx = group_max(mx);
      const float mn = fmaxf(m[qb], mx);
      const float msc = (mn == neg_inf()) ? 0.f : mn * p.c;
      const float alpha = fast_exp2(m[qb] * p.c - msc);
      m[qb] = mn;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(fmaf(s[kb][qb][i], p.c, -msc));
          s[kb][qb][i] = e;
          rs += e;
        }
      l[qb] = l[qb] * alpha + rs;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const float a = sV[(kb * 16 + g * 4 + i) * S + db * 16 + n];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            acc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, s[kb][qb][i], acc[db][qb], 0, 0, 0);
        }
  }
  float* O = p.o + b * p.so.b + hd * p.so.h;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = group_sum(l[qb]);
    const int query = qw + qb * 16 + n;
    if (query < N) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(O + (int64_t)query * p.so.n + db * 16 + g * 4) =
            acc[db][qb] * inv;
      if (g == 0)
        p.lse[(size_t)bh * N + query] =
            lt > 0.f ? (m[qb] * p.c + fast_log2(lt)) * kLn2 : neg_inf();
    }
  }
}

// Explicit instantiations of every kernel the launchers below can select.
// (Without them the host pass of this compiler leaves some kernel-template
// launch stubs undefined.)
#define FA_FWD_INSTANTIATE(T, D)                                                              \
  template __global__ void fwd_kernel<T, D, 4, 32, false, true, false>(FwdParams);           \
  template __global__ void fwd_kernel<T, D, 4, FwdShape<D>::QW, true, false, false>(          \
      FwdParams);                                                                            \
  template __global__ void fwd_kernel<T, D, 4, FwdShape<D>::QW, false, false, false>(         \
      FwdParams);                                                                            \
  template __global__ void fwd_kernel<T, D, 4, 32, true, false, true>(FwdParams);            \
  template __global__ void fwd_kernel<T, D, 4, 32, false, false, true>(FwdParams);
// the two-wave, 32-query dense kernels that small grids select where 64 is
// the default
#define FA_FWD_INSTANTIATE_SMALL(T, D)                                                        \
  template __global__ void fwd_kernel<T, D, 2, 32, true, false, false>(FwdParams);           \
  template __global__ void fwd_kernel<T, D, 2, 32, false, false, false>(FwdParams);

#define FA_FWD_INSTANTIATE_D(D)                                                               \
  FA_FWD_INSTANTIATE(__bf16, D)                                                              \
  FA_FWD_INSTANTIATE(_Float16, D)                                                            \
  template __global__ void fwd_f32_kernel<D, true>(FwdParamsF32);                            \
  template __global__ void fwd_f32_kernel<D, false>(FwdParamsF32);
FA_FWD_INSTANTIATE_D(32)
FA_FWD_INSTANTIATE_D(64)
FA_FWD_INSTANTIATE_D(96)
FA_FWD_INSTANTIATE_D(128)
static_assert(FwdShape<32>::QW == 64 && FwdShape<64>::QW == 64, "small-grid variants below");
FA_FWD_INSTANTIATE_SMALL(__bf16, 32)
FA_FWD_INSTANTIATE_SMALL(_Float16, 32)
FA_FWD_INSTANTIATE_SMALL(__bf16, 64)
FA_FWD_INSTANTIATE_SMALL(_Float16, 64)
#undef FA_FWD_INSTANTIATE_SMALL
#undef FA_FWD_INSTANTIATE_D
#undef FA_FWD_INSTANTIATE

template <typename T, int D, int QW, bool CAUSAL, bool SPARSE, bool DROP, int NWD = 4>
hipError_t launch_fwd_kernel(const FwdArgs& a) {
  // block-sparse workgroups cover exactly one 128-query mask row; dense
  // ones NWD waves
  constexpr int NW = SPARSE ? 128 / QW : NWD;
  constexpr int BR = NW * QW;
  FwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
  p.lse = a.lse;
  p.H = a.H;
  p.N = a.N;
  p.BH = a.B * a.H;
  p.nqt = (a.N + BR - 1) / BR;
  p.period = 0;  // plain order: causal grids longest tile first
  p.c = a.scale * kLog2e;
  p.key_len = a.key_len;
  p.block_mask = a.block_mask;
  p.nblk = (a.N + 127) / 128;
  p.drop = a.drop;
  p.sq = a.lay.q;
  p.sk = a.lay.k;
  p.sv = a.lay.v;
  p.so = a.lay.o;
  hipLaunchKernelGGL((fwd_kernel<T, D, NW, QW, CAUSAL, SPARSE, DROP>),
                     dim3(p.nqt * p.BH), dim3(64 * NW), 0, a.stream, p);
  return hipGetLastError();
}

// Queries per wave: 32 with dropout (the generator's registers do not fit
// next to two query blocks) and for block-sparse masks (four waves share
// each K/V tile of a 128-query mask row: measured 3-5 % faster than two
// waves of 64 queries).  Dense 64-query waves at d <= 64 halve the LDS
// reads per MFMA, but when their grid holds less work than one full tile per
// compute unit (a causal grid counting half its tiles, the average causal
// tile seeing half the keys), workgroups of two 32-query waves (four times
// the workgroups) finish sooner (causal B = 8, H = 12, N = 1024: 768
// instead of 192 workgroup-equivalents, 45.6 -> 33.8 us; four waves of 32
// queries: 37.0 us; with 256 workgroup-equivalents on 256 CUs, 64-query
// waves stay ahead).
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
hipError_t run_fwd(const FwdArgs& a) {
  constexpr int QW = (DROP || SPARSE) ? 32 : FwdShape<D>::QW;
  if constexpr (QW == 64) {
    const int nqt = (a.N + 4 * QW - 1) / (4 * QW);
    const long wgs = (long)(CAUSAL ? (nqt + 1) / 2 : nqt) * a.B * a.H;
    const int cus = device_cu_count();
    if (cus > 0 && wgs < cus) return launch_fwd_kernel<T, D, 32, CAUSAL, SPARSE, DROP, 2>(a);
  }
  return launch_fwd_kernel<T, D, QW, CAUSAL, SPARSE, DROP>(a);
}

template <int D, bool CAUSAL>
hipError_t run_fwd_f32(const FwdArgs& a) {
  FwdParamsF32 p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.o = static_cast<float*>(a.o);
  p.lse = a.lse;
  p.H = a.H;
  p.N = a.N;
  p.BH = a.B * a.H;
  p.nqt = (a.N + kBR - 1) / kBR;
  p.period = CAUSAL ? snake_period(p.BH) : 0;
  p.c = a.scale * kLog2e;
  p.key_len = a.key_len;
  p.sq = a.lay.q;
  p.sk = a.lay.k;
  p.sv = a.lay.v;
  p.so = a.lay.o;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(p.nqt * p.BH), dim3(256), 0, a.stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dispatch_mask(const FwdArgs& a) {
  if constexpr (std::is_same<T, float>::value) {
    return a.causal ? run_fwd_f32<D, true>(a) : run_fwd_f32<D, false>(a);
  } else {
    if (a.block_mask) return run_fwd<T, D, false, true, false>(a);
    if (a.drop.on)
      return a.causal ? run_fwd<T, D, true, false, true>(a) : run_fwd<T, D, false, false, true>(a);
    return a.causal ? run_fwd<T, D, true, false, false>(a) : run_fwd<T, D, false, false, false>(a);
  }
}

template <typename T>
hipError_t dispatch_dim(const FwdArgs& a) {
  switch (a.d) {
    case 32: return dispatch_mask<T, 32>(a);
    case 64: return dispatch_mask<T, 64>(a);
    case 96: return dispatch_mask<T, 96>(a);
    default: return dispatch_mask<T, 128>(a);
  }
}

}  // namespace fwd

using namespace fwd;

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.dtype == 0) return dispatch_dim<float>(a);  // FA_F32
  if (a.dtype == 1) return dispatch_dim<_Float16>(a);
  return dispatch_dim<__bf16>(a);
}

}  // namespace fa
