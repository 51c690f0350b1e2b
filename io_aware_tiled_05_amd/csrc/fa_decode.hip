// fa_decode.hip — attention of a few new queries against a long key/value
// sequence (decode), split over the keys.
//
// Same exact attention as the forward ([ODP] "FlashAttention: Fast and
// Memory-Efficient Exact Attention with IO-Awareness", section "The key
// idea": a running maximum and running sum per query, partial outputs
// rescaled as key tiles arrive), arranged for the decode shape: with one
// or a few queries there is too little work per head to fill the GPU with
// query tiles, and the cost is reading K and V from HBM once.  The keys of
// each head are therefore cut into chunks, one workgroup per (chunk, head,
// group of 4 queries, or the single query when there is one), and every
// workgroup leaves a partial result (m, l, O)
// for its chunk; a second launch merges a query's partials by rescaling
// them to the common maximum — the same rescaling the online softmax does
// between key tiles.
//
// Partial kernel: a key row of d values is read by d/8 lanes, 16 bytes each
// (8 keys per wave and step at d = 64, 4 at d = 128), coalesced across the
// wave.  Per key and query the lanes reduce q.k with DPP moves inside their
// row of lanes (no LDS round trip); each lane
// keeps its own running (m, l, O-slice) in base 2 for the keys it sees.
// The key slots of a wave are merged with shuffles, the 4 waves through
// LDS.  The work is HBM-bound: about 4 d bytes of K and V per key against
// 4 d flops per key and query.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace dec {

constexpr int kQG = 4;  // queries per workgroup when there are several

// x of the lane that DPP control CTRL selects (every lane of the wave active)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum of x over each aligned group of G lanes (G = 4, 8, 16), in every lane
// of the group: quad swaps [1,0,3,2] and [2,3,0,1], then lane i <- 7 - i
// inside 8 lanes (row_half_mirror) and lane i <- 15 - i inside 16
// (row_mirror), each one DPP move.
template <int G>
__device__ __forceinline__ float group_sum_dpp(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  if constexpr (G >= 8) x += dpp_mov<0x141>(x);
  if constexpr (G >= 16) x += dpp_mov<0x140>(x);
  return x;
}

struct DecodeParams {
  const uint16_t* q;  // element type T (fp32 is read as two 16-byte halves)
  const uint16_t* k;
  const uint16_t* v;
  float* part;  // [BH][Nq][nchunks][d + 2]: O slice (d floats), m, l
  int H, Nq, Nk, BH, nchunks, chunk;
  float c;  // scale * log2(e)
  const int32_t* key_len;
};

// 8 consecutive elements of a row: raw 16-bit pairs (or fp32 values) as
// loaded, then widened to fp32 where they are used.  The loads are
// non-temporal: every cached key and value is read exactly once per call,
// so keeping it in the caches only displaces other lines (measured with
// B = 16, H = 16, 16384 keys, d = 64, bf16: 5932 -> 6430 GB/s).
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
template <typename T> struct Ld;
template <> struct Ld<__bf16> {
  static constexpr int ES = 2, NR = 1;  // bytes per element, 16-byte loads per 8 elements
  __device__ static void load(const uint16_t* p, u32x4 (&r)[NR]) { r[0] = ld_stream(p); }
  __device__ static void widen(const u32x4 (&r)[NR], float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __builtin_bit_cast(float, r[0][j] << 16);
      x[2 * j + 1] = __builtin_bit_cast(float, r[0][j] & 0xffff0000u);
    }
  }
};
template <> struct Ld<_Float16> {
  static constexpr int ES = 2, NR = 1;
  __device__ static void load(const uint16_t* p, u32x4 (&r)[NR]) { r[0] = ld_stream(p); }
  __device__ static void widen(const u32x4 (&r)[NR], float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(r[0][j] & 0xffffu));
      x[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(r[0][j] >> 16));
    }
  }
};
template <> struct Ld<float> {
  static constexpr int ES = 4, NR = 2;
  __device__ static void load(const uint16_t* p, u32x4 (&r)[NR]) {
    const f32x4* f = reinterpret_cast<const f32x4*>(p);
    r[0] = ld_stream(f);
    r[1] = ld_stream(f + 1);
  }
  __device__ static void widen(const u32x4 (&r)[NR], float (&x)[8]) {
    const f32x4 a = __builtin_bit_cast(f32x4, r[0]), b = __builtin_bit_cast(f32x4, r[1]);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};
template <typename T>
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  u32x4 r[Ld<T>::NR];
  Ld<T>::load(p, r);
  Ld<T>::widen(r, x);
}

// exp2(a - b) with exp2(-inf - -inf) taken as 0 (a partial without keys)
__device__ __forceinline__ float rel_exp2(float a, float b) {
  return a == neg_inf() ? 0.f : fast_exp2(a - b);
}

// grid: x = chunk + nchunks * bh, y = query group of QG queries; 256 threads
template <typename T, int D, int QG>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeParams p) {
  // lanes per key row: one per 8 elements, rounded up to a power of two for
  // the shuffle reductions (d = 96: 16 lanes, the last 4 hold no elements)
  constexpr int LPK = D / 8 <= 4 ? 4 : D / 8 <= 8 ? 8 : 16;
  constexpr int KPW = 64 / LPK;   // keys per wave and step
  constexpr int EB = Ld<T>::ES;   // bytes per element
  __shared__ float sm[4][QG], sl[4][QG];
  __shared__ float sO[4][QG][D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = blockIdx.x % p.nchunks, bh = blockIdx.x / p.nchunks;
  const int q0 = blockIdx.y * QG;
  const int nq = p.Nq - q0 < QG ? p.Nq - q0 : QG;
  const int b = bh / p.H;
  int L = p.Nk;
  if (p.key_len) {
    const int kl = p.key_len[b];
    L = kl < 0 ? 0 : (kl > p.Nk ? p.Nk : kl);
  }
  const int slot = lane / LPK, dsl = (lane % LPK) * 8;
  const bool dok = dsl < D;  // this lane holds a d-slice
  // this wave's keys: a quarter of the chunk
  const int wlen = p.chunk / 4;
  const int kb = chunk * p.chunk + wave * wlen;
  const int ke = kb + wlen < L ? kb + wlen : L;

  // queries (scaled by c, base 2), this lane's d-slice
  float qv[QG][8];
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    if (i < nq && dok) {
      const size_t off = (((size_t)bh * p.Nq + q0 + i) * D + dsl) * (EB / 2);
      load8<T>(p.q + off, qv[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[i][e] *= p.c;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[i][e] = 0.f;
    }
  }
  float m[QG], l[QG], o[QG][8];
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    m[i] = neg_inf();
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[i][e] = 0.f;
  }

  const size_t kvbase = (size_t)bh * p.Nk * D;
  // U key steps per iteration: their K and V loads are issued together
  // before any of them is used, so that several 16-byte loads per lane are
  // in flight (the loop holds cross-lane moves, which the compiler does not
  // unroll).  16-bit data: 16 steps (32 loads in flight per lane, about 160
  // registers; measured 2-3 % above 4 or 8 steps); fp32 takes two loads per
  // step and keeps 4 (16 steps would need over 256 registers).
#ifndef FA_DEC_STEPS
#define FA_DEC_STEPS 16
#endif
  constexpr int U = Ld<T>::ES == 4 ? 4 : FA_DEC_STEPS;
  constexpr int NR = Ld<T>::NR;
  for (int k0 = kb; k0 < ke; k0 += KPW * U) {
    u32x4 kr[U][NR], vr[U][NR];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = k0 + u * KPW + slot;
      ok[u] = key < ke;
      if (ok[u] && dok) {
        const size_t off = (kvbase + (size_t)key * D + dsl) * (EB / 2);
        Ld<T>::load(p.k + off, kr[u]);
        Ld<T>::load(p.v + off, vr[u]);
      } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) kr[u][r] = vr[u][r] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8], vf[8];
      Ld<T>::widen(kr[u], kf);
      Ld<T>::widen(vr[u], vf);
#pragma unroll
      for (int i = 0; i < QG; ++i) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(qv[i][e], kf[e], s);
        s = group_sum_dpp<LPK>(s);
        s = ok[u] ? s : neg_inf();
        const float mn = fmaxf(m[i], s);
        const float alpha = rel_exp2(m[i], mn);
        const float pv = rel_exp2(s, mn);
        m[i] = mn;
        l[i] = fmaf(l[i], alpha, pv);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[i][e] = fmaf(o[i][e], alpha, pv * vf[e]);
      }
    }
  }

  // merge the key slots of the wave (lanes LPK apart hold the same d-slice)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < QG; ++i) {
      const float mo = __shfl_xor(m[i], off), lo = __shfl_xor(l[i], off);
      const float mn = fmaxf(m[i], mo);
      const float a = rel_exp2(m[i], mn), bb = rel_exp2(mo, mn);
      l[i] = l[i] * a + lo * bb;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[i][e] = o[i][e] * a + __shfl_xor(o[i][e], off) * bb;
      m[i] = mn;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int i = 0; i < QG; ++i) {
      if (dok)
#pragma unroll
        for (int e = 0; e < 8; ++e) sO[wave][i][dsl + e] = o[i][e];
      if (lane == 0) {
        sm[wave][i] = m[i];
        sl[wave][i] = l[i];
      }
    }
  }
  __syncthreads();
  // merge the 4 waves and write the chunk's partial: thread = (query, d)
  for (int t = tid; t < nq * D; t += 256) {
    const int i = t / D, dd = t % D;
    float mn = sm[0][i];
#pragma unroll
    for (int w = 1; w < 4; ++w) mn = fmaxf(mn, sm[w][i]);
    float ls = 0.f, os = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = rel_exp2(sm[w][i], mn);
      ls += sl[w][i] * a;
      os += sO[w][i][dd] * a;
    }
    float* out = p.part + (((size_t)bh * p.Nq + q0 + i) * p.nchunks + chunk) * (D + 2);
    out[dd] = os;
    if (dd == 0) {
      out[D] = mn;
      out[D + 1] = ls;
    }
  }
}

// one workgroup of D threads per (head, query): combine the chunk partials
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* part, uint16_t* o,
                                                          float* lse, int nchunks) {
  const int row = blockIdx.x, dd = threadIdx.x;  // row = bh * Nq + query
  const float* pr = part + (size_t)row * nchunks * (D + 2);
  float mn = neg_inf();
#pragma unroll 8
  for (int c = 0; c < nchunks; ++c) mn = fmaxf(mn, pr[(size_t)c * (D + 2) + D]);
  float ls = 0.f, os = 0.f;
  if (mn != neg_inf()) {
#pragma unroll 8
    for (int c = 0; c < nchunks; ++c) {
      const float* pc = pr + (size_t)c * (D + 2);
      const float a = rel_exp2(pc[D], mn);
      ls += pc[D + 1] * a;
      os += pc[dd] * a;
    }
  }
  const float val = ls > 0.f ? os / ls : 0.f;
  if constexpr (Ld<T>::ES == 4) {
    reinterpret_cast<float*>(o)[(size_t)row * D + dd] = val;
  } else {
    o[(size_t)row * D + dd] = __builtin_bit_cast(uint16_t, (T)val);
  }
  if (dd == 0) lse[row] = ls > 0.f ? (mn + fast_log2(ls)) * kLn2 : neg_inf();
}

#define FA_DEC_INSTANTIATE(T, D)                                                  \
  template __global__ void decode_partial_kernel<T, D, 1>(DecodeParams);         \
  template __global__ void decode_partial_kernel<T, D, kQG>(DecodeParams);       \
  template __global__ void decode_merge_kernel<T, D>(const float*, uint16_t*, float*, int);
#define FA_DEC_INSTANTIATE_D(D) \
  FA_DEC_INSTANTIATE(__bf16, D) FA_DEC_INSTANTIATE(_Float16, D) FA_DEC_INSTANTIATE(float, D)
FA_DEC_INSTANTIATE_D(32)
FA_DEC_INSTANTIATE_D(64)
FA_DEC_INSTANTIATE_D(96)
FA_DEC_INSTANTIATE_D(128)
#undef FA_DEC_INSTANTIATE_D
#undef FA_DEC_INSTANTIATE

template <typename T, int D>
hipError_t run_decode(const DecodeArgs& a) {
  const DecodeSplit sp = decode_split(a.B, a.H, a.Nq, a.Nk, a.d);
  DecodeParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.part = static_cast<float*>(a.workspace);
  p.H = a.H;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.BH = a.B * a.H;
  p.nchunks = sp.nchunks;
  p.chunk = sp.chunk;
  p.c = a.scale * kLog2e;
  p.key_len = a.key_len;
  // one query: a group of one (no idle query slots in the inner loop)
  const dim3 grid((unsigned)(sp.nchunks * p.BH), (unsigned)((a.Nq + kQG - 1) / kQG));
  if (a.Nq == 1)
    hipLaunchKernelGGL((decode_partial_kernel<T, D, 1>), grid, dim3(256), 0, a.stream, p);
  else
    hipLaunchKernelGGL((decode_partial_kernel<T, D, kQG>), grid, dim3(256), 0, a.stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)(p.BH * a.Nq)), dim3(D), 0,
                     a.stream, p.part, static_cast<uint16_t*>(a.o), a.lse, sp.nchunks);
  return hipGetLastError();
}

}  // namespace dec

namespace dec {
template <typename T>
hipError_t dispatch_dim(const DecodeArgs& a) {
  switch (a.d) {
    case 32: return run_decode<T, 32>(a);
    case 64: return run_decode<T, 64>(a);
    case 96: return run_decode<T, 96>(a);
    default: return run_decode<T, 128>(a);
  }
}
}  // namespace dec

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.dtype == 0) return dec::dispatch_dim<float>(a);
  if (a.dtype == 1) return dec::dispatch_dim<_Float16>(a);
  return dec::dispatch_dim<__bf16>(a);
}

}  // namespace fa
