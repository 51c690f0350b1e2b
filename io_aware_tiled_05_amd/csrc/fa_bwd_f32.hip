// fa_bwd_f32.hip — fp32 backward of exact tiled attention (dense, causal,
// key padding).
//
// Same recomputation as the 16-bit backward ([ODP] "FlashAttention: Fast
// and Memory-Efficient Exact Attention with IO-Awareness", section "The key
// idea"; [DEC] "FlashAttention, Decoded", "The Hardware Picture: Why Tiling
// Wins"): P is rebuilt tile by tile from Q, K and the forward's log-sum-exp;
// dV = P^T dO, dP = dO V^T, dS = P (dP - D), dQ = scale dS K, dK = scale
// dS^T Q with D_i = sum_c dO_ic O_ic.  Every product is an fp32 matrix-core
// product (v_mfma_f32_16x16x4_f32: A lane (n, g) = row n, k = g; B lane
// (n, g) = column n, k = g; accumulator element i of lane (n, g) = row
// 4g + i, column n) and P, dS stay fp32.
//
// The products that contract over the tile's rows take their k-operand
// straight from the score accumulator: the MFMA for element i of a 16-row
// block contracts over rows {4g + i} (k = g), so lane (n, g) supplies its
// own element i and the other operand is read from LDS at row 4g + i.
//
// Three launches: D and the base-2 shift per row; dK/dV (one workgroup per
// 64 keys, 16 per wave, query tiles of 64 through LDS); dQ (one workgroup
// per 64 queries, 16 per wave, key tiles of 64 through LDS).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace bwd32 {

constexpr int kT = 64;  // rows per LDS tile and per workgroup

struct Params {
  const float* q;
  const float* k;
  const float* v;
  const float* dO;
  const float* D;      // D_i
  const float* shift;  // lse_i log2(e); +inf for rows without keys
  float* dq;
  float* dk;
  float* dv;
  int H, N, BH, ntiles;
  float c, scale;  // c = scale log2(e)
  const int32_t* key_len;
  Layout lay;  // element strides of the caller's tensors (D and shift are packed)
};

__device__ __forceinline__ int valid_keys(const int32_t* key_len, int b, int N) {
  if (!key_len) return N;
  const int kl = key_len[b];
  return kl < 0 ? 0 : (kl > N ? N : kl);
}

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// D_i = sum_c dO_ic O_ic and shift_i = lse_i log2(e) (+inf when lse = -inf);
// 16 lanes per row, 16 rows per workgroup
template <int D>
__global__ __launch_bounds__(256) void pre_kernel(const float* o, const float* dO,
                                                  const float* lse, float* Dbuf, float* shift,
                                                  int64_t rows, int H, int N, Layout lay) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  float s = 0.f;
  if (row < rows) {
    const int64_t bh = row / N, r = row - bh * N, b = bh / H, hd = bh - b * H;
    const float* orow = o + b * lay.o.b + hd * lay.o.h + r * lay.o.n;
    const float* grow = dO + b * lay.dO.b + hd * lay.dO.h + r * lay.dO.n;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const int c = sub + 16 * j;
      s = fmaf(orow[c], grow[c], s);
    }
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  s += __shfl_xor(s, 8);
  if (row < rows && sub == 0) {
    Dbuf[row] = s;
    const float l = lse[row];
    shift[row] = l == neg_inf() ? pos_inf() : l * kLog2e;
  }
}

// rows r0 .. r0 + 63 of a matrix with D elements per row and row stride rs
// into LDS (row stride D + 1), zeros past N
template <int D>
__device__ __forceinline__ void load_tile(const float* g, int64_t rs, int r0, int N, float* s,
                                          int tid) {
  for (int c = tid; c < kT * D; c += 256) {
    const int r = c / D, col = c % D;
    s[r * (D + 1) + col] = r0 + r < N ? g[(int64_t)(r0 + r) * rs + col] : 0.f;
  }
}

__device__ __forceinline__ int64_t head_offset(const Strides& s, int bh, int H) {
  const int b = bh / H;
  return b * s.b + (bh - b * H) * s.h;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void dkdv_kernel(Params p) {
  constexpr int S = D + 1, KS = D / 4, DB = D / 16;
  __shared__ float sQ[kT * S], sO[kT * S], sD[kT], sL[kT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  int rank, bh;
  map_workgroup(blockIdx.x, p.ntiles, p.BH, 0, &rank, &bh);
  const int b = bh / p.H, N = p.N;
  const int L = valid_keys(p.key_len, b, N);
  const int k0 = rank * kT, key = k0 + wave * 16 + n;
  const float* const Q = p.q + head_offset(p.lay.q, bh, p.H);
  const float* const dOt = p.dO + head_offset(p.lay.dO, bh, p.H);

  // this wave's 16 keys and values as B operands (column n = key, k = d)
  float kf[KS], vf[KS];
  const float* const krow = p.k + head_offset(p.lay.k, bh, p.H) + (int64_t)key * p.lay.k.n;
  const float* const vrow = p.v + head_offset(p.lay.v, bh, p.H) + (int64_t)key * p.lay.v.n;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = key < N ? krow[4 * ks + g] : 0.f;
    vf[ks] = key < N ? vrow[4 * ks + g] : 0.f;
  }
  f32x4 dk[DB], dv[DB];  // dK^T, dV^T: row d = 16 db + 4g + i, column = key
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int t0 = CAUSAL ? k0 / kT : 0;  // earlier queries see none of these keys
  const int nqt = (N + kT - 1) / kT;
  for (int t = (k0 < L ? t0 : nqt); t < nqt; ++t) {
    const int q0 = t * kT;
    __syncthreads();
    load_tile<D>(Q, p.lay.q.n, q0, N, sQ, tid);
    load_tile<D>(dOt, p.lay.dO.n, q0, N, sO, tid);
    if (tid < kT) {
      const int r = q0 + tid;
      sD[tid] = r < N ? p.D[(size_t)bh * N + r] : 0.f;
      sL[tid] = r < N ? p.shift[(size_t)bh * N + r] : pos_inf();
    }
    __syncthreads();
    // S, dP: rows = queries 16 qb + 4g + i, column = this lane's key
    f32x4 s[4], dp[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) s[qb] = dp[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        s[qb] = mfma(sQ[(16 * qb + n) * S + 4 * ks + g], kf[ks], s[qb]);
        dp[qb] = mfma(sO[(16 * qb + n) * S + 4 * ks + g], vf[ks], dp[qb]);
      }
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * qb + 4 * g + i, query = q0 + r;
        const bool vis = (key < L) & (query < N) & (!CAUSAL | (key <= query));
        const float pv = vis ? fast_exp2(fmaf(s[qb][i], p.c, -sL[r])) : 0.f;
        s[qb][i] = pv;
        dp[qb][i] = pv * (dp[qb][i] - sD[r]);
      }
    // dV^T += dO^T P, dK^T += Q^T dS: k = rows {16 qb + 4g + i} for element i
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * qb + 4 * g + i;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = mfma(sO[r * S + 16 * db + n], s[qb][i], dv[db]);
          dk[db] = mfma(sQ[r * S + 16 * db + n], dp[qb][i], dk[db]);
        }
      }
  }
  if (key < N) {
    float* const dkrow = p.dk + head_offset(p.lay.dk, bh, p.H) + (int64_t)key * p.lay.dk.n;
    float* const dvrow = p.dv + head_offset(p.lay.dv, bh, p.H) + (int64_t)key * p.lay.dv.n;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int off = 16 * db + 4 * g + i;
        dkrow[off] = dk[db][i] * p.scale;
        dvrow[off] = dv[db][i];
      }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void dq_kernel(Params p) {
  constexpr int S = D + 1, KS = D / 4, DB = D / 16;
  __shared__ float sK[kT * S], sV[kT * S];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  int rank, bh;
  map_workgroup(blockIdx.x, p.ntiles, p.BH, 0, &rank, &bh);
  const int qt = CAUSAL ? p.ntiles - 1 - rank : rank;  // longest rows first
  const int b = bh / p.H, N = p.N;
  const int L = valid_keys(p.key_len, b, N);
  const int q0 = qt * kT, query = q0 + wave * 16 + n;
  const float* const K = p.k + head_offset(p.lay.k, bh, p.H);
  const float* const V = p.v + head_offset(p.lay.v, bh, p.H);

  float qf[KS], of[KS];  // B operands: column n = query, k = d
  const float* const qrow = p.q + head_offset(p.lay.q, bh, p.H) + (int64_t)query * p.lay.q.n;
  const float* const orow = p.dO + head_offset(p.lay.dO, bh, p.H) + (int64_t)query * p.lay.dO.n;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = query < N ? qrow[4 * ks + g] : 0.f;
    of[ks] = query < N ? orow[4 * ks + g] : 0.f;
  }
  const float shift = query < N ? p.shift[(size_t)bh * N + query] : pos_inf();
  const float Dq = query < N ? p.D[(size_t)bh * N + query] : 0.f;
  f32x4 acc[DB];  // dQ^T: row d = 16 db + 4g + i, column = query
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  int nkt = (L + kT - 1) / kT;
  if (CAUSAL) {
    const int last = (q0 + kT < N ? q0 + kT : N) - 1;
    nkt = nkt < last / kT + 1 ? nkt : last / kT + 1;
  }
  for (int t = 0; t < nkt; ++t) {
    const int kt0 = t * kT;
    __syncthreads();
    load_tile<D>(K, p.lay.k.n, kt0, N, sK, tid);
    load_tile<D>(V, p.lay.v.n, kt0, N, sV, tid);
    __syncthreads();
    // S^T, dP^T: rows = keys 16 kb + 4g + i, column = this lane's query
    f32x4 s[4], dp[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb] = dp[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = mfma(sK[(16 * kb + n) * S + 4 * ks + g], qf[ks], s[kb]);
        dp[kb] = mfma(sV[(16 * kb + n) * S + 4 * ks + g], of[ks], dp[kb]);
      }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kt0 + 16 * kb + 4 * g + i;
        const bool vis = (key < L) & (!CAUSAL | (key <= query));
        const float pv = vis ? fast_exp2(fmaf(s[kb][i], p.c, -shift)) : 0.f;
        dp[kb][i] = pv * (dp[kb][i] - Dq);
      }
    // dQ^T += K^T dS^T: k = keys {16 kb + 4g + i} for element i
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * kb + 4 * g + i;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = mfma(sK[r * S + 16 * db + n], dp[kb][i], acc[db]);
      }
  }
  if (query < N) {
    float* const dqrow = p.dq + head_offset(p.lay.dq, bh, p.H) + (int64_t)query * p.lay.dq.n;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<f32x4*>(dqrow + 16 * db + 4 * g) = acc[db] * p.scale;
  }
}

#define FA_BWD32_INSTANTIATE(D)                                                        \
  template __global__ void pre_kernel<D>(const float*, const float*, const float*,    \
                                         float*, float*, int64_t, int, int, Layout);   \
  template __global__ void dkdv_kernel<D, true>(Params);                               \
  template __global__ void dkdv_kernel<D, false>(Params);                              \
  template __global__ void dq_kernel<D, true>(Params);                                 \
  template __global__ void dq_kernel<D, false>(Params);
FA_BWD32_INSTANTIATE(32)
FA_BWD32_INSTANTIATE(64)
FA_BWD32_INSTANTIATE(96)
FA_BWD32_INSTANTIATE(128)
#undef FA_BWD32_INSTANTIATE

template <int D, bool CAUSAL>
hipError_t run(const BwdArgs& a, int stage) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.H, a.N, a.d);
  char* ws = static_cast<char*>(a.workspace);
  Params p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.dO = static_cast<const float*>(a.dO);
  p.D = reinterpret_cast<const float*>(ws + w.D);
  p.shift = reinterpret_cast<const float*>(ws + w.shift);
  p.dq = static_cast<float*>(a.dq);
  p.dk = static_cast<float*>(a.dk);
  p.dv = static_cast<float*>(a.dv);
  p.H = a.H;
  p.N = a.N;
  p.BH = a.B * a.H;
  p.ntiles = (a.N + kT - 1) / kT;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  p.key_len = a.key_len;
  p.lay = a.lay;
  hipError_t e = hipSuccess;
  if (stage == 0 || stage == 1) {
    const int64_t rows = (int64_t)p.BH * a.N;
    hipLaunchKernelGGL((pre_kernel<D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                       a.stream, static_cast<const float*>(a.o), p.dO, a.lse,
                       reinterpret_cast<float*>(ws + w.D), reinterpret_cast<float*>(ws + w.shift),
                       rows, a.H, a.N, a.lay);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage == 0 || stage == 2 || stage == 4) {
    hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL>), dim3(p.ntiles * p.BH), dim3(256), 0, a.stream,
                       p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage == 0 || stage == 3 || stage == 4) {
    hipLaunchKernelGGL((dq_kernel<D, CAUSAL>), dim3(p.ntiles * p.BH), dim3(256), 0, a.stream,
                       p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace bwd32

hipError_t launch_bwd_f32(const BwdArgs& a, int stage) {
  using namespace bwd32;
  switch (a.d) {
    case 32: return a.causal ? run<32, true>(a, stage) : run<32, false>(a, stage);
    case 64: return a.causal ? run<64, true>(a, stage) : run<64, false>(a, stage);
    case 96: return a.causal ? run<96, true>(a, stage) : run<96, false>(a, stage);
    default: return a.causal ? run<128, true>(a, stage) : run<128, false>(a, stage);
  }
}

}  // namespace fa
