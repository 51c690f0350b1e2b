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
// Three launches, no atomics (deterministic):
//   bwd_pre   D for every query row (bandwidth-bound, one pass over O, dO);
//   bwd_dkdv  one workgroup per 128 keys (32 per wave), query tiles of 64
//             rows streamed through LDS: S = Q K^T and dP = dO V^T come out
//             with the key in the lane's column, so bf16(P) and bf16(dS) are
//             directly the k-operands of dV^T += dO^T P and dK^T += Q^T dS
//             (dO^T and Q^T via the LDS transpose read);
//   bwd_dq    one workgroup per 128 queries (32 per wave), key tiles of 64
//             rows streamed through LDS: S^T = K Q^T and dP^T = V dO^T keep
//             the query in the lane's column, and dQ^T += K^T dS^T.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBKV = 128;  // keys per dK/dV workgroup (= block-sparse block)
constexpr int kBQ = 64;    // query rows per LDS tile in the dK/dV kernel
constexpr int kBR = 128;   // queries per dQ workgroup (= block-sparse block)
constexpr int kBC = 64;    // key rows per LDS tile in the dQ kernel

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

// ---------------------------------------------------------------------------
// D_i = sum_c dO_ic O_ic
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* o, const uint16_t* dO,
                                                      float* Dbuf, int64_t rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements (16 B) each
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / TPR;
  const int c = (int)(gid % TPR) * 8;
  float s = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + c);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s = fmaf(to_f32<T>(a[j] & 0xffffu), to_f32<T>(b[j] & 0xffffu), s);
      s = fmaf(to_f32<T>(a[j] >> 16), to_f32<T>(b[j] >> 16), s);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && c == 0) Dbuf[row] = s;
}

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dO;
  const float* lse;
  const float* Dbuf;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int H, N, BH, ntiles;
  float c;      // scale * log2(e)
  float scale;
  const int32_t* key_len;
  const uint8_t* block_mask;
  int nblk;
};

// lse (natural log) -> the base-2 shift used in exp2(c*s - shift); rows
// without keys (lse = -inf) get +inf so that their probabilities are 0.
__device__ __forceinline__ float lse_shift(float lse) {
  return lse == neg_inf() ? pos_inf() : lse * kLog2e;
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 128 keys
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int S = D + 8, KS = D / 32, DB = D / 16, CPR = D / 8;
  typedef typename Elt<T>::vec8 vec8;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kBQ * S];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[kBQ * S];
  __shared__ __attribute__((aligned(16))) float sLse[kBQ];
  __shared__ __attribute__((aligned(16))) float sD[kBQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  int rank, bh;
  map_workgroup(blockIdx.x, p.ntiles, p.BH, &rank, &bh);
  const int kt = rank;  // causal: the lowest key tiles see the most queries, so go first
  const int b = bh / p.H, N = p.N;
  const size_t base = (size_t)bh * N * D;
  const uint16_t* Q = p.q + base;
  const uint16_t* dO = p.dO + base;
  const float* lse = p.lse + (size_t)bh * N;
  const float* Dr = p.Dbuf + (size_t)bh * N;
  const int L = valid_keys(p.key_len, b, N);
  const int k0 = kt * kBKV, kw = k0 + wave * 32;

  // this wave's 32 keys and values as B operands (column = key)
  vec8 kf[2][KS], vf[2][KS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kw + kb * 16 + n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[kb][ks] = as_vec8<T>(ldg16(p.k + base + (size_t)key * D + ks * 32 + g * 8, key < N));
      vf[kb][ks] = as_vec8<T>(ldg16(p.v + base + (size_t)key * D + ks * 32 + g * 8, key < N));
    }
  }
  f32x4 dk[DB][2], dv[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      dk[db][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[db][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int nqt = (N + kBQ - 1) / kBQ;
  int qt_begin = 0;
  if (CAUSAL) qt_begin = k0 / kBQ;   // queries before k0 see none of these keys
  const bool any_key = k0 < L;       // all keys padded away -> zero gradients

  auto tile = [&](int q0) {
    __syncthreads();
#pragma unroll
    for (int c = tid; c < kBQ * CPR; c += 256) {
      const int r = c / CPR, col = (c % CPR) * 8, row = q0 + r;
      const bool ok = row < N;
      sts16(sQ + r * S + col, ldg16(Q + (size_t)row * D + col, ok));
      sts16(sdO + r * S + col, ldg16(dO + (size_t)row * D + col, ok));
    }
    if (tid < kBQ) {
      const int row = q0 + tid;
      sLse[tid] = row < N ? lse_shift(lse[row]) : pos_inf();
    } else if (tid < 2 * kBQ) {
      const int row = q0 + tid - kBQ;
      sD[tid - kBQ] = row < N ? Dr[row] : 0.f;
    }
    __syncthreads();
    if (kw >= L) return;                            // every key of this wave is padded
    if (CAUSAL && q0 + kBQ - 1 < kw) return;        // tile entirely before the keys

    f32x4 s[4][2], dp[4][2];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const vec8 aq = as_vec8<T>(lds16(sQ + (qb * 16 + n) * S + ks * 32 + g * 8));
        const vec8 ao = as_vec8<T>(lds16(sdO + (qb * 16 + n) * S + ks * 32 + g * 8));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[qb][kb] = Elt<T>::mfma(aq, kf[kb][ks], s[qb][kb]);
          dp[qb][kb] = Elt<T>::mfma(ao, vf[kb][ks], dp[qb][kb]);
        }
      }

    // P = exp2(c s - shift_row), dS = P (dP - D_row); rows = queries
    const bool need_mask = (kw + 32 > L) || (CAUSAL && q0 < kw + 31);
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const f32x4 sh = *reinterpret_cast<const f32x4*>(sLse + qb * 16 + g * 4);
      const f32x4 dd = *reinterpret_cast<const f32x4*>(sD + qb * 16 + g * 4);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float pv = fast_exp2(fmaf(s[qb][kb][i], p.c, -sh[i]));
          if (need_mask) {
            const int query = q0 + qb * 16 + g * 4 + i, key = kw + kb * 16 + n;
            if (key >= L || (CAUSAL && key > query)) pv = 0.f;
          }
          s[qb][kb][i] = pv;
          dp[qb][kb][i] = pv * (dp[qb][kb][i] - dd[i]);
        }
    }

    // dV^T += dO^T P, dK^T += Q^T dS  (k = 32 queries per MFMA).  For bf16
    // the probabilities and dS enter as a hi + lo pair of bf16 operands: a
    // single bf16 rounding of P (relative 2^-9) accumulated over a column
    // costs up to ~0.01 absolute in dV, on top of the output rounding.
    constexpr bool kSplit = kIsBf16<T>;
#pragma unroll
    for (int kq = 0; kq < kBQ / 32; ++kq) {
      const int r0 = (2 * kq) * 16 + g * 4 + (n >> 2), r1 = r0 + 16;
      vec8 pb[2], sb[2], pl[2], sl[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        pb[kb] = pack8<T>(s[2 * kq][kb], s[2 * kq + 1][kb]);
        sb[kb] = pack8<T>(dp[2 * kq][kb], dp[2 * kq + 1][kb]);
        if (kSplit) {
          pl[kb] = pack8<T>(residual16<T>(s[2 * kq][kb]), residual16<T>(s[2 * kq + 1][kb]));
          sl[kb] = pack8<T>(residual16<T>(dp[2 * kq][kb]), residual16<T>(dp[2 * kq + 1][kb]));
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = db * 16 + (n & 3) * 4;
        const vec8 ao = join8<T>(lds_tr4(sdO + r0 * S + col), lds_tr4(sdO + r1 * S + col));
        const vec8 aq = join8<T>(lds_tr4(sQ + r0 * S + col), lds_tr4(sQ + r1 * S + col));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          dv[db][kb] = Elt<T>::mfma(ao, pb[kb], dv[db][kb]);
          dk[db][kb] = Elt<T>::mfma(aq, sb[kb], dk[db][kb]);
          if (kSplit) {
            dv[db][kb] = Elt<T>::mfma(ao, pl[kb], dv[db][kb]);
            dk[db][kb] = Elt<T>::mfma(aq, sl[kb], dk[db][kb]);
          }
        }
      }
    }
  };

  if (any_key) {
    if (SPARSE) {
      const int jb = kt;  // 128 keys = one mask block column
      for (int ib = 0; ib < p.nblk; ++ib) {
        if (!p.block_mask[(size_t)ib * p.nblk + jb]) continue;
        for (int t = 2 * ib; t < 2 * ib + 2 && t < nqt; ++t) tile(t * kBQ);
      }
    } else {
      for (int t = qt_begin; t < nqt; ++t) tile(t * kBQ);
    }
  }

  // store dK = scale * dK^T^T, dV (lane: key column, 4 consecutive d)
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kw + kb * 16 + n;
    if (key < N) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const size_t off = base + (size_t)key * D + db * 16 + g * 4;
        *reinterpret_cast<u32x2*>(p.dk + off) = pack4<T>(dk[db][kb] * p.scale);
        *reinterpret_cast<u32x2*>(p.dv + off) = pack4<T>(dv[db][kb]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 128 queries
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dq_kernel(BwdParams p) {
  constexpr int S = D + 8, KS = D / 32, DB = D / 16, CPR = D / 8;
  typedef typename Elt<T>::vec8 vec8;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBC * S];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kBC * S];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  int rank, bh;
  map_workgroup(blockIdx.x, p.ntiles, p.BH, &rank, &bh);
  const int qt = CAUSAL ? p.ntiles - 1 - rank : rank;
  const int b = bh / p.H, N = p.N;
  const size_t base = (size_t)bh * N * D;
  const uint16_t* K = p.k + base;
  const uint16_t* V = p.v + base;
  const int L = valid_keys(p.key_len, b, N);
  const int q0 = qt * kBR, qw = q0 + wave * 32;

  vec8 qf[2][KS], of[2][KS];
  float sh[2], dd[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qw + qb * 16 + n;
    const bool ok = row < N;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[qb][ks] = as_vec8<T>(ldg16(p.q + base + (size_t)row * D + ks * 32 + g * 8, ok));
      of[qb][ks] = as_vec8<T>(ldg16(p.dO + base + (size_t)row * D + ks * 32 + g * 8, ok));
    }
    sh[qb] = ok ? lse_shift(p.lse[(size_t)bh * N + row]) : pos_inf();
    dd[qb] = ok ? p.Dbuf[(size_t)bh * N + row] : 0.f;
  }
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

  auto tile = [&](int kt0) {
    __syncthreads();
#pragma unroll
    for (int c = tid; c < kBC * CPR; c += 256) {
      const int r = c / CPR, col = (c % CPR) * 8, key = kt0 + r;
      const bool ok = key < N;
      sts16(sK + r * S + col, ldg16(K + (size_t)key * D + col, ok));
      sts16(sV + r * S + col, ldg16(V + (size_t)key * D + col, ok));
    }
    __syncthreads();
    if (qw >= N) return;
    if (CAUSAL && kt0 > qw + 31) return;

    f32x4 s[4][2], dp[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const vec8 ak = as_vec8<T>(lds16(sK + (kb * 16 + n) * S + ks * 32 + g * 8));
        const vec8 av = as_vec8<T>(lds16(sV + (kb * 16 + n) * S + ks * 32 + g * 8));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          s[kb][qb] = Elt<T>::mfma(ak, qf[qb][ks], s[kb][qb]);
          dp[kb][qb] = Elt<T>::mfma(av, of[qb][ks], dp[kb][qb]);
        }
      }
    const bool need_mask = (kt0 + kBC > L) || (CAUSAL && kt0 + kBC - 1 > qw);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float pv = fast_exp2(fmaf(s[kb][qb][i], p.c, -sh[qb]));
          if (need_mask) {
            const int key = kt0 + kb * 16 + g * 4 + i, query = qw + qb * 16 + n;
            if (key >= L || (CAUSAL && key > query)) pv = 0.f;
          }
          dp[kb][qb][i] = pv * (dp[kb][qb][i] - dd[qb]);
        }
    // dQ^T += K^T dS^T  (k = 32 keys per MFMA)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      vec8 sb[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) sb[qb] = pack8<T>(dp[2 * kk][qb], dp[2 * kk + 1][qb]);
      const int r0 = (2 * kk) * 16 + g * 4 + (n >> 2), r1 = r0 + 16;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = db * 16 + (n & 3) * 4;
        const vec8 a = join8<T>(lds_tr4(sK + r0 * S + col), lds_tr4(sK + r1 * S + col));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) acc[db][qb] = Elt<T>::mfma(a, sb[qb], acc[db][qb]);
      }
    }
  };

  if (SPARSE) {
    const uint8_t* mrow = p.block_mask + (size_t)qt * p.nblk;
    for (int jb = 0; jb < p.nblk; ++jb) {
      if (!mrow[jb]) continue;
      for (int t = 2 * jb; t < 2 * jb + 2 && t < nkt; ++t) tile(t * kBC);
    }
  } else {
    for (int t = 0; t < nkt; ++t) tile(t * kBC);
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int query = qw + qb * 16 + n;
    if (query < N) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<u32x2*>(p.dq + base + (size_t)query * D + db * 16 + g * 4) =
            pack4<T>(acc[db][qb] * p.scale);
    }
  }
}

template <typename T, int D, bool CAUSAL, bool SPARSE>
hipError_t run_bwd(const BwdArgs& a, int stage) {
  hipError_t e = hipSuccess;
  if (stage == 0 || stage == 1) {
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    const int64_t pre_threads = rows * (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((pre_threads + 255) / 256)),
                       dim3(256), 0, a.stream, static_cast<const uint16_t*>(a.o),
                       static_cast<const uint16_t*>(a.dO), a.Dbuf, rows);
    e = hipGetLastError();
    if (e != hipSuccess || stage == 1) return e;
  }

  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.dO = static_cast<const uint16_t*>(a.dO);
  p.lse = a.lse;
  p.Dbuf = a.Dbuf;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.H = a.H;
  p.N = a.N;
  p.BH = a.B * a.H;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  p.key_len = a.key_len;
  p.block_mask = a.block_mask;
  p.nblk = (a.N + 127) / 128;

  if (stage == 0 || stage == 2) {
    p.ntiles = (a.N + kBKV - 1) / kBKV;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, SPARSE>), dim3(p.ntiles * p.BH),
                       dim3(256), 0, a.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage == 0 || stage == 3) {
    p.ntiles = (a.N + kBR - 1) / kBR;
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, SPARSE>), dim3(p.ntiles * p.BH),
                       dim3(256), 0, a.stream, p);
    e = hipGetLastError();
  }
  return e;
}

template <typename T, int D>
hipError_t dispatch_mask(const BwdArgs& a, int stage) {
  if (a.block_mask) return run_bwd<T, D, false, true>(a, stage);
  return a.causal ? run_bwd<T, D, true, false>(a, stage) : run_bwd<T, D, false, false>(a, stage);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int stage) {
  if (a.dtype == 1)
    return a.d == 64 ? dispatch_mask<_Float16, 64>(a, stage) : dispatch_mask<_Float16, 128>(a, stage);
  return a.d == 64 ? dispatch_mask<__bf16, 64>(a, stage) : dispatch_mask<__bf16, 128>(a, stage);
}

}  // namespace fa
