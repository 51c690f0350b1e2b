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
// Work split (16-bit path): 256 threads = 4 waves, 128 query rows per
// workgroup, 32 per wave (two 16-column MFMA blocks).  Key/value tiles are
// 64 rows.  Each wave computes the TRANSPOSED score tile S^T = K Q^T
// (keys x queries) with v_mfma_f32_16x16x32, so a lane holds 4 keys of one
// query column: the row maximum over keys is an in-register max plus two
// cross-lane steps, and the accumulator, rounded to 16 bits, is already laid
// out as the k-operand of the second contraction O^T += V^T P^T (V^T is read
// from the row-major V tile with the LDS transpose read).  Softmax runs in
// base 2 with scale*log2(e) folded into one FMA per score.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int H, N, BH, nqt;
  float c;  // scale * log2(e)
  const int32_t* key_len;
  const uint8_t* block_mask;
  int nblk;
};

constexpr int kBR = 128;  // query rows per workgroup (= block-sparse block)
constexpr int kBC = 64;   // key rows per LDS tile

__device__ __forceinline__ int valid_keys(const int32_t* key_len, int b, int N) {
  if (!key_len) return N;
  int kl = key_len[b];
  return kl < 0 ? 0 : (kl > N ? N : kl);
}

template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
  constexpr int S = D + 8;        // LDS row stride (elements): +16 B pad
  constexpr int KS = D / 32;      // k-steps of the S contraction
  constexpr int DB = D / 16;      // 16-row blocks of O^T
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  typedef typename Elt<T>::vec8 vec8;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBC * S];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kBC * S];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  int rank, bh;
  map_workgroup(blockIdx.x, p.nqt, p.BH, &rank, &bh);
  const int qt = CAUSAL ? p.nqt - 1 - rank : rank;  // longest rows first
  const int b = bh / p.H, N = p.N;
  const size_t base = (size_t)bh * N * D;
  const uint16_t* Q = p.q + base;
  const uint16_t* K = p.k + base;
  const uint16_t* V = p.v + base;
  const int L = valid_keys(p.key_len, b, N);
  const int q0 = qt * kBR, qw = q0 + wave * 32;

  // This wave's queries as B operands of S^T = K Q^T (kept in registers).
  vec8 qf[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qw + qb * 16 + n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[qb][ks] = as_vec8<T>(ldg16(Q + (size_t)row * D + ks * 32 + g * 8, row < N));
  }

  float m[2] = {neg_inf(), neg_inf()};  // running max of raw scores q.k
  float l[2] = {0.f, 0.f};              // running sum (this lane's keys)
  f32x4 acc[DB][2];                     // O^T, unnormalised
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
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int c = tid; c < kBC * CPR; c += 256) {
      const int r = c / CPR, col = (c % CPR) * 8, key = kt0 + r;
      const bool ok = key < N;
      sts16(sK + r * S + col, ldg16(K + (size_t)key * D + col, ok));
      sts16(sV + r * S + col, ldg16(V + (size_t)key * D + col, ok));
    }
    __syncthreads();
    if (qw >= N) return;                      // wave has no query rows
    if (CAUSAL && kt0 > qw + 31) return;      // tile fully above the diagonal

    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const vec8 a = as_vec8<T>(lds16(sK + (kb * 16 + n) * S + ks * 32 + g * 8));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[kb][qb] = Elt<T>::mfma(a, qf[qb][ks], s[kb][qb]);
      }

    // additive -inf mask, only on tiles that cross the diagonal or the end
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

    // online softmax update
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

    // O^T += V^T P^T, 32 keys per MFMA k-step
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      vec8 pk[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) pk[qb] = pack8<T>(s[2 * kk][qb], s[2 * kk + 1][qb]);
      const int r0 = (2 * kk) * 16 + g * 4 + (n >> 2), r1 = r0 + 16;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = db * 16 + (n & 3) * 4;
        const vec8 a = join8<T>(lds_tr4(sV + r0 * S + col), lds_tr4(sV + r1 * S + col));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) acc[db][qb] = Elt<T>::mfma(a, pk[qb], acc[db][qb]);
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

  // epilogue: O = O^T / l, lse = scale*m + ln(l)
  uint16_t* O = p.o + base;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = group_sum(l[qb]);
    const int query = qw + qb * 16 + n;
    if (query < N) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<u32x2*>(O + (size_t)query * D + db * 16 + g * 4) =
            pack4<T>(acc[db][qb] * inv);
      if (g == 0)
        p.lse[(size_t)bh * N + query] =
            lt > 0.f ? (m[qb] * p.c + fast_log2(lt)) * kLn2 : neg_inf();
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
  float c;
  const int32_t* key_len;
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
  map_workgroup(blockIdx.x, p.nqt, p.BH, &rank, &bh);
  const int qt = CAUSAL ? p.nqt - 1 - rank : rank;
  const int b = bh / p.H, N = p.N;
  const size_t base = (size_t)bh * N * D;
  const float* Q = p.q + base;
  const float* K = p.k + base;
  const float* V = p.v + base;
  const int L = valid_keys(p.key_len, b, N);
  const int q0 = qt * kBR, qw = q0 + wave * 32;

  float qf[2][D / 4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qw + qb * 16 + n;
#pragma unroll
    for (int ks = 0; ks < D / 4; ++ks)
      qf[qb][ks] = row < N ? Q[(size_t)row * D + ks * 4 + g] : 0.f;
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
      sK[r * S + col] = key < N ? K[(size_t)key * D + col] : 0.f;
      sV[r * S + col] = key < N ? V[(size_t)key * D + col] : 0.f;
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
  float* O = p.o + base;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = group_sum(l[qb]);
    const int query = qw + qb * 16 + n;
    if (query < N) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(O + (size_t)query * D + db * 16 + g * 4) = acc[db][qb] * inv;
      if (g == 0)
        p.lse[(size_t)bh * N + query] =
            lt > 0.f ? (m[qb] * p.c + fast_log2(lt)) * kLn2 : neg_inf();
    }
  }
}

template <typename T, int D, bool CAUSAL, bool SPARSE>
hipError_t run_fwd(const FwdArgs& a) {
  FwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
  p.lse = a.lse;
  p.H = a.H;
  p.N = a.N;
  p.BH = a.B * a.H;
  p.nqt = (a.N + kBR - 1) / kBR;
  p.c = a.scale * kLog2e;
  p.key_len = a.key_len;
  p.block_mask = a.block_mask;
  p.nblk = (a.N + 127) / 128;
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, SPARSE>), dim3(p.nqt * p.BH), dim3(256), 0,
                     a.stream, p);
  return hipGetLastError();
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
  p.c = a.scale * kLog2e;
  p.key_len = a.key_len;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(p.nqt * p.BH), dim3(256), 0, a.stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dispatch_mask(const FwdArgs& a) {
  if (a.block_mask) return run_fwd<T, D, false, true>(a);
  return a.causal ? run_fwd<T, D, true, false>(a) : run_fwd<T, D, false, false>(a);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.dtype == 0) {  // FA_F32
    if (a.d == 64) return a.causal ? run_fwd_f32<64, true>(a) : run_fwd_f32<64, false>(a);
    return a.causal ? run_fwd_f32<128, true>(a) : run_fwd_f32<128, false>(a);
  }
  if (a.dtype == 1) return a.d == 64 ? dispatch_mask<_Float16, 64>(a) : dispatch_mask<_Float16, 128>(a);
  return a.d == 64 ? dispatch_mask<__bf16, 64>(a) : dispatch_mask<__bf16, 128>(a);
}

}  // namespace fa
