// fa_internal.h — argument bundles passed from the validated C entry points
// (fa_api.cpp) to the kernel launchers (fa_fwd.hip, fa_bwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Dropout on the probabilities (off unless `on`): element (b, h, i, j) is
// kept iff 16-bit draw t(j) of Philox4x32-10(counter = (g(j), i, b H + h,
// offset), key = (k0, k1)) is >= thresh (< 2^16); kept values are
// multiplied by rinv.  g(j) = 2 (j div 16) + (j div 4) mod 2 and
// t(j) = 4 ((j div 8) mod 2) + j mod 4; draw t is the low (t even) or high
// half of output word t div 2.  A lane of the kernels holds, for one query,
// exactly the 8 keys of one call: keys 16 c + 4 h + {0..3, 8..11}.
__host__ __device__ inline int drop_call(int j) { return 2 * (j >> 4) + ((j >> 2) & 1); }
struct Dropout {
  int on = 0;
  uint32_t thresh = 0;
  float rinv = 1.f;
  // ceil(log2(rinv)): the 16-bit backward takes 2^-rexp into P, so that
  // P M rinv 2^-rexp <= 1 and dS keeps the same fp16 range bound as
  // without dropout (undone exactly in the gradients' fp32 epilogues)
  int rexp = 0;
  uint32_t k0 = 0, k1 = 0, offset = 0;
};

// Element strides of one [B][H][N][d] tensor view: element (b, h, i, c) is
// at b * b_ + h * h_ + i * n + c (the d index is contiguous).  Packed
// tensors have n = d, h_ = N d, b_ = H N d.
struct Strides {
  int64_t b, h, n;
};
inline Strides packed_strides(int64_t H, int64_t N, int64_t d) { return {H * N * d, N * d, d}; }

// Strides of every tensor an entry point touches (those it does not use are
// ignored).
struct Layout {
  Strides q, k, v, o, dO, dq, dk, dv;
};
inline Layout packed_layout(int64_t H, int64_t N, int64_t d) {
  const Strides s = packed_strides(H, N, d);
  return {s, s, s, s, s, s, s, s};
}

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  float scale;
  int causal;
  const int32_t* key_len;    // nullable
  const uint8_t* block_mask; // nullable; [nb][nb], block 128
  int dtype;                 // fa_dtype
  hipStream_t stream;
  Dropout drop = {};
  Layout lay = {};           // q, k, v, o
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  int B, H, N, d;
  float scale;
  int causal;
  const int32_t* key_len;
  const uint8_t* block_mask;
  void* workspace;           // bwd_workspace_layout(B, H, N, d).total bytes
  int dtype;
  hipStream_t stream;
  Dropout drop = {};
  Layout lay = {};           // every tensor; the workspace copies are packed
};

// Backward workspace, regions 256-byte aligned, in this order:
//   D      f32 [BHN]      D_i = sum_c dO_ic O_ic
//   shift  f32 [BHN]      lse_i * log2(e), +inf for rows without keys
//   nDs    f32 [BHN]      -D_i * 2^-(eo+ev)
//   nsh    f32 [BHN]      -shift_i * 2^-f
//   maxes  u32 [4][BH]    max |Q|, |K|, |V|, |dO| per (b, h), float bits
//   part   u32 [4][BH][kPreChunks]  the same per workgroup of the D pass
//   q16    f16 [BHN d]    c Q * 2^-eq    (c = scale * log2(e))
//   do16   f16 [BHN d]    dO * 2^-eo
//   k16    f16 [BHN d]    K * 2^-ek
// (BHN = B*H*N; eq, ek, ev, eo and f = eq + ek are the per-(b, h)
// power-of-two exponents that the kernels derive from the maxima.)
struct BwdWorkspace {
  size_t D, shift, nDs, nsh, maxes, part, q16, do16, k16, total;
};

// Most D-pass workgroups per (b, h): each leaves one partial maximum per
// tensor, which the convert pass reduces.
constexpr int kPreChunks = 128;

inline size_t ws_align(size_t x) { return (x + 255) & ~size_t(255); }

inline BwdWorkspace bwd_workspace_layout(int64_t B, int64_t H, int64_t N, int64_t d) {
  const size_t bhn = size_t(B * H * N), bh = size_t(B * H);
  BwdWorkspace w;
  w.D = 0;
  w.shift = ws_align(w.D + 4 * bhn);
  w.nDs = ws_align(w.shift + 4 * bhn);
  w.nsh = ws_align(w.nDs + 4 * bhn);
  w.maxes = ws_align(w.nsh + 4 * bhn);
  w.part = ws_align(w.maxes + 16 * bh);
  w.q16 = ws_align(w.part + 16 * bh * kPreChunks);
  w.do16 = ws_align(w.q16 + 2 * bhn * size_t(d));
  w.k16 = ws_align(w.do16 + 2 * bhn * size_t(d));
  w.total = ws_align(w.k16 + 2 * bhn * size_t(d));
  return w;
}

// The checks of fa_bwd's arguments (everything but the workspace; the
// strides when `lay` is given), made before any HIP call; FA_OK or the
// status to return.
int bwd_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dO, const void* dq, const void* dk, const void* dv, int B, int H,
              int N, int d, float scale, int causal, bool block_sparse, int dtype,
              bool dropout, const Layout* lay);

// Compute units of the current device (0 if the query fails); cached.
int device_cu_count();

// Dispatch-round length for map_workgroup's snake order: CUs per XCD when
// the heads are grouped by XCD (head count a multiple of 8), else all CUs.
inline int snake_period(int nheads) {
  const int n = device_cu_count();
  return (nheads & 7) == 0 ? n / 8 : n;
}

// Decode: Nq queries against Nk keys per (b, h), no causal order between
// them; keys j >= key_len[b] hidden.  The keys are split into chunks of
// `chunk` rows, one workgroup per (chunk, head, group of 4 queries); the
// workspace holds one partial (O slice, m, l) per (head, query, chunk).
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Nq, Nk, d;
  float scale;
  const int32_t* key_len;
  void* workspace;
  int dtype;
  hipStream_t stream;
};

struct DecodeSplit {
  int chunk, nchunks;
  size_t ws_bytes;
};

// Chunks of 1024 keys, halved (down to 256) while the launch would have
// fewer than 1024 workgroups.
inline DecodeSplit decode_split(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d) {
  const int64_t groups = B * H * ((Nq + 3) / 4);
  int64_t chunk = 1024;
  while (chunk > 256 && groups * ((Nk + chunk - 1) / chunk) < 1024) chunk /= 2;
  DecodeSplit s;
  s.chunk = (int)chunk;
  s.nchunks = (int)((Nk + chunk - 1) / chunk);
  s.ws_bytes = size_t(B * H * Nq) * size_t(s.nchunks) * size_t(d + 2) * sizeof(float);
  return s;
}

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_fwd(const FwdArgs& a);
// stage 0: the whole backward (16-bit: the D pass, then one launch that runs
// the dK/dV and dQ workgroups together); 1: D only; 2: dK/dV only; 3: dQ only;
// 4: dK/dV and dQ as stage 0 runs them (16-bit: the one launch)
hipError_t launch_bwd(const BwdArgs& a, int stage);
// fp32 inputs (dense, causal, key padding; no block mask); same stages
hipError_t launch_bwd_f32(const BwdArgs& a, int stage);

}  // namespace fa
