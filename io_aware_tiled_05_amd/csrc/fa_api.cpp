// fa_api.cpp — the extern "C" entry points declared in include/fa.h.
//
// Every argument is validated before any HIP call; a request that passes
// validation is forwarded to the kernel launchers, which only enqueue work
// on the caller's stream.
#include "fa.h"

#include <atomic>
#include <cmath>
#include <cstdint>

#include "fa_internal.h"

namespace {

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;

int check_sizes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID;
  const int64_t bh = int64_t(B) * H;
  if (bh > 65535LL * 65535LL) return FA_ERR_INVALID;
  if (bh * N * d > kMaxElems) return FA_ERR_INVALID;
  // grid size: one workgroup per 128 rows per head
  if (bh * ((int64_t(N) + 127) / 128) > kMaxElems) return FA_ERR_INVALID;
  if (d != 32 && d != 64 && d != 96 && d != 128) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_scale(float scale) {
  return (std::isfinite(scale) && scale > 0.f) ? FA_OK : FA_ERR_INVALID;
}

int check_dtype(int dtype) {
  return (dtype == FA_F32 || dtype == FA_F16 || dtype == FA_BF16) ? FA_OK : FA_ERR_INVALID;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Dropout with probability p in [0, 1): keep iff the element's Philox word
// is >= floor(p 2^32), scale kept values by 1 / (1 - p).  p = 0 is off.
int make_dropout(float p, uint64_t seed, uint32_t offset, fa::Dropout* out) {
  if (!std::isfinite(p) || p < 0.f || p >= 1.f) return FA_ERR_INVALID;
  fa::Dropout dr;
  dr.on = p > 0.f;
  const double t = std::floor((double)p * 65536.0);  // 16-bit draws
  dr.thresh = t >= 65535.0 ? 65535u : (uint32_t)t;
  dr.rinv = (float)(1.0 / (1.0 - (double)p));
  int e = 0;  // smallest e with 2^e >= rinv
  while (e < 30 && std::ldexp(1.0, e) < (double)dr.rinv) ++e;
  dr.rexp = e;
  dr.k0 = (uint32_t)(seed & 0xFFFFFFFFu);
  dr.k1 = (uint32_t)(seed >> 32);
  dr.offset = offset;
  *out = dr;
  return FA_OK;
}

// One tensor view's strides: non-negative; the row, head and batch strides
// keep every row's start 16-byte aligned (the kernels move rows in 16-byte
// chunks); row strides below 2^24 elements (tile offsets are 32-bit); an
// output's rows must not overlap (row stride >= d).
bool strides_ok(const fa::Strides& s, int d, int dtype, bool output) {
  const int64_t align = dtype == FA_F32 ? 4 : 8;  // elements per 16 bytes
  if (s.b < 0 || s.h < 0 || s.n < 1 || s.n >= (int64_t(1) << 24)) return false;
  if (s.b % align || s.h % align || s.n % align) return false;
  if (output && s.n < d) return false;
  return s.b < (int64_t(1) << 46) && s.h < (int64_t(1) << 46);
}

fa::Layout layout_of(const fa_layout* l, int H, int N, int d) {
  if (!l) return fa::packed_layout(H, N, d);
  auto cv = [](const fa_strides& s) { return fa::Strides{s.batch, s.head, s.row}; };
  return {cv(l->q), cv(l->k), cv(l->v), cv(l->o), cv(l->dO), cv(l->dq), cv(l->dk), cv(l->dv)};
}

int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int B,
               int H, int N, int d, float scale, int causal, const int32_t* key_len,
               const uint8_t* block_mask, int dtype, void* stream,
               const fa::Dropout& drop = fa::Dropout{}, const fa_layout* layout = nullptr) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  const fa::Layout lay = layout_of(layout, H, N, d);
  if (!strides_ok(lay.q, d, dtype, false) || !strides_ok(lay.k, d, dtype, false) ||
      !strides_ok(lay.v, d, dtype, false) || !strides_ok(lay.o, d, dtype, true))
    return FA_ERR_INVALID;
  int st = check_dtype(dtype);
  if (st == FA_OK) st = check_scale(scale);
  if (st == FA_OK) st = check_sizes(B, H, N, d);
  if (st != FA_OK) return st;
  if (block_mask && dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (drop.on && dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, causal, key_len, block_mask, dtype,
                static_cast<hipStream_t>(stream), drop, lay};
  return hip_status(fa::launch_fwd(a));
}

int bwd_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d,
               float scale, int causal, const int32_t* key_len, const uint8_t* block_mask,
               void* workspace, size_t workspace_bytes, int dtype, void* stream,
               int stage, const fa::Dropout& drop = fa::Dropout{},
               const fa_layout* layout = nullptr) {
  if (!workspace || !aligned16(workspace)) return FA_ERR_INVALID;
  const fa::Layout lay = layout_of(layout, H, N, d);
  const int st = fa::bwd_check(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal,
                               block_mask != nullptr, dtype, drop.on != 0, &lay);
  if (st != FA_OK) return st;
  if (workspace_bytes < fa_bwd_workspace_size(B, H, N, d)) return FA_ERR_INVALID;
  fa::BwdArgs a{q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, key_len,
                block_mask, workspace, dtype,
                static_cast<hipStream_t>(stream), drop, lay};
  return hip_status(fa::launch_bwd(a, stage));
}

// the mask arguments of the strided entry points: a block mask excludes
// causal, key lengths and dropout, and needs 128-row blocks
int mask_check(int causal, const int32_t* key_len, const uint8_t* block_mask, int block_size,
               float dropout_p) {
  if (!block_mask) return FA_OK;
  if (causal || key_len || dropout_p != 0.f) return FA_ERR_INVALID;
  if (block_size != 128) return block_size < 1 ? FA_ERR_INVALID : FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace

namespace fa {

int bwd_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dO, const void* dq, const void* dk, const void* dv, int B, int H,
              int N, int d, float scale, int causal, bool block_sparse, int dtype,
              bool dropout, const Layout* lay) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (lay && (!strides_ok(lay->q, d, dtype, false) || !strides_ok(lay->k, d, dtype, false) ||
              !strides_ok(lay->v, d, dtype, false) || !strides_ok(lay->o, d, dtype, false) ||
              !strides_ok(lay->dO, d, dtype, false) || !strides_ok(lay->dq, d, dtype, true) ||
              !strides_ok(lay->dk, d, dtype, true) || !strides_ok(lay->dv, d, dtype, true)))
    return FA_ERR_INVALID;
  int st = check_dtype(dtype);
  if (st == FA_OK) st = check_scale(scale);
  if (st == FA_OK) st = check_sizes(B, H, N, d);
  if (st != FA_OK) return st;
  if (dtype == FA_F32 && (block_sparse || dropout)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int device_cu_count() {
  // per device id; 0 = not queried yet.  Concurrent callers may both query
  // and store the same value; the atomics make that well defined.
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  if (dev < 64 && n > 0) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace fa

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int N, int d, float scale, int causal, const int32_t* key_len, int dtype,
           void* stream) {
  return fwd_common(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, nullptr, dtype,
                    stream);
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
  return fa::bwd_workspace_layout(B, H, N, d).total;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d,
           float scale, int causal, const int32_t* key_len, void* workspace,
           size_t workspace_bytes, int dtype, void* stream) {
  return bwd_common(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, key_len,
                    nullptr, workspace, workspace_bytes, dtype, stream, 0);
}

int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
                 int N, int d, float scale, int causal, const int32_t* key_len,
                 const uint8_t* block_mask, int block_size, void* workspace,
                 size_t workspace_bytes, int dtype, void* stream) {
  if (stage < FA_BWD_STAGE_D || stage > FA_BWD_STAGE_GRADS) return FA_ERR_INVALID;
  if (block_mask) {
    if (causal || key_len) return FA_ERR_INVALID;
    if (block_size != 128) return block_size < 1 ? FA_ERR_INVALID : FA_ERR_UNSUPPORTED;
  }
  return bwd_common(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, key_len,
                    block_mask, workspace, workspace_bytes, dtype, stream, stage);
}

int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, float scale, const uint8_t* block_mask,
                       int block_size, int dtype, void* stream) {
  if (!block_mask) return FA_ERR_INVALID;
  if (block_size != 128) return block_size < 1 ? FA_ERR_INVALID : FA_ERR_UNSUPPORTED;
  return fwd_common(q, k, v, o, lse, B, H, N, d, scale, 0, nullptr, block_mask, dtype,
                    stream);
}

int fa_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dO, void* dq, void* dk, void* dv, int B,
                       int H, int N, int d, float scale, const uint8_t* block_mask,
                       int block_size, void* workspace, size_t workspace_bytes, int dtype,
                       void* stream) {
  if (!block_mask) return FA_ERR_INVALID;
  if (block_size != 128) return block_size < 1 ? FA_ERR_INVALID : FA_ERR_UNSUPPORTED;
  return bwd_common(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, 0, nullptr,
                    block_mask, workspace, workspace_bytes, dtype, stream, 0);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int N, int d, float scale, int causal, const int32_t* key_len,
                   float dropout_p, uint64_t seed, uint32_t offset, int dtype, void* stream) {
  fa::Dropout dr;
  const int st = make_dropout(dropout_p, seed, offset, &dr);
  if (st != FA_OK) return st;
  return fwd_common(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, nullptr, dtype,
                    stream, dr);
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   float scale, int causal, const int32_t* key_len, float dropout_p,
                   uint64_t seed, uint32_t offset, void* workspace, size_t workspace_bytes,
                   int dtype, void* stream) {
  fa::Dropout dr;
  const int st = make_dropout(dropout_p, seed, offset, &dr);
  if (st != FA_OK) return st;
  return bwd_common(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, key_len,
                    nullptr, workspace, workspace_bytes, dtype, stream, 0, dr);
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int N, int d, float scale, int causal, const int32_t* key_len,
                   const uint8_t* block_mask, int block_size, float dropout_p, uint64_t seed,
                   uint32_t offset, const fa_layout* layout, int dtype, void* stream) {
  int st = mask_check(causal, key_len, block_mask, block_size, dropout_p);
  if (st != FA_OK) return st;
  fa::Dropout dr;
  st = make_dropout(dropout_p, seed, offset, &dr);
  if (st != FA_OK) return st;
  return fwd_common(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, block_mask, dtype,
                    stream, dr, layout);
}

int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   float scale, int causal, const int32_t* key_len, const uint8_t* block_mask,
                   int block_size, float dropout_p, uint64_t seed, uint32_t offset,
                   const fa_layout* layout, void* workspace, size_t workspace_bytes, int dtype,
                   void* stream) {
  int st = mask_check(causal, key_len, block_mask, block_size, dropout_p);
  if (st != FA_OK) return st;
  fa::Dropout dr;
  st = make_dropout(dropout_p, seed, offset, &dr);
  if (st != FA_OK) return st;
  return bwd_common(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, key_len,
                    block_mask, workspace, workspace_bytes, dtype, stream, 0, dr, layout);
}

size_t fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return 0;
  return fa::decode_split(B, H, Nq, Nk, d).ws_bytes;
}

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int Nq, int Nk, int d, float scale, const int32_t* key_len, void* workspace,
              size_t workspace_bytes, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(workspace))
    return FA_ERR_INVALID;
  int st = check_dtype(dtype);
  if (st == FA_OK) st = check_scale(scale);
  if (st == FA_OK) st = check_sizes(B, H, Nq, d);
  if (st == FA_OK) st = check_sizes(B, H, Nk, d);
  if (st != FA_OK) return st;
  if (workspace_bytes < fa_decode_workspace_size(B, H, Nq, Nk, d)) return FA_ERR_INVALID;
  fa::DecodeArgs a{q, k, v, o, lse, B, H, Nq, Nk, d, scale, key_len, workspace, dtype,
                   static_cast<hipStream_t>(stream)};
  return hip_status(fa::launch_decode(a));
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_HIP: return "HIP launch error";
    case FA_ERR_TOO_LARGE:
      return "problem too large for the library's fixed scratch buffer (fa_bwd_noalloc)";
    default: return "unknown status";
  }
}

}  // extern "C"
