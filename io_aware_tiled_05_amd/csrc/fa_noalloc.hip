// fa_noalloc.hip — fa_bwd_noalloc: the backward of fa_bwd with its workspace
// in a fixed device array of this library, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The array `scratch` is a file-scope __device__ variable: every GPU the
// library runs on holds its own copy, at its own address, from the time the
// code object is loaded until the process ends.  Host code never uses the
// array's name as an address (in host code it names a host-side stand-in);
// the device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and only that pointer is handed to the kernels.
// The backward's workspace needs no clearing (every region is written before
// it is read within one call), so nothing is cleared here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "fa_internal.h"

namespace {

constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size keeps the workspace regions aligned");

__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};

DeviceScratch g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call per device), or nullptr if the lookup failed.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  DeviceScratch& s = g_scratch[dev];
  std::call_once(s.once, [&s]() {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    s.ptr = s.err == hipSuccess ? p : nullptr;
  });
  return s.ptr;
}

}  // namespace

extern "C" {

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   float scale, int causal, const int32_t* key_len, int dtype, void* stream) {
  // fa_bwd's checks of the caller's arguments, then the scratch limit, all
  // before any HIP call
  const int st = fa::bwd_check(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal,
                               false, dtype, false, nullptr);
  if (st != FA_OK) return st;
  if (fa_bwd_workspace_size(B, H, N, d) > kScratchBytes) return FA_ERR_TOO_LARGE;
  void* ws = scratch_on_current_device();
  if (!ws) return FA_ERR_HIP;
  return fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, key_len, ws,
                kScratchBytes, dtype, stream);
}

}  // extern "C"
