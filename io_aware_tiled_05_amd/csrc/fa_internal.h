// fa_internal.h — argument bundles passed from the validated C entry points
// (fa_api.cpp) to the kernel launchers (fa_fwd.hip, fa_bwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

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
  float* workspace;          // [2][B][H][N]: D_i = sum_c dO_ic O_ic, then lse_i * log2(e)
  int dtype;
  hipStream_t stream;
};

hipError_t launch_fwd(const FwdArgs& a);
// stage 0: all three launches; 1: D only; 2: dK/dV only; 3: dQ only
hipError_t launch_bwd(const BwdArgs& a, int stage);

}  // namespace fa
