// Internal launch interface between the C ABI (fa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* seqlens;
  int B, H, N;
  float scale;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;    // float32 [B,H,N] scratch: D_i = dO_i . o_i
  const int32_t* seqlens;
  int B, H, N;
  float scale;
};

// Return hipSuccess or the launch error.  dtype: 0 = bf16, 1 = fp32.
// The backward pass is three launches: stage 1 = D, stage 2 = dK and dV,
// stage 3 = dQ.  Stages 2 and 3 each need only stage 1's D.
hipError_t launch_fwd(const FwdArgs& a, int d, int dtype, bool causal, hipStream_t stream);
hipError_t launch_bwd_stage(int stage, const BwdArgs& a, int d, int dtype, bool causal, hipStream_t stream);

}  // namespace fa
