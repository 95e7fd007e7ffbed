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
  float* lse2;     // float32 [B*H][Npad] scratch: lse_i * log2(e), +inf for rows >= L
  float* delta;    // float32 [B*H][Npad] scratch: -D_i = -(dO_i . o_i), 0 for rows >= L
  const int32_t* seqlens;
  int B, H, N;
  float scale;
};

// Return hipSuccess or the launch error.  dtype: 0 = bf16, 1 = fp32.
// Backward stages: 1 = the row vectors (D, lse in base 2), 2 = dK and dV,
// 3 = dQ, 4 = dK, dV and dQ in one launch.  Stages 2-4 need only stage 1.
hipError_t launch_fwd(const FwdArgs& a, int d, int dtype, bool causal, hipStream_t stream);

// Rows per head of the backward's row vectors: N rounded up to a whole
// number of 128-row blocks, so block-sized copies never run past a head.
__host__ __device__ inline int padded_rows(int N) { return (N + 127) / 128 * 128; }
hipError_t launch_bwd_stage(int stage, const BwdArgs& a, int d, int dtype, bool causal, hipStream_t stream);

}  // namespace fa
