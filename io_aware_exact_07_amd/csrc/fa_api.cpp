// C ABI of the attention library: argument validation, workspace layout and
// dispatch to the gfx950 kernels.  Declarations and the full contract are in
// include/fa.h.  Nothing here allocates device memory.
#include "fa.h"

#include <math.h>

#include <mutex>

#include "fa_launch.h"

namespace {

constexpr int kMaxN = 1 << 24;  // per-head row offsets stay within 32-bit arithmetic

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Common shape/scalar checks.  Returns FA_OK, an error, or 1 for "empty: nothing to do".
int check_common(int B, int H, int N, int d, float scale, int dtype) {
  if (dtype != FA_BF16 && dtype != FA_FP32) return FA_ERR_INVALID_ARG;
  if (B < 0 || H < 0 || N < 0 || N > kMaxN) return FA_ERR_INVALID_ARG;
  if (!(isfinite(scale) && scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 96 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  // The largest launch (the interleaved gradient lists) has 2 workgroups per
  // head and 128-row block; its grid must fit a 32-bit dimension.
  if (2LL * B * H * ((N + 127) / 128) > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  if (B == 0 || H == 0 || N == 0) return 1;
  return FA_OK;
}

bool tensor_ok(const void* p) { return p != nullptr && aligned(p, 16); }

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, const int32_t* seqlens, int dtype, void* stream) {
  int st = check_common(B, H, N, d, scale, dtype);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o)) return FA_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  if (seqlens != nullptr && !aligned(seqlens, 4)) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{q, k, v, o, lse, seqlens, B, H, N, scale};
  hipError_t e = fa::launch_fwd(a, d, dtype, causal != 0, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return FA_ERR_HIP;
  }
  return FA_OK;
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype) {
  int st = check_common(B, H, N, d, 1.0f, dtype);
  if (st != FA_OK) return 0;
  return 2 * round_up((size_t)B * H * fa::padded_rows(N) * sizeof(float), 256);
}

namespace {

enum Stage { kAll = 0, kPrepare = 1, kDkDv = 2, kDq = 3, kGrads = 4 };

// Validation of the backward entry points' shapes, scalars and tensor
// pointers (everything but the workspace).  Returns FA_OK, an error, or 1
// for "empty: nothing to do".
int bwd_check(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse, void* dq,
              void* dk, void* dv, int B, int H, int N, int d, float scale, const int32_t* seqlens, int dtype,
              int stage) {
  int st = check_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  const bool compute = stage == kAll || stage == kDkDv || stage == kDq || stage == kGrads;
  if (compute && (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v))) return FA_ERR_INVALID_ARG;
  if ((stage == kAll || stage == kPrepare) && (!tensor_ok(o) || lse == nullptr || !aligned(lse, 4)))
    return FA_ERR_INVALID_ARG;
  if (!tensor_ok(dO)) return FA_ERR_INVALID_ARG;
  if ((stage == kAll || stage == kDkDv || stage == kGrads) && (!tensor_ok(dk) || !tensor_ok(dv)))
    return FA_ERR_INVALID_ARG;
  if ((stage == kAll || stage == kDq || stage == kGrads) && !tensor_ok(dq)) return FA_ERR_INVALID_ARG;
  if (compute && (lse == nullptr || !aligned(lse, 4))) return FA_ERR_INVALID_ARG;
  if (seqlens != nullptr && !aligned(seqlens, 4)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// bwd_check plus the workspace; fills `a` on success.
int bwd_setup(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
              void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, const int32_t* seqlens,
              void* workspace, size_t workspace_bytes, int dtype, int stage, fa::BwdArgs* a) {
  int st = bwd_check(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, seqlens, dtype, stage);
  if (st != FA_OK) return st;
  const size_t need = fa_bwd_workspace_bytes(B, H, N, d, dtype);
  if (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < need) return FA_ERR_WORKSPACE;
  float* lse2 = static_cast<float*>(workspace);
  float* delta = reinterpret_cast<float*>(static_cast<char*>(workspace) + need / 2);
  *a = fa::BwdArgs{q, k, v, o, dO, lse, dq, dk, dv, lse2, delta, seqlens, B, H, N, scale};
  return FA_OK;
}

int run_stage(int stage, const fa::BwdArgs& a, int d, int dtype, int causal, void* stream) {
  hipError_t e = fa::launch_bwd_stage(stage, a, d, dtype, causal != 0, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// Both gradient stages.  Under a causal mask or per-sequence lengths the
// blocks of a lone dK/dV or dQ launch differ in work, and its heaviest blocks
// run on after the rest of the grid has drained; one launch that interleaves
// the two lists heaviest first evens the load out.  That pays for short
// sequences and small problems.  Otherwise the two lists run one after the
// other: with equal blocks there is nothing to even out, the single-list
// launches place each head's blocks on as few XCDs as possible (fewer L2
// misses), and once the operands the two lists stream (Q, dO and K, V of
// every head) outgrow the last-level cache together, each list's working set
// stays resident.  Measured: one launch is ahead at N <= 2048 and at 64 MiB
// or less, level from there to 128 MiB at N >= 4096, and behind beyond.  At
// bf16 d = 128 the dK/dV-only launch runs one wave per SIMD while the
// interleaved one runs two, so there one launch stays ahead up to 128 MiB.
int run_grads(const fa::BwdArgs& a, int d, int dtype, int causal, void* stream) {
  const double streamed = 4.0 * a.B * a.H * (double)a.N * d * (dtype == FA_BF16 ? 2 : 4);
  const bool uneven = causal || a.seqlens != nullptr;
  const bool small = streamed <= 64.0 * (1 << 20) ||
                     ((a.N <= 2048 || (dtype == FA_BF16 && d == 128)) && streamed <= 128.0 * (1 << 20));
  if (uneven && small) return run_stage(kGrads, a, d, dtype, causal, stream);
  const int st = run_stage(kDkDv, a, d, dtype, causal, stream);
  if (st != FA_OK) return st;
  return run_stage(kDq, a, d, dtype, causal, stream);
}

}  // namespace

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse, void* dq,
           void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, const int32_t* seqlens,
           void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  fa::BwdArgs a;
  int st = bwd_setup(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, seqlens, workspace, workspace_bytes, dtype,
                     kAll, &a);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  st = run_stage(kPrepare, a, d, dtype, causal, stream);
  if (st != FA_OK) return st;
  return run_grads(a, d, dtype, causal, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free backward: the workspace is a static device array.  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory, so the
// kernels only ever receive the address hipGetSymbolAddress returns for the
// current device, looked up once per device and kept here.
namespace {

constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array, or nullptr on a HIP error.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                   const int32_t* seqlens, int dtype, void* stream) {
  // Every argument is validated, and problems whose row vectors exceed the
  // array are rejected, before any HIP call.
  int st = bwd_check(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, seqlens, dtype, kAll);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  if (fa_bwd_workspace_bytes(B, H, N, d, dtype) > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = scratch_for_current_device();
  if (ws == nullptr) return FA_ERR_HIP;
  fa::BwdArgs a;
  st = bwd_setup(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, seqlens, ws, kScratchBytes, dtype, kAll, &a);
  if (st != FA_OK) return st;
  // The row vectors are fully rewritten by the prepare stage (padding rows
  // included), so nothing in the array needs clearing between calls.
  st = run_stage(kPrepare, a, d, dtype, causal, stream);
  if (st != FA_OK) return st;
  return run_grads(a, d, dtype, causal, stream);
}

int fa_bwd_prepare(const void* o, const void* dO, const float* lse, int B, int H, int N, int d,
                   const int32_t* seqlens, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  fa::BwdArgs a;
  int st = bwd_setup(nullptr, nullptr, nullptr, o, dO, lse, nullptr, nullptr, nullptr, B, H, N, d, 1.0f, seqlens,
                     workspace, workspace_bytes, dtype, kPrepare, &a);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  return run_stage(kPrepare, a, d, dtype, 0, stream);
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse, void* dk, void* dv,
                int B, int H, int N, int d, float scale, int causal, const int32_t* seqlens, void* workspace,
                size_t workspace_bytes, int dtype, void* stream) {
  fa::BwdArgs a;
  int st = bwd_setup(q, k, v, nullptr, dO, lse, nullptr, dk, dv, B, H, N, d, scale, seqlens, workspace,
                     workspace_bytes, dtype, kDkDv, &a);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  return run_stage(kDkDv, a, d, dtype, causal, stream);
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse, void* dq, int B, int H,
              int N, int d, float scale, int causal, const int32_t* seqlens, void* workspace, size_t workspace_bytes,
              int dtype, void* stream) {
  fa::BwdArgs a;
  int st = bwd_setup(q, k, v, nullptr, dO, lse, dq, nullptr, nullptr, B, H, N, d, scale, seqlens, workspace,
                     workspace_bytes, dtype, kDq, &a);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  return run_stage(kDq, a, d, dtype, causal, stream);
}

int fa_bwd_dkdv_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse, void* dq, void* dk,
                   void* dv, int B, int H, int N, int d, float scale, int causal, const int32_t* seqlens,
                   void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  fa::BwdArgs a;
  int st = bwd_setup(q, k, v, nullptr, dO, lse, dq, dk, dv, B, H, N, d, scale, seqlens, workspace, workspace_bytes,
                     dtype, kGrads, &a);
  if (st == 1) return FA_OK;
  if (st != FA_OK) return st;
  return run_grads(a, d, dtype, causal, stream);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (d must be 64, 96 or 128)";
    case FA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case FA_ERR_HIP: return "HIP kernel launch failed";
    case FA_ERR_SCRATCH:
      return "problem too large for the allocation-free entry point's static scratch (see FA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
