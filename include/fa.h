/*
 * fa.h -- C ABI of the exact tiled attention library for MI355X (gfx950).
 *
 * The operation is exact scaled-dot-product attention computed tile by tile:
 * the forward pass keeps each block of scores on chip, folds it into the
 * output with the online running-maximum softmax, and saves only one
 * statistic per query row; the backward pass rebuilds every score block from
 * Q, K and that statistic instead of reading a stored N x N matrix
 * (dmarx anthology record SOTA-087, "Why recomputation is cheaper here than
 * storing" and "Condition"; Brenndoerfer, "FlashAttention Algorithm >
 * Recomputation Strategy", section "What Gets Stored vs Recomputed").
 *
 * Mathematics (per batch b, head h; L = valid length of sequence b):
 *   allowed(i,j) = i < L  and  j < L  and  (!causal or j <= i)
 *   S_ij   = scale * q_i . k_j  where allowed, -inf elsewhere
 *   lse_i  = ln sum_j exp(S_ij)           (natural log, scale included)
 *   P_ij   = exp(S_ij - lse_i),  o_i = sum_j P_ij v_j
 *   rows i >= L: o_i = 0, lse_i = -inf, and every gradient of row i is 0.
 * Backward of f = sum(o * dO):  dV = P^T dO;  dP = dO V^T;
 *   dS_ij = P_ij (dP_ij - D_i) with D_i = dO_i . o_i;
 *   dQ = scale * dS K;  dK = scale * dS^T Q.
 *
 * Layout: q, k, v, o, dO, dq, dk, dv are contiguous [B, H, N, d] arrays,
 * d fastest, of element type `dtype`, on the device, 16-byte aligned.
 * lse is a contiguous float32 [B, H, N] device array.  seqlens is NULL (every
 * sequence has length N) or a device int32 [B] array; each value is clamped
 * to [0, N] on the device.  Sizes: N <= 2^24, B*H <= 2^31 - 1 and
 * 2*B*H*ceil(N/128) <= 2^31 - 1 (the largest launch grid); larger sizes return
 * FA_ERR_INVALID_ARG.
 *
 * Ownership: the caller allocates and frees every buffer, including the
 * backward workspace; the library never allocates or frees device memory and
 * keeps no pointer after a call returns (kernels already queued on `stream`
 * still read and write the buffers until they finish).  The only mutable
 * global state is fa_bwd_noalloc's per-device scratch array and its address
 * table (guarded by a mutex); every other entry point is stateless, so calls
 * from several threads are safe.
 *
 * Ordering: every call only enqueues work on `stream` (a hipStream_t; NULL is
 * the default stream) and returns; the caller synchronises.
 *
 * Errors: every entry point returns an fa_status.  Invalid arguments are
 * reported before any HIP call and have no side effects.  FA_ERR_HIP means a
 * kernel launch failed; the HIP error state is cleared before returning.
 * Calls whose B, H or N is 0 do nothing and return FA_OK.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_BF16 = 0, /* bfloat16 inputs/outputs; MFMA bf16 x bf16 -> fp32 */
  FA_FP32 = 1  /* float32 inputs/outputs; MFMA fp32 -> fp32, P never rounded */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, negative or too large size, bad scale or dtype */
  FA_ERR_UNSUPPORTED = -2, /* head dimension other than 64, 96 or 128 */
  FA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than fa_bwd_workspace_bytes() */
  FA_ERR_HIP = -4,         /* a kernel launch failed */
  FA_ERR_SCRATCH = -5      /* fa_bwd_noalloc: row vectors exceed FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

/* Size of fa_bwd_noalloc's static device scratch array, per GPU. */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * Forward pass.  Writes o [B,H,N,d] (dtype) and lse [B,H,N] (float32).
 * The score matrix exists only tile by tile in registers; no N x N buffer is
 * ever formed (SOTA-087, "Why recomputation is cheaper here than storing").
 * scale must be finite and > 0.  d must be 64, 96 or 128 (the head
 * dimensions of 64-128 the pages discuss, in 32-wide matrix-core tiles).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal,
           const int32_t* seqlens, int dtype, void* stream);

/*
 * Bytes of device workspace fa_bwd needs: two float32 row vectors per head,
 * -D_i (D_i = dO_i . o_i) and lse_i * log2(e), each holding N rounded up to a
 * multiple of 128 rows per head (the padding rows are written too), each
 * rounded up to 256 bytes.  Linear in N.  Returns 0 for empty or invalid
 * shapes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype);

/*
 * Backward pass.  Reads q, k, v, o, dO and the forward's lse; writes dq, dk,
 * dv (dtype, [B,H,N,d]), fully overwriting them (0 at padded positions).
 * Recomputes every score block from Q, K and lse instead of reading a stored
 * probability matrix (Brenndoerfer, "What Gets Stored vs Recomputed").
 * `workspace` (device, 16-byte aligned, at least fa_bwd_workspace_bytes())
 * is scratch owned by the caller; its contents on entry are ignored.
 * Deterministic: every output is bitwise reproducible run to run.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
           const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal,
           const int32_t* seqlens, void* workspace, size_t workspace_bytes,
           int dtype, void* stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, outputs and results (bit for bit)
 * as fa_bwd; the row vectors live in a static device array of
 * FA_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs on holds
 * until the process ends.  Its address on the current device is looked up
 * with hipGetSymbolAddress on the first call on that device.  The call
 * allocates nothing (no hipMalloc/hipFree, no allocating library routine).
 * Limit: fa_bwd_workspace_bytes(B, H, N, d, dtype) must not exceed
 * FA_NOALLOC_SCRATCH_BYTES (B*H*ceil(N/128)*128 <= 2^21 rows), else
 * FA_ERR_SCRATCH is returned before any HIP call.  Nothing in the array needs
 * clearing: each call rewrites every row it reads.  Every call on a GPU shares
 * that GPU's array, so calls whose work overlaps on one GPU (several streams
 * or host threads without ordering between them) race: order them.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                   const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal,
                   const int32_t* seqlens, int dtype, void* stream);

/*
 * The stages of fa_bwd, exposed for callers that time them separately or
 * schedule them themselves.  fa_bwd is prepare followed by dkdv_dq; prepare
 * followed by dkdv and dq (in either order, or on two streams ordered after
 * prepare) computes the same, bit for bit.
 *   prepare: -D_i (D_i = dO_i . o_i) and lse_i in base 2 into the workspace (reads
 *            o, dO, lse).  A row of the softmax-Jacobian product reduces to
 *            dS_ij = P_ij (dP_ij - D_i) because sum_j P_ij dP_ij = dO_i . o_i.
 *   dkdv:    recomputes the score blocks key block by key block and writes
 *            dk and dv (reads q, k, v, dO, lse and the prepared workspace).
 *   dq:      recomputes the score blocks query block by query block and
 *            writes dq (same inputs).
 *   dkdv_dq: both of the above.  With a causal mask or seqlens, and with
 *            streamed operands (4*B*H*N*d elements) of at most 64 MiB, or at
 *            most 128 MiB when N <= 2048 or at bf16 d = 128, it is one
 *            launch that interleaves the two block lists heaviest first (a
 *            lone list's heaviest blocks outlast the average load of a
 *            resident workgroup); otherwise it is dkdv then dq on `stream`.
 *            Either way the gradients are bitwise the same.
 * Validation and errors are as for fa_bwd; each stage checks only the
 * pointers it uses (the others may be NULL).
 */
int fa_bwd_prepare(const void* o, const void* dO, const float* lse, int B, int H, int N,
                   int d, const int32_t* seqlens, void* workspace, size_t workspace_bytes,
                   int dtype, void* stream);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                const float* lse, void* dk, void* dv, int B, int H, int N, int d,
                float scale, int causal, const int32_t* seqlens, void* workspace,
                size_t workspace_bytes, int dtype, void* stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
              const float* lse, void* dq, int B, int H, int N, int d,
              float scale, int causal, const int32_t* seqlens, void* workspace,
              size_t workspace_bytes, int dtype, void* stream);
int fa_bwd_dkdv_dq(const void* q, const void* k, const void* v, const void* dO,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int N,
                   int d, float scale, int causal, const int32_t* seqlens, void* workspace,
                   size_t workspace_bytes, int dtype, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
