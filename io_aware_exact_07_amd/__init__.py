"""Exact tiled attention for MI355X (gfx950): Python binding of libfa.so.

The binding only marshals arguments: every step of the forward and backward
pass runs in the HIP kernels behind the C ABI declared in include/fa.h.
PyTorch supplies device memory and the stream.  If the library has not been
built the import of the native part fails loudly; there is no fallback.

Raw entry points (same names and argument order as the C ABI, pointers as
ints): fa_fwd, fa_bwd, fa_bwd_noalloc, fa_bwd_prepare, fa_bwd_dkdv, fa_bwd_dq, fa_bwd_dkdv_dq,
fa_bwd_workspace_bytes, fa_status_string.
Tensor helpers: forward(q, k, v, ...) -> (o, lse) and
backward(q, k, v, o, do, lse, ...) -> (dq, dk, dv).
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_BF16 = 0
FA_FP32 = 1
FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_WORKSPACE = -3
FA_ERR_HIP = -4
FA_ERR_SCRATCH = -5
FA_NOALLOC_SCRATCH_BYTES = 16 << 20

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")
        self.status = status


def lib():
    """The loaded libfa.so (ctypes.CDLL).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -c \"import __graft_entry__ as g; "
                              f"g.build()\"` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, ci, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, vp, ci, vp]
        L.fa_fwd.restype = ci
        L.fa_bwd_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
        L.fa_bwd_workspace_bytes.restype = sz
        L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, vp, vp, sz, ci, vp]
        L.fa_bwd.restype = ci
        L.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, vp, ci, vp]
        L.fa_bwd_noalloc.restype = ci
        L.fa_bwd_prepare.argtypes = [vp, vp, vp, ci, ci, ci, ci, vp, vp, sz, ci, vp]
        L.fa_bwd_prepare.restype = ci
        L.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, vp, vp, sz, ci, vp]
        L.fa_bwd_dkdv.restype = ci
        L.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, vp, vp, sz, ci, vp]
        L.fa_bwd_dq.restype = ci
        L.fa_bwd_dkdv_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, vp, vp, sz, ci, vp]
        L.fa_bwd_dkdv_dq.restype = ci
        L.fa_status_string.argtypes = [ci]
        L.fa_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


# ---- raw C-ABI mirrors ------------------------------------------------------

def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, seqlens, dtype, stream) -> int:
    return lib().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, int(bool(causal)), seqlens, dtype, stream)


def fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, seqlens, workspace, workspace_bytes,
           dtype, stream) -> int:
    return lib().fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, int(bool(causal)), seqlens,
                        workspace, workspace_bytes, dtype, stream)


def fa_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, seqlens, dtype, stream) -> int:
    return lib().fa_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, int(bool(causal)), seqlens,
                                dtype, stream)


def fa_bwd_prepare(o, dO, lse, B, H, N, d, seqlens, workspace, workspace_bytes, dtype, stream) -> int:
    return lib().fa_bwd_prepare(o, dO, lse, B, H, N, d, seqlens, workspace, workspace_bytes, dtype, stream)


def fa_bwd_dkdv(q, k, v, dO, lse, dk, dv, B, H, N, d, scale, causal, seqlens, workspace, workspace_bytes,
                dtype, stream) -> int:
    return lib().fa_bwd_dkdv(q, k, v, dO, lse, dk, dv, B, H, N, d, scale, int(bool(causal)), seqlens,
                             workspace, workspace_bytes, dtype, stream)


def fa_bwd_dq(q, k, v, dO, lse, dq, B, H, N, d, scale, causal, seqlens, workspace, workspace_bytes, dtype,
              stream) -> int:
    return lib().fa_bwd_dq(q, k, v, dO, lse, dq, B, H, N, d, scale, int(bool(causal)), seqlens, workspace,
                           workspace_bytes, dtype, stream)


def fa_bwd_dkdv_dq(q, k, v, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, seqlens, workspace, workspace_bytes,
                   dtype, stream) -> int:
    return lib().fa_bwd_dkdv_dq(q, k, v, dO, lse, dq, dk, dv, B, H, N, d, scale, int(bool(causal)), seqlens,
                                workspace, workspace_bytes, dtype, stream)


def fa_bwd_workspace_bytes(B, H, N, d, dtype) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, H, N, d, dtype))


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(status).decode()


# ---- torch helpers ----------------------------------------------------------
#
# Every argument is checked here before any pointer reaches the library: a
# host, wrongly typed or short lse / workspace / gradient tensor would
# otherwise make the kernels read or write out of bounds.  The checks compare
# each tensor with q (shape, dtype, device, contiguity) and only at the end
# require q to live on a GPU, so each one is testable on a host without one.

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(ts, shape, dev, dt, what="q, k, v, o, do, dq, dk, dv"):
    for t in ts:
        if t.shape != shape or t.device != dev or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous [B,H,N,d] tensors of one dtype on one device")


def _check_lse(lse, q):
    torch = _torch()
    B, H, N, _ = q.shape
    if (lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.device != q.device
            or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 [B,H,N] = [{B},{H},{N}] tensor on {q.device}, "
                         f"got {tuple(lse.shape)} {lse.dtype} on {lse.device}")


def _check_workspace(ws, q, need):
    nbytes = ws.numel() * ws.element_size()
    if ws.device != q.device or not ws.is_contiguous() or nbytes < need:
        raise ValueError(f"workspace must be a contiguous tensor of at least {need} bytes on {q.device}, "
                         f"got {nbytes} bytes on {ws.device}")


def _on_gpu(q):
    if q.device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU (got {q.device}): the library takes device pointers")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream_ctx(stream):
    """Context that makes `stream` current, so that every tensor allocated
    for a call (outputs, workspace, the seqlens copy) belongs to the stream the
    kernels run on: the caching allocator then never hands that memory to
    other work before the kernels are done, and the seqlens copy is ordered
    before them."""
    torch = _torch()
    import contextlib
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _check_seqlens(seqlens, B):
    if seqlens is not None and tuple(seqlens.shape) != (B,):
        raise ValueError(f"seqlens must have shape [B] = [{B}], got {tuple(seqlens.shape)}")


def _seqlens(seqlens, dev):
    torch = _torch()
    if seqlens is None:
        return None
    return seqlens.to(device=dev, dtype=torch.int32).contiguous()


def forward(q, k, v, causal=False, scale=None, seqlens=None, out=None, lse=None, stream=None):
    """o, lse = attention forward.  q, k, v: [B,H,N,d] bf16 or fp32 on the GPU.

    With `stream` the outputs are allocated and the kernels run on that
    stream (the caller orders q, k, v before it)."""
    torch = _torch()
    B, H, N, d = q.shape
    _check((q, k, v), q.shape, q.device, q.dtype)
    if out is not None:
        _check((out,), q.shape, q.device, q.dtype, "out")
    if lse is not None:
        _check_lse(lse, q)
    _check_seqlens(seqlens, B)
    code = _dtype_code(q)
    _on_gpu(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with _stream_ctx(stream):
        o = torch.empty_like(q) if out is None else out
        lse_t = torch.empty((B, H, N), device=q.device, dtype=torch.float32) if lse is None else lse
        sl = _seqlens(seqlens, q.device)
        st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_t.data_ptr(), B, H, N, d, scale,
                    causal, _ptr(sl), code, torch.cuda.current_stream(q.device).cuda_stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd")
    return o, lse_t


def backward(q, k, v, o, do, lse, causal=False, scale=None, seqlens=None, workspace=None, grads=None,
             stream=None):
    """dq, dk, dv = attention backward, recomputing every score block.

    `workspace` (optional) is any contiguous tensor on q's device of at least
    fa_bwd_workspace_bytes() bytes.  With `stream` the gradients and the
    workspace are allocated and the kernels run on that stream."""
    torch = _torch()
    B, H, N, d = q.shape
    _check((q, k, v, o, do), q.shape, q.device, q.dtype)
    _check_lse(lse, q)
    code = _dtype_code(q)
    need = fa_bwd_workspace_bytes(B, H, N, d, code)
    if workspace is not None:
        _check_workspace(workspace, q, need)
    if grads is not None:
        if len(grads) != 3:
            raise ValueError("grads must be (dq, dk, dv)")
        _check(grads, q.shape, q.device, q.dtype, "dq, dk, dv")
    _check_seqlens(seqlens, B)
    _on_gpu(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with _stream_ctx(stream):
        if workspace is None:
            workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
        if grads is None:
            grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        dq, dk, dv = grads
        sl = _seqlens(seqlens, q.device)
        st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                    dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, scale, causal, _ptr(sl),
                    workspace.data_ptr(), workspace.numel() * workspace.element_size(), code,
                    torch.cuda.current_stream(q.device).cuda_stream)
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv
