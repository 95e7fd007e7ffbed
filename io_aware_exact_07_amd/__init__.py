"""Exact tiled attention for MI355X (gfx950): Python binding of libfa.so.

The binding only marshals arguments: every step of the forward and backward
pass runs in the HIP kernels behind the C ABI declared in include/fa.h.
PyTorch supplies device memory and the stream.  If the library has not been
built the import of the native part fails loudly; there is no fallback.

Raw entry points (same names and argument order as the C ABI, pointers as
ints): fa_fwd, fa_bwd, fa_bwd_prepare, fa_bwd_dkdv, fa_bwd_dq, fa_bwd_dkdv_dq,
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


def _check(ts, shape, dev, dt):
    for t in ts:
        if t.shape != shape or t.device != dev or t.dtype != dt or not t.is_contiguous():
            raise ValueError("q, k, v, o, do, dq, dk, dv must be contiguous [B,H,N,d] tensors of one dtype "
                             "on one device")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, dev):
    torch = _torch()
    s = torch.cuda.current_stream(dev) if stream is None else stream
    return s.cuda_stream


def _seqlens(seqlens, dev, B):
    torch = _torch()
    if seqlens is None:
        return None
    s = seqlens.to(device=dev, dtype=torch.int32).contiguous()
    if s.shape != (B,):
        raise ValueError("seqlens must have shape [B]")
    return s


def forward(q, k, v, causal=False, scale=None, seqlens=None, out=None, lse=None, stream=None):
    """o, lse = attention forward.  q, k, v: [B,H,N,d] bf16 or fp32 on the GPU."""
    torch = _torch()
    B, H, N, d = q.shape
    _check((q, k, v), q.shape, q.device, q.dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), device=q.device, dtype=torch.float32) if lse is None else lse
    _check((o,), q.shape, q.device, q.dtype)
    sl = _seqlens(seqlens, q.device, B)
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_t.data_ptr(), B, H, N, d, scale,
                causal, _ptr(sl), _dtype_code(q), _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd")
    return o, lse_t


def backward(q, k, v, o, do, lse, causal=False, scale=None, seqlens=None, workspace=None, grads=None,
             stream=None):
    """dq, dk, dv = attention backward, recomputing every score block."""
    torch = _torch()
    B, H, N, d = q.shape
    _check((q, k, v, o, do), q.shape, q.device, q.dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    need = fa_bwd_workspace_bytes(B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    _check((dq, dk, dv), q.shape, q.device, q.dtype)
    sl = _seqlens(seqlens, q.device, B)
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, scale, causal, _ptr(sl),
                workspace.data_ptr(), workspace.numel(), code, _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv
