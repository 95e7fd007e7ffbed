"""torch.autograd binding of the attention path.

`attention(q, k, v, causal=False, scale=None, seqlens=None)` returns o and
records a node whose backward calls the recomputing backward pass; between
the two passes only q, k, v, o and the per-row lse are kept, never the N x N
probability matrix (Brenndoerfer, "FlashAttention Algorithm > Recomputation
Strategy", "What Gets Stored vs Recomputed").  Both directions run in the
HIP kernels through the C ABI; this module only marshals tensors.
"""
from __future__ import annotations

import torch

from . import backward as _backward
from . import forward as _forward


class Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale, seqlens):
        o, lse = _forward(q, k, v, causal=causal, scale=scale, seqlens=seqlens)
        ctx.save_for_backward(q, k, v, o, lse, seqlens if seqlens is not None else torch.empty(0))
        ctx.causal = causal
        ctx.scale = scale
        ctx.has_seqlens = seqlens is not None
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, dlse):
        q, k, v, o, lse, sl = ctx.saved_tensors
        dq, dk, dv = _backward(q, k, v, o, do.contiguous(), lse, causal=ctx.causal, scale=ctx.scale,
                               seqlens=sl if ctx.has_seqlens else None)
        return dq, dk, dv, None, None, None


def attention(q, k, v, causal=False, scale=None, seqlens=None):
    """o = softmax(scale * q k^T + mask) v for [B,H,N,d] bf16/fp32 GPU tensors."""
    o, _ = Attention.apply(q.contiguous(), k.contiguous(), v.contiguous(), causal, scale, seqlens)
    return o
