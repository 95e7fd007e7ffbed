"""Seeded synthetic inputs for the attention workloads.

This module only draws random tensors and describes shapes; it holds none of
the attention arithmetic.  Both the CPU oracle (through the tests) and the GPU
path (through the tests, the smoke check and the bench) take their inputs from
here, so the two sides always see bit-identical data.

The workloads stand in for the GPT-2 and BERT-large training runs that the
FlashAttention pages quote end-to-end numbers for (dmarx anthology record
SOTA-087, section "Why recomputation is cheaper here than storing"): only the
attention shapes are kept, filled with i.i.d. normal data.

Recipe (one reading, since the pages fix no generator):
  * torch.Generator('cpu').manual_seed(seed)
  * randn float32 [B,H,N,d] drawn in the order Q, K, V, dO
  * for the sharp-softmax long-context workload Q and K are multiplied by 2
    before any cast
  * for key-padded workloads, seqlens = randint(lo, hi+1, (B,)) drawn after dO
  * bf16 workloads are rounded once (round-to-nearest-even) from float32
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "bf16" or "fp32"
    causal: bool
    seed: int
    qk_gain: float = 1.0
    pad_range: Optional[tuple] = None   # (lo, hi) inclusive, per-sequence key lengths
    scale: Optional[float] = None       # default 1/sqrt(d)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def flops(self):
        """Counted FLOPs: 4*B*H*N^2*d forward, 2.5x that backward, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        if self.causal:
            f *= 0.5
        return f, 2.5 * f


# The five workloads.  Names say what they are.
SINGLE_HEAD_FP32 = Workload("single-head fp32 N=128 d=64", 1, 1, 128, 64, "fp32", False, 0,
                            scale=1.0 / math.sqrt(64))
GPT2_SMALL = Workload("GPT-2-small attention B=8 H=12 N=1024 d=64 causal", 8, 12, 1024, 64, "bf16", True, 1)
BERT_LARGE_PADDED = Workload("BERT-large attention B=16 H=16 N=512 d=64 key-padded", 16, 16, 512, 64, "bf16",
                             False, 2, pad_range=(128, 512))
GPT2_LONG = Workload("GPT-2 head long context B=1 H=12 N=8192 d=64 causal, QK x2", 1, 12, 8192, 64, "bf16", True,
                     3, qk_gain=2.0)
VERY_LONG = Workload("very long context B=1 H=16 N=32768 d=128 causal", 1, 16, 32768, 128, "bf16", True, 4)

ALL = [SINGLE_HEAD_FP32, GPT2_SMALL, BERT_LARGE_PADDED, GPT2_LONG, VERY_LONG]


def make_inputs(w: Workload, N: Optional[int] = None, B: Optional[int] = None, H: Optional[int] = None,
                seed: Optional[int] = None):
    """Return dict(q, k, v, do, seqlens) as CPU tensors in the workload dtype.

    N, B, H and seed may be overridden to draw a smaller instance of the same
    recipe (same distribution and masking structure).  seqlens is an int32
    tensor [B] or None.
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    seed = w.seed if seed is None else seed
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (B, H, N, w.d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    do = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.qk_gain != 1.0:
        q.mul_(w.qk_gain)
        k.mul_(w.qk_gain)
    seqlens = None
    if w.pad_range is not None:
        lo, hi = w.pad_range
        hi = min(hi, N)
        lo = min(lo, hi)
        seqlens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    dt = w.torch_dtype
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), do=do.to(dt), seqlens=seqlens)


def random_inputs(B, H, N, d, dtype="bf16", seed=0, gain=1.0, seqlens=None):
    """Free-form seeded inputs for edge-case tests (same recipe, any shape)."""
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (B, H, N, d)
    t = [torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(4)]
    t[0].mul_(gain)
    t[1].mul_(gain)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32)
    return dict(q=t[0].to(dt), k=t[1].to(dt), v=t[2].to(dt), do=t[3].to(dt), seqlens=sl)
