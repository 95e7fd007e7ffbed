"""Shared helpers for the GPU parity tests: run the HIP path, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import io_aware_exact_07_amd as fa

# Tolerances: max|gpu - ref| / max|ref| over valid positions (LSE: max abs error).
TOL = {
    "bf16": dict(o=2e-2, dq=5e-2, dk=5e-2, dv=5e-2, lse=1e-3),
    "fp32": dict(o=1e-4, dq=1e-4, dk=1e-4, dv=1e-4, lse=1e-3),
}


def gpu_run(inp, causal, scale, backward=True, dev="cuda:0"):
    """Run fa_fwd (+ fa_bwd) on the GPU; returns CPU tensors."""
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    sl = inp.get("seqlens")
    sl = None if sl is None else sl.to(dev)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale, seqlens=sl)
    out = dict(o=o, lse=lse)
    if backward:
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=causal, scale=scale, seqlens=sl)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in out.items()}


def f64(t):
    return t.detach().to(torch.float64).numpy()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    num = np.max(np.abs(got - ref))
    return float(num / den) if den > 0 else float(num)


def lse_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), "LSE -inf pattern differs"
    return float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0


def valid_rows(seqlens, b, N):
    return N if seqlens is None else int(min(max(int(seqlens[b]), 0), N))


def host_workers(per_job_bytes, cap=16):
    """Thread count for oracle jobs: at most the host's CPUs (16 on a one-GPU
    box) and as many jobs as fit in half the free memory (64 GB at most)."""
    import os
    try:
        import psutil
        free = psutil.virtual_memory().available
    except Exception:
        free = 32 << 30
    budget = min(64 << 30, free // 2)
    n = min(cap, len(os.sched_getaffinity(0)), max(1, int(budget // max(per_job_bytes, 1))))
    return max(1, n)


def parallel_map(fn, jobs, workers):
    """[fn(j) for j in jobs] on a thread pool, BLAS held to one thread per call
    so the workers do not oversubscribe the cores (numpy's array kernels and
    BLAS release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, jobs))
