"""The allocation-free backward (fa_bwd_noalloc) through the C ABI: on two
calls in a row, the second smaller than the first, it returns exactly what
fa_bwd returns with a caller-allocated workspace (both run the same kernels on
the same row vectors).  Between the calls the static array keeps the first
call's larger contents, which the second call must not depend on."""
import pytest
import torch

import io_aware_exact_07_amd as fa
import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = "cuda:0"


def run_both(B, H, N, d, dtype, causal, seqlens, seed):
    print(f"noalloc case B={B} H={H} N={N} d={d} {dtype} causal={causal} seqlens={seqlens}", flush=True)
    inp = W.random_inputs(B, H, N, d, dtype, seed=seed, gain=1.5, seqlens=seqlens)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    sl = None if inp["seqlens"] is None else inp["seqlens"].to(DEV)
    slp = None if sl is None else sl.data_ptr()
    code = fa.FA_BF16 if dtype == "bf16" else fa.FA_FP32
    scale = d ** -0.5
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale, seqlens=sl)
    sp = torch.cuda.current_stream().cuda_stream
    wsb = fa.fa_bwd_workspace_bytes(B, H, N, d, code)
    ws = torch.empty(wsb, device=DEV, dtype=torch.uint8)
    ref = [torch.full_like(q, 3.0) for _ in range(3)]
    got = [torch.full_like(q, 5.0) for _ in range(3)]
    p = lambda t: t.data_ptr()
    st = fa.fa_bwd(p(q), p(k), p(v), p(o), p(do), p(lse), *map(p, ref), B, H, N, d, scale, causal, slp, p(ws), wsb,
                   code, sp)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    st = fa.fa_bwd_noalloc(p(q), p(k), p(v), p(o), p(do), p(lse), *map(p, got), B, H, N, d, scale, causal, slp,
                           code, sp)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a, b), name


def test_noalloc_matches_fa_bwd_on_two_calls_the_second_smaller():
    run_both(2, 6, 1000, 64, "bf16", True, None, seed=1)
    run_both(3, 2, 257, 64, "bf16", False, [257, 40, 0], seed=2)


def test_noalloc_other_head_dims_and_fp32():
    run_both(1, 4, 700, 128, "bf16", True, None, seed=3)
    run_both(2, 2, 300, 96, "bf16", False, [300, 131], seed=4)
    run_both(1, 2, 190, 64, "fp32", True, None, seed=5)


def test_noalloc_at_the_size_limit():
    """B*H*Npad = 2^21 rows: exactly the static array (16 heads of N = 131072
    would be 4 GB of inputs; 512 heads of N = 4096 are 256 MB each)."""
    B, H, N, d = 8, 64, 4096, 64
    assert fa.fa_bwd_workspace_bytes(B, H, N, d, fa.FA_BF16) == fa.FA_NOALLOC_SCRATCH_BYTES
    run_both(B, H, N, d, "bf16", True, None, seed=6)
