"""GPU properties beyond parity: determinism, exact special cases, guard bands,
empty inputs and linear memory."""
import math

import pytest
import torch

import io_aware_exact_07_amd as fa
import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = "cuda:0"


def test_forward_and_backward_are_bitwise_deterministic():
    inp = W.random_inputs(2, 3, 700, 64, "bf16", seed=5, gain=2.0)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o1, l1 = fa.forward(q, k, v, causal=True)
    o2, l2 = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    do = inp["do"].to(DEV)
    g1 = fa.backward(q, k, v, o1, do, l1, causal=True)
    g2 = fa.backward(q, k, v, o1, do, l1, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):   # no atomics anywhere: every gradient is bitwise reproducible
        assert torch.equal(a, b)


def test_zero_queries_give_prefix_means():
    B, H, N, d = 1, 2, 300, 64
    inp = W.random_inputs(B, H, N, d, "fp32", seed=9)
    q = torch.zeros(B, H, N, d, device=DEV)
    k, v = inp["k"].to(DEV), inp["v"].to(DEV)
    o, lse = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    ref = torch.cumsum(inp["v"].double(), dim=2) / torch.arange(1, N + 1, dtype=torch.float64)[None, None, :, None]
    assert (o.cpu().double() - ref).abs().max().item() < 1e-5
    assert (lse.cpu().double() - torch.log(torch.arange(1, N + 1, dtype=torch.float64))).abs().max().item() < 1e-5


def test_outputs_leave_guard_bands_untouched():
    B, H, N, d = 2, 2, 190, 128
    inp = W.random_inputs(B, H, N, d, "bf16", seed=3, seqlens=[190, 55])
    n = B * H * N * d
    guard = 4096
    bufs = {}
    for name in ("o", "dq", "dk", "dv"):
        t = torch.full((n + 2 * guard,), 7.0, device=DEV, dtype=torch.bfloat16)
        bufs[name] = t
    lse_buf = torch.full((B * H * N + 2 * guard,), 7.0, device=DEV)
    view = lambda t: t[guard:guard + n].view(B, H, N, d)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    sl = inp["seqlens"].to(DEV)
    lse = lse_buf[guard:guard + B * H * N].view(B, H, N)
    o, _ = fa.forward(q, k, v, causal=False, seqlens=sl, out=view(bufs["o"]), lse=lse)
    fa.backward(q, k, v, o, do, lse, causal=False, seqlens=sl,
                grads=(view(bufs["dq"]), view(bufs["dk"]), view(bufs["dv"])))
    torch.cuda.synchronize()
    for name, t in list(bufs.items()) + [("lse", lse_buf)]:
        assert torch.all(t[:guard] == 7.0) and torch.all(t[-guard:] == 7.0), f"{name} guard band written"
    assert torch.all(view(bufs["o"])[1, :, 55:] == 0)


def test_empty_inputs_are_noops():
    x = torch.empty(0, 2, 128, 64, device=DEV, dtype=torch.bfloat16)
    o, lse = fa.forward(x, x, x)
    assert o.shape == x.shape
    y = torch.empty(1, 2, 0, 64, device=DEV, dtype=torch.bfloat16)
    o, lse = fa.forward(y, y, y)
    dq, dk, dv = fa.backward(y, y, y, o, y, lse)
    torch.cuda.synchronize()


def test_seqlens_clamped_on_device():
    inp = W.random_inputs(2, 1, 96, 64, "bf16", seed=12)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o_a, l_a = fa.forward(q, k, v, seqlens=torch.tensor([96, 0], dtype=torch.int32, device=DEV))
    o_b, l_b = fa.forward(q, k, v, seqlens=torch.tensor([1000, -5], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b)
    assert torch.all(o_a[1] == 0) and torch.all(torch.isneginf(l_a[1]))


def test_workspace_and_memory_are_linear_in_N():
    sizes = [1024, 2048, 4096, 8192]
    ws = [fa.fa_bwd_workspace_bytes(1, 12, n, 64, fa.FA_BF16) for n in sizes]
    assert all(b == 2 * a for a, b in zip(ws, ws[1:]))
    peaks = []
    for n in sizes:
        inp = W.random_inputs(1, 12, n, 64, "bf16", seed=1)
        q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        o, lse = fa.forward(q, k, v, causal=True)
        fa.backward(q, k, v, o, do, lse, causal=True)
        torch.cuda.synchronize()
        peaks.append(torch.cuda.max_memory_allocated() - base)
        del q, k, v, do, o, lse
    # every byte the path allocates (outputs + workspace) is linear in N: an
    # N x N fp32 buffer at N = 8192 would be 3.2 GB for 12 heads
    per_n = [p / n for p, n in zip(peaks, sizes)]
    assert max(per_n) <= 1.05 * min(per_n), peaks
    n = sizes[-1]
    expected = 4 * (12 * n * 64 * 2) + 12 * n * 4 + ws[-1]   # o, dq, dk, dv + lse + workspace
    assert peaks[-1] <= 1.05 * expected, (peaks[-1], expected)


@pytest.mark.parametrize("d", [64, 96, 128])
def test_separate_and_fused_gradient_stages_agree_bitwise(d):
    """fa_bwd (prepare, then one interleaved launch under the causal mask or with
    seqlens, two launches otherwise) equals prepare + dkdv + dq.  At d > 64 the
    dQ-only launch has its own register budget and tile grouping."""
    scale = 0.125
    for causal, seqlens in ((True, None), (False, [300, 77]), (False, None)):
        inp = W.random_inputs(2, 3, 300, d, "bf16", seed=21, gain=1.5, seqlens=seqlens)
        q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
        sl = None if inp["seqlens"] is None else inp["seqlens"].to(DEV)
        o, lse = fa.forward(q, k, v, causal=causal, scale=scale, seqlens=sl)
        ref = fa.backward(q, k, v, o, do, lse, causal=causal, scale=scale, seqlens=sl)
        B, H, N, d = q.shape
        wsb = fa.fa_bwd_workspace_bytes(B, H, N, d, fa.FA_BF16)
        ws = torch.empty(wsb, device=DEV, dtype=torch.uint8)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        sp = torch.cuda.current_stream().cuda_stream
        slp = None if sl is None else sl.data_ptr()
        assert fa.fa_bwd_prepare(o.data_ptr(), do.data_ptr(), lse.data_ptr(), B, H, N, d, slp, ws.data_ptr(), wsb,
                                 fa.FA_BF16, sp) == 0
        assert fa.fa_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                            B, H, N, d, scale, causal, slp, ws.data_ptr(), wsb, fa.FA_BF16, sp) == 0
        assert fa.fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), B, H, N, d, scale, causal, slp, ws.data_ptr(), wsb,
                              fa.FA_BF16, sp) == 0
        torch.cuda.synchronize()
        for a, b in zip(ref, (dq, dk, dv)):
            assert torch.equal(a, b)


def test_autograd_binding_matches_direct_calls_and_oracle():
    from io_aware_exact_07_amd.autograd import attention
    import oracle
    inp = W.random_inputs(1, 2, 150, 64, "bf16", seed=33, gain=1.5)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    qr, kr, vr = (t.clone().requires_grad_() for t in (q, k, v))
    o = attention(qr, kr, vr, causal=True)
    o.backward(do)
    o2, lse = fa.forward(q, k, v, causal=True)
    g = fa.backward(q, k, v, o2, do, lse, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for a, b in zip((qr.grad, kr.grad, vr.grad), g):
        assert torch.equal(a, b)
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], 0.125, causal=True)
    import numpy as np
    err = np.max(np.abs(qr.grad.float().cpu().numpy() - ref["dq"])) / np.max(np.abs(ref["dq"]))
    assert err < 5e-2


def test_stored_activations_equal_the_recomputation_page_model():
    """A 12-layer GPT-2-config causal stack through the autograd binding keeps
    exactly what the page's training-memory model counts for the recomputing
    method: Q, K, V, O per layer plus two 16-bit row statistics per (position,
    head) -- here one float32 lse (Brenndoerfer, code cell In[17] / Out[18])."""
    from io_aware_exact_07_amd.autograd import attention
    from oracle.memory_model import training_memory
    for N in (512, 2048):
        g = torch.Generator("cpu").manual_seed(N)
        qkv = [[torch.randn(1, 12, N, 64, generator=g).to(DEV, torch.bfloat16).requires_grad_() for _ in range(3)]
               for _ in range(12)]
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        outs = [attention(q, k, v, causal=True) for q, k, v in qkv]
        torch.cuda.synchronize()
        stored = torch.cuda.memory_allocated() - base
        inputs = sum(t.numel() * t.element_size() for l in qkv for t in l)
        model = training_memory(N, d_model=768, heads=12, layers=12, elem_bytes=2)
        assert stored + inputs == round(model.recompute_gb * 1e9)
        del outs, qkv


def test_side_stream_matches_default_stream_bitwise():
    """forward/backward with stream= run, allocate and copy seqlens on that
    stream; the results equal the default-stream run bit for bit."""
    inp = W.random_inputs(3, 2, 333, 64, "bf16", seed=44, gain=1.5, seqlens=[333, 100, 7])
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    sl = inp["seqlens"]                      # host tensor: the binding copies it on the call's stream
    ref_o, ref_l = fa.forward(q, k, v, causal=True, seqlens=sl)
    ref_g = fa.backward(q, k, v, ref_o, do, ref_l, causal=True, seqlens=sl)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, lse = fa.forward(q, k, v, causal=True, seqlens=sl, stream=side)
    g = fa.backward(q, k, v, o, do, lse, causal=True, seqlens=sl, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
    for a, b in zip(g, ref_g):
        assert torch.equal(a, b)


@pytest.mark.parametrize("causal,seqlens", [(True, None), (False, [200, 77, 1])])
def test_explicit_baseline_matches_the_oracle(causal, seqlens):
    """The explicit-attention baseline that bench.py --compare-explicit times
    (materialised P, hand-written backward, causal or key-padding mask)
    computes the same attention as the oracle within the bf16 tolerances, with
    zero outputs and gradients at padded positions."""
    import numpy as np
    import oracle
    from bench import explicit_attention_step, explicit_mask
    from parity_util import TOL, f64, lse_err, rel_err
    B = 2 if seqlens is None else len(seqlens)
    H, N, d = 2, 200, 64
    inp = W.random_inputs(B, H, N, d, "bf16", seed=8, gain=1.5, seqlens=seqlens)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    sl = None if inp["seqlens"] is None else inp["seqlens"].to(DEV)
    allowed = explicit_mask(B, N, causal, sl, DEV)
    got = [t.cpu() for t in explicit_attention_step(q, k, v, do, 0.125, allowed)]
    torch.cuda.synchronize()
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], 0.125, causal,
                                    None if seqlens is None else np.array(seqlens))
    tol = TOL["bf16"]
    for b in range(B):
        L = N if seqlens is None else seqlens[b]
        for h in range(H):
            for name, t in zip(("o", "dq", "dk", "dv"), got):
                g = f64(t[b, h])
                assert rel_err(g[:L], ref[name][b, h][:L]) <= tol[name], (name, b, h)
                assert np.all(g[L:] == 0), (name, b, h)


def test_bench_line_carries_consistent_contract_fields():
    """One short `bench.py` run on its default workload prints one JSON line
    whose rate, stage times and roofline agree with each other: value is the
    counted FLOPs over ms_per_step, achieved is the gradient launch's
    algorithmic FLOPs over its average duration, frac is achieved over the
    bf16 peak, and that duration fits inside a step."""
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print("bench.py --steps 5 --warmup 2 --no-cpu-baseline", flush=True)
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--steps", "5", "--warmup", "2",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=300, cwd=root)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 5 and rec["warmup"] == 2
    assert rec["unit"] == "TFLOP/s" and rec["higher_is_better"] is True and rec["dtype"] == "bf16"
    cfg = rec["config"]
    assert (cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"]) == (1, 12, 8192, 64, True)
    counted = cfg["fwd_gflop"] + cfg["bwd_gflop"]                      # GFLOP per step
    assert math.isclose(rec["value"], counted / rec["ms_per_step"], rel_tol=2e-3)
    rf = rec["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert rf["kernel"] == "bwd_grad_kernel"
    assert math.isclose(rf["algorithmic_gflop_per_launch"], cfg["bwd_gflop"], rel_tol=1e-6)
    assert math.isclose(rf["achieved"], rf["algorithmic_gflop_per_launch"] / rf["avg_launch_ms"], rel_tol=2e-3)
    assert math.isclose(rf["frac"], rf["achieved"] / rf["peak"], rel_tol=2e-3)
    assert 0 < rf["avg_launch_ms"] < rec["ms_per_step"] * 1.5
    assert rf["traffic"] is None or rf["traffic"] > 0
