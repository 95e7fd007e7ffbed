"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases are compared element by element over every output.  Of the five
full-size workloads, the single-head, GPT-2-small, BERT-large and
long-context GPT-2 shapes are compared element by element on every head; the
very long N = 32768 shape on 256 query rows (O, lse, dQ) and 256 key rows
(dK, dV) of every head, plus properties that hold at any size.  The oracle
runs head by head on a thread pool.
"""
import dataclasses
import math
import os
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import TOL, f64, gpu_run, host_workers, lse_err, parallel_map, rel_err, valid_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def compare_heads(inp, got, causal, scale, heads, dtype, jacobian="auto", workers=1):
    """Every listed head of the GPU result against the oracle, element by
    element over the valid rows; padded rows must be exactly 0 / -inf."""
    sl = inp.get("seqlens")
    x = {n: inp[n] for n in ("q", "k", "v", "do")}
    N = inp["q"].shape[2]
    tol = TOL[dtype]

    def one(bh):
        b, h = bh
        L = valid_rows(sl, b, N)
        r = oracle.head_backward(*(oracle.to_f64(x[n][b, h]) for n in ("q", "k", "v", "do")), scale, causal, L,
                                 jacobian)
        errs = {}
        for name in ("o", "dq", "dk", "dv"):
            g = f64(got[name][b, h])
            errs[name] = rel_err(g[:L], r[name][:L]) if L > 0 else 0.0
            assert np.all(g[L:] == 0), f"{name} padded rows not zero (head {(b, h)})"
        errs["lse"] = lse_err(f64(got["lse"][b, h]), r["lse"])
        return errs

    worst = {}
    for (b, h), errs in zip(heads, parallel_map(one, heads, workers)):
        for name, e in errs.items():
            assert e <= tol[name], f"{name} head {(b, h)} err {e:.3e} > {tol[name]}"
            worst[name] = max(worst.get(name, 0.0), e)
    return worst


SMALL = [
    # (B, H, N, d, dtype, causal, seqlens)
    (1, 1, 1, 64, "bf16", False, None),
    (1, 2, 17, 64, "bf16", True, None),
    (2, 1, 100, 128, "bf16", False, None),
    (1, 2, 129, 64, "bf16", True, None),
    (2, 2, 300, 64, "bf16", True, None),
    (2, 2, 300, 128, "bf16", False, None),
    (3, 2, 257, 64, "bf16", False, [257, 1, 130]),
    (3, 1, 200, 128, "bf16", True, [0, 77, 200]),
    (2, 1, 190, 64, "fp32", True, None),
    (2, 1, 160, 128, "fp32", False, [99, 160]),
    (1, 1, 333, 128, "fp32", True, None),
    # head dimension 96 (the pages' d = 64..128 range in 32-wide tiles)
    (2, 2, 300, 96, "bf16", True, None),
    (2, 1, 257, 96, "bf16", False, [257, 130]),
    (1, 1, 200, 96, "fp32", True, None),
]


@pytest.mark.parametrize("B,H,N,d,dtype,causal,seqlens", SMALL)
def test_small_full_parity(B, H, N, d, dtype, causal, seqlens):
    say(f"small parity B={B} H={H} N={N} d={d} {dtype} causal={causal} seqlens={seqlens}")
    inp = W.random_inputs(B, H, N, d, dtype, seed=N + d, gain=1.5, seqlens=seqlens)
    scale = 1.0 / math.sqrt(d)
    got = gpu_run(inp, causal, scale)
    compare_heads(inp, got, causal, scale, [(b, h) for b in range(B) for h in range(H)], dtype)


def test_single_head_fp32_workload():
    w = W.SINGLE_HEAD_FP32
    say(f"workload {w.name}")
    inp = W.make_inputs(w)
    got = gpu_run(inp, w.causal, w.softmax_scale)
    compare_heads(inp, got, w.causal, w.softmax_scale, [(0, 0)], w.dtype)


@pytest.mark.parametrize("w", [W.GPT2_SMALL, W.BERT_LARGE_PADDED, W.GPT2_LONG], ids=lambda w: w.name)
def test_full_size_every_head(w):
    """Every head in full: O, lse, dQ, dK and dV element by element (the
    oracle's factored Jacobian, pinned equal to the explicit one)."""
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    say(f"workload {w.name}: all {len(heads)} heads")
    inp = W.make_inputs(w)
    t0 = time.time()
    got = gpu_run(inp, w.causal, w.softmax_scale)
    say(f"  gpu done {time.time() - t0:.1f}s")
    workers = host_workers(12 * w.N * w.N * 8)
    worst = compare_heads(inp, got, w.causal, w.softmax_scale, heads, w.dtype, jacobian="factored",
                          workers=workers)
    say(f"  oracle compare done {time.time() - t0:.1f}s ({workers} threads), worst {worst}")
    check_invariants(inp, got, w)


def check_invariants(inp, got, w):
    """Properties that hold over the full tensors at any size."""
    sl = inp.get("seqlens")
    B, H, N, d = inp["q"].shape
    dk = got["dk"].to(torch.float64)
    dv = got["dv"].to(torch.float64)
    do = inp["do"].to(torch.float64)
    for b in range(B):
        L = valid_rows(sl, b, N)
        # sum over keys of dK is 0; sum over keys of dV equals sum over valid queries of dO
        s_dk = dk[b, :, :L].sum(dim=1).abs().max().item()
        s_dv = (dv[b, :, :L].sum(dim=1) - do[b, :, :L].sum(dim=1)).abs().max().item()
        scale_dk = dk[b].abs().max().item() * math.sqrt(max(L, 1)) + 1e-30
        scale_dv = do[b].abs().max().item() * math.sqrt(max(L, 1)) + 1e-30
        assert s_dk <= 0.05 * scale_dk, f"sum dK = {s_dk} (batch {b})"
        assert s_dv <= 0.05 * scale_dv, f"sum dV - sum dO = {s_dv} (batch {b})"
        assert torch.all(got["o"][b, :, L:] == 0) and torch.all(got["dq"][b, :, L:] == 0)
        assert torch.all(torch.isneginf(got["lse"][b, :, L:]))
    if w.causal:
        # row 0 attends only key 0: its output is exactly v_0
        assert torch.equal(got["o"][:, :, 0], inp["v"][:, :, 0])


def sampled_rows_and_keys(w, inp, got, nrows, nkeys, key_heads):
    """nrows random query rows in every head (O, lse, dQ: each row is its own
    softmax, so the oracle's row mode is the full definition for it) and nkeys
    random key rows in each head of key_heads (dK, dV: the oracle streams every
    query past them).  Rows and keys are drawn per head from the workload seed."""
    tol = TOL[w.dtype]
    x = {n: inp[n][0] for n in ("q", "k", "v", "do")}

    def rows_job(h):
        rng = np.random.default_rng([w.seed, h])
        rows = np.sort(rng.choice(w.N, nrows, replace=False))
        q64, k64, v64, do64 = (oracle.to_f64(x[n][h]) for n in ("q", "k", "v", "do"))
        O, lse, dq = oracle.rows_forward_backward(q64, k64, v64, do64, w.softmax_scale, rows, w.causal)
        return dict(o=rel_err(f64(got["o"][0, h])[rows], O), dq=rel_err(f64(got["dq"][0, h])[rows], dq),
                    lse=lse_err(f64(got["lse"][0, h])[rows], lse))

    def keys_job(h):
        rng = np.random.default_rng([w.seed, 1000 + h])
        cols = np.sort(rng.choice(w.N, nkeys, replace=False))
        q64, k64, v64, do64 = (oracle.to_f64(x[n][h]) for n in ("q", "k", "v", "do"))
        dk, dv = oracle.key_columns_backward(q64, k64, v64, do64, w.softmax_scale, cols, w.causal)
        return dict(dk=rel_err(f64(got["dk"][0, h])[cols], dk), dv=rel_err(f64(got["dv"][0, h])[cols], dv))

    t0 = time.time()
    errs = parallel_map(rows_job, list(range(w.H)), host_workers(8 * nrows * w.N * 8))
    say(f"  query rows of {w.H} heads checked {time.time() - t0:.1f}s")
    kerrs = parallel_map(keys_job, list(key_heads), host_workers(10 * 512 * w.N * 8))
    say(f"  key rows of {len(key_heads)} heads checked {time.time() - t0:.1f}s")
    worst = {}
    for h, e in list(zip(range(w.H), errs)) + list(zip(key_heads, kerrs)):
        for name, v in e.items():
            assert v <= tol[name], f"{name} head {h} err {v:.3e} > {tol[name]}"
            worst[name] = max(worst.get(name, 0.0), v)
    say(f"  worst {worst}")


@pytest.mark.timeout(900)
def test_very_long_rows_and_keys_every_head():
    """N = 32768, d = 128, causal: 256 random query rows and 256 random key
    rows in every one of the 16 heads."""
    w = W.VERY_LONG
    say(f"workload {w.name}")
    inp = W.make_inputs(w)
    t0 = time.time()
    got = gpu_run(inp, w.causal, w.softmax_scale)
    say(f"  gpu done {time.time() - t0:.1f}s")
    sampled_rows_and_keys(w, inp, got, 256, 256, range(w.H))
    check_invariants(inp, got, w)


@pytest.mark.parametrize("d", [96, 128])
def test_long_context_other_head_dims_sampled(d):
    """The long-context GPT-2 head recipe at d = 96 and 128: 256 query rows of
    every head and 128 key rows of two heads."""
    w = dataclasses.replace(W.GPT2_LONG, d=d, name=f"GPT-2 head long context B=1 H=12 N=8192 d={d} causal, QK x2")
    say(f"workload {w.name}")
    inp = W.make_inputs(w)
    t0 = time.time()
    got = gpu_run(inp, w.causal, w.softmax_scale)
    say(f"  gpu done {time.time() - t0:.1f}s")
    sampled_rows_and_keys(w, inp, got, 256, 128, (0, w.H // 2))
    check_invariants(inp, got, w)


@pytest.mark.parametrize("d", [64, 96, 128])
def test_long_ragged_length_sampled(d):
    """A length far past the workloads and off every block size (N = 100003,
    prime), causal: 128 random query rows per head against the oracle, plus the
    dK/dV invariants and the exact first row."""
    N = 100003
    w = W.Workload(f"ragged long B=1 H=2 N={N} d={d} causal", 1, 2, N, d, "bf16", True, 7)
    say(f"workload {w.name}")
    inp = W.make_inputs(w)
    t0 = time.time()
    got = gpu_run(inp, True, w.softmax_scale)
    say(f"  gpu done {time.time() - t0:.1f}s")
    tol = TOL["bf16"]
    rng = np.random.default_rng(11)
    rows = np.sort(np.concatenate([rng.choice(N - 200, 120, replace=False), np.arange(N - 8, N)]))
    errs = dict(o=0.0, dq=0.0, lse=0.0)
    for h in range(w.H):
        q64, k64, v64, do64 = (f64(inp[n][0, h]) for n in ("q", "k", "v", "do"))
        O, lse, dq = oracle.rows_forward_backward(q64, k64, v64, do64, w.softmax_scale, rows, True)
        errs["o"] = max(errs["o"], rel_err(f64(got["o"][0, h])[rows], O))
        errs["dq"] = max(errs["dq"], rel_err(f64(got["dq"][0, h])[rows], dq))
        errs["lse"] = max(errs["lse"], lse_err(f64(got["lse"][0, h])[rows], lse))
    say(f"  rows checked {time.time() - t0:.1f}s errs {errs}")
    assert errs["o"] <= tol["o"] and errs["dq"] <= tol["dq"] and errs["lse"] <= tol["lse"], errs
    check_invariants(inp, got, w)


@pytest.mark.parametrize("causal", [False, True])
def test_many_small_heads_ragged_lengths(causal):
    """Many short heads with per-sequence lengths from 0 to N (large grids,
    blocks that are almost all padding, empty sequences): every head checked
    element by element against the oracle."""
    B, H, N, d = 37, 3, 77, 64
    rng = np.random.default_rng(5)
    seqlens = [int(x) for x in rng.integers(0, N + 1, B)]
    seqlens[0], seqlens[1], seqlens[2] = 0, N, 1
    say(f"many heads B={B} H={H} N={N} causal={causal} seqlens={seqlens[:6]}...")
    inp = W.random_inputs(B, H, N, d, "bf16", seed=77, gain=1.5, seqlens=seqlens)
    scale = 1.0 / math.sqrt(d)
    got = gpu_run(inp, causal, scale)
    heads = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, np.array(seqlens),
                                    heads=heads)
    tol = TOL["bf16"]
    for b, h in heads:
        L = seqlens[b]
        for name in ("o", "dq", "dk", "dv", "lse"):
            g = f64(got[name][b, h])
            if name == "lse":
                assert lse_err(g, ref["lse"][b, h]) <= tol["lse"]
                continue
            assert np.all(g[L:] == 0), f"{name} padded rows not zero (head {(b, h)})"
            if L == 0:
                continue
            r = ref[name][b, h][:L]
            err = np.max(np.abs(g[:L] - r))
            bound = tol[name] * np.max(np.abs(r))
            if name in ("dq", "dk"):
                # D_i = dO_i . o_i is formed from the stored bf16 o, so it
                # carries up to 2^-8 relative rounding per term (the bf16
                # unit roundoff); through
                # dS_ij = P_ij (dP_ij - D_i) that adds at most
                # scale * sum_j P_ij |dD_i| |k_j| to dQ (|q_i| to dK).  With
                # very few visible keys dP - D cancels and the exact gradient
                # is small, so this term is stated explicitly.
                q64, k64, do64 = (f64(inp[n][b, h][:L]) for n in ("q", "k", "do"))
                o64 = ref["o"][b, h][:L]
                dD = 2.0 ** -8 * np.sum(np.abs(do64) * np.abs(o64), axis=1)
                s = (q64 @ k64.T) * scale
                if causal:
                    s[np.triu_indices(L, 1)] = -np.inf
                P = np.exp(s - ref["lse"][b, h][:L, None])
                prop = scale * ((P * dD[:, None]) @ np.abs(k64) if name == "dq" else (P * dD[:, None]).T @ np.abs(q64))
                bound += np.max(prop)
            assert err <= bound, f"{name} head {(b, h)} L={L}: err {err:.3e} > {bound:.3e}"
