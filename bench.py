#!/usr/bin/env python3
"""Throughput of exact tiled attention (forward + recomputing backward) on one MI355X.

One step = one forward and one backward pass (fa_fwd, then fa_bwd's two
stages) over the long-context GPT-2 head workload: B=1, H=12, N=8192, d=64,
bf16, causal, Q and K scaled by 2 (inputs resident in HBM before timing).
FLOPs are counted as 4*B*H*N^2*d forward and 2.5x that backward, halved for
the causal mask.

Prints one JSON line.  Besides the whole-step rate it carries:
  roofline      the kernel with the longest average launch (the forward, or the
                gradient kernel that runs the dK/dV and dQ blocks in one
                launch) against the bf16 dense matrix-core peak: its
                algorithmic FLOPs (2*N^2*d per matrix product per head, halved
                when causal, times the products the method needs: 2 forward,
                5 backward -- S, dP, dV, dK, dQ) over its average duration,
                timed with HIP events on the stream the kernels run on, in
                the timed region, on every SAMPLE_EVERY-th step only (each
                event record costs the stream a few microseconds; recording
                them on every step would inflate the step time).  The
                gradient kernel executes 7 products (its dQ blocks recompute S
                and dP); that rate is reported beside it as
                `executed_tflops`, never as `achieved`.  `traffic` is the HBM
                bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE
                counters recorded under profiles/ when they were taken on the
                current kernel source, else null
  cpu_baseline  the fp64 CPU oracle timed on this host on whole heads of the
                same workload (about 10 s of work), in the same unit
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       (without --warmup: untimed steps for at least 1 s and 10 steps before timing)
                       [--workload gpt2_long|gpt2_small|bert_large|very_long|single_head]
                       [--head-dim 64|96|128] [--cold]
       (the same JSON line for another workload; `traffic` is reported only
        for the default one, whose counters are recorded)
       python bench.py --copy-probe        (plain 256 MiB copy, for counter calibration)
       python bench.py --memory-scaling    (JSON lines: peak memory of a 12-layer GPT-2-config
                                            causal attention stack, N = 512..32768, vs the
                                            recomputation page's model and explicit attention)
       python bench.py --compare-explicit  (JSON lines: fwd+bwd time vs explicit attention)
       python bench.py --sweep             (JSON lines: causal H=12 d=64, N = 1k..32k, B = 16384/N)
       python bench.py --calibrate         (JSON line from the fa_calib microbenchmarks: sustained
                                            matrix-core rate, exp/FMA rates, matrix/vector overlap,
                                            LDS and HBM bandwidth, float-atomic rate)
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s at 1 MI355X (bf16, d=64, N=1k–32k); % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X published dense bf16 matrix-core peak
PEAK_FP32_TFLOPS = 157.3   # MI355X published dense fp32 matrix-core peak
PEAK_HBM_GBS = 8000.0
# --workload choices -> workloads module attribute
WORKLOAD_KEYS = {"single_head": "SINGLE_HEAD_FP32", "gpt2_small": "GPT2_SMALL", "bert_large": "BERT_LARGE_PADDED",
                 "gpt2_long": "GPT2_LONG", "very_long": "VERY_LONG"}
KERNELS = {
    # name: (source file, matrix products per score element the method needs,
    #        matrix products per score element the kernel executes)
    "fwd_kernel": ("io_aware_exact_07_amd/csrc/fa_fwd.hip", 2, 2),
    # backward: S, dP, dV, dK, dQ; the dQ blocks recompute S and dP (4 + 3)
    "bwd_grad_kernel": ("io_aware_exact_07_amd/csrc/fa_bwd.hip", 5, 7),
}


# Steps of the timed region that also record per-stage events (fwd_ms,
# bwd_stage_ms and the roofline's launch duration): one in SAMPLE_EVERY.
SAMPLE_EVERY = 10
# Default warm-up: at least 10 steps and this much wall time, GPU-synchronised.
WARM_SECONDS = 1.0


def warm_up(step, warmup, sync) -> int:
    """Untimed steps before the timed region: exactly `warmup` if given, else
    at least 10 steps and WARM_SECONDS of GPU time, so that the GPU clocks reach
    the steady state a training loop runs at (after only 10 steps the
    GPT-2-small step read 17 % slower, the long-context step 4 %).  Returns the
    number of steps run."""
    if warmup is not None:
        for _ in range(warmup):
            step()
        sync()
        return warmup
    n, t0 = 0, time.time()
    while n < 10 or time.time() - t0 < WARM_SECONDS:
        for _ in range(10):
            step()
        n += 10
        sync()
    return n


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in (KERNELS[kernel][0], "io_aware_exact_07_amd/csrc/fa_common.h", "io_aware_exact_07_amd/csrc/fa_place.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_file(kernel: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_gpt2_long_traffic.txt")


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` on this workload, if the recorded
    counters were taken on the current kernel source."""
    path = traffic_file(kernel)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe():
    import torch
    n = 256 * 1024 * 1024
    x = torch.ones(n // 4, device="cuda:0", dtype=torch.float32)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 3}), flush=True)


def explicit_mask(B, N, causal, seqlens, device):
    """Boolean [B or 1, 1, N, N]: key j may be attended by query i (causal
    and per-sequence key padding; a padded query row has no allowed key)."""
    import torch
    allowed = torch.ones(N, N, dtype=torch.bool, device=device)
    if causal:
        allowed = allowed.tril()
    allowed = allowed[None, None]
    if seqlens is not None:
        valid = torch.arange(N, device=device)[None, :] < seqlens.to(device=device, dtype=torch.int64)[:, None]
        allowed = allowed & valid[:, None, :, None] & valid[:, None, None, :]
    return allowed


def explicit_attention_step(q, k, v, do, scale, allowed):
    """Standard attention that materialises the score and probability
    matrices (the baseline the recomputation pages compare against), forward
    and backward by hand in the input dtype.  `allowed` is explicit_mask();
    rows with no allowed key (padded queries) get P = 0, so their output and
    every gradient they feed are 0.  Every batched product gets contiguous
    operands.  Used only to measure memory and time beside the tiled path;
    returns (o, dq, dk, dv)."""
    import torch
    kt = k.transpose(-1, -2).contiguous()
    s = torch.matmul(q, kt).float() * scale
    s.masked_fill_(~allowed, float("-inf"))
    p = torch.nan_to_num(torch.softmax(s, dim=-1), nan=0.0).to(q.dtype)
    del s
    o = torch.matmul(p, v)
    pt = p.transpose(-1, -2).contiguous()
    dv = torch.matmul(pt, do)
    del pt
    vt = v.transpose(-1, -2).contiguous()
    dp = torch.matmul(do, vt).float()
    pf = p.float()
    ds = (pf * (dp - (pf * dp).sum(-1, keepdim=True))).to(q.dtype)
    del dp, pf
    dq = torch.matmul(ds, k) * scale
    dst = ds.transpose(-1, -2).contiguous()
    dk = torch.matmul(dst, q) * scale
    return o, dq, dk, dv


def memory_scaling(seq_lens=(512, 2048, 8192, 32768), layers=12, d_model=768, heads=12):
    """Peak device memory of a stack of causal attention layers (GPT-2 config),
    forward and backward through the autograd binding, against the recomputation
    page's training-memory model and (where it fits) explicit attention."""
    import torch
    from io_aware_exact_07_amd.autograd import attention
    from oracle.memory_model import training_memory
    dev = torch.device("cuda:0")
    d = d_model // heads
    for N in seq_lens:
        g = torch.Generator("cpu").manual_seed(N)
        qkv = [[torch.randn(1, heads, N, d, generator=g).to(dev, torch.bfloat16).requires_grad_() for _ in range(3)]
               for _ in range(layers)]
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        outs = [attention(q, k, v, causal=True) for q, k, v in qkv]
        torch.cuda.synchronize()
        stored = torch.cuda.memory_allocated() - base
        loss = sum(o.float().square().sum() for o in outs)
        loss.backward()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        inputs = sum(t.numel() * t.element_size() for l in qkv for t in l)
        model = training_memory(N, d_model=d_model, heads=heads, layers=layers, elem_bytes=2)
        rec = {"mode": "memory_scaling", "N": N, "layers": layers, "d_model": d_model, "heads": heads,
               "inputs_qkv_bytes": inputs, "stored_after_forward_bytes": stored,
               "stored_incl_qkv_bytes": stored + inputs,
               "model_recompute_bytes": round(model.recompute_gb * 1e9),
               "model_standard_bytes": round(model.standard_gb * 1e9),
               "peak_fwd_bwd_extra_bytes": peak}
        del outs, loss, qkv
        torch.cuda.empty_cache()
        # explicit attention for one layer, where its N x N matrices fit comfortably
        if model.attn_matrix_gb / layers < 40:
            q, k, v, do = (torch.randn(1, heads, N, d, generator=g).to(dev, torch.bfloat16) for _ in range(4))
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats()
            b0 = torch.cuda.memory_allocated()
            r = explicit_attention_step(q, k, v, do, 1.0 / d ** 0.5, explicit_mask(1, N, True, None, dev))
            torch.cuda.synchronize()
            rec["explicit_one_layer_peak_extra_bytes"] = torch.cuda.max_memory_allocated() - b0
            del r, q, k, v, do
            torch.cuda.empty_cache()
        else:
            rec["explicit_one_layer_peak_extra_bytes"] = None
        print(json.dumps(rec), flush=True)


def compare_explicit(steps=10):
    """fwd+bwd time of the tiled path vs explicit attention on the same inputs."""
    import torch
    import io_aware_exact_07_amd as fa
    import workloads as W
    dev = torch.device("cuda:0")
    for w in (W.GPT2_SMALL, W.BERT_LARGE_PADDED, W.GPT2_LONG):
        inp = W.make_inputs(w)
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
        sl = None if inp["seqlens"] is None else inp["seqlens"].to(dev)

        def ours():
            o, lse = fa.forward(q, k, v, causal=w.causal, seqlens=sl)
            fa.backward(q, k, v, o, do, lse, causal=w.causal, seqlens=sl)

        allowed = explicit_mask(w.B, w.N, w.causal, sl, dev)   # built once, outside the timed region

        def explicit():
            explicit_attention_step(q, k, v, do, w.softmax_scale, allowed)

        res = {"mode": "compare_explicit", "workload": w.name}
        for name, fn in (("tiled", ours), ("explicit", explicit)):
            warm_up(fn, None, torch.cuda.synchronize)  # both sides timed with settled clocks
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            res[name + "_ms"] = round(a.elapsed_time(b) / steps, 4)
        res["speedup"] = round(res["explicit_ms"] / res["tiled_ms"], 2)
        print(json.dumps(res), flush=True)
        del q, k, v, do
        torch.cuda.empty_cache()


def hbm_model_bytes(B, H, N, d, e, causal):
    """Per-launch HBM bytes of the forward and the gradient launch: the
    compulsory count (every input read once, every output written once) and
    the count of the tiled algorithm with 128-row blocks and no cache, as in
    the pages' Theorem 2 (each resident block streams every block of the other
    side that it needs; a causal mask halves the pairs).  The gradient launch
    streams Q, dO and the two row vectors past each key block (dK/dV list) and
    K, V past each query block (dQ list)."""
    heads = B * H
    nb = -(-N // 128)
    rereads = (nb * nb / 2 - nb) if causal else (nb * nb - nb)   # block pairs beyond the first read
    fwd_c = heads * (e * 4 * N * d + 4 * N)                       # q, k, v read, o written; lse
    grad_c = heads * (e * 4 * N * d + 8 * N + e * 3 * N * d)      # q, k, v, dO, lse2, D in; dk, dv, dq out
    fwd_t = fwd_c + heads * rereads * (2 * 128 * d * e)
    grad_t = grad_c + heads * rereads * (2 * 128 * d * e + 2 * 128 * 4 + 2 * 128 * d * e)
    return {"fwd_compulsory": int(fwd_c), "fwd_tiled_model": int(fwd_t),
            "grad_compulsory": int(grad_c), "grad_tiled_model": int(grad_t)}


def sweep(steps=20, warmup=None):
    """fwd+bwd rate over sequence lengths at a fixed token count: H=12, d=64,
    causal, N = 1k .. 32k, B = 16384 / N (B = 1 at N = 32k; one JSON line per N,
    with the compulsory and tiled-model HBM bytes per launch of both kernels)."""
    import torch
    import io_aware_exact_07_amd as fa
    import workloads as W
    dev = torch.device("cuda:0")
    for N in (1024, 2048, 4096, 8192, 16384, 32768):
        B = max(1, 16384 // N)  # N = 32k: one sequence
        w = W.Workload(f"causal sweep B={B} H=12 N={N} d=64", B, 12, N, 64, "bf16", True, 5)
        inp = W.make_inputs(w)
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))

        def step():
            o, lse = fa.forward(q, k, v, causal=True)
            fa.backward(q, k, v, o, do, lse, causal=True)

        n_warm = warm_up(step, warmup, torch.cuda.synchronize)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            step()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        f_fwd, f_bwd = w.flops()
        print(json.dumps({"mode": "sweep", "workload": w.name, "B": B, "N": N, "ms_per_step": round(ms, 5),
                          "tflops": round((f_fwd + f_bwd) / (ms * 1e-3) / 1e12, 3),
                          "pct_peak": round(100 * (f_fwd + f_bwd) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                          "launches_per_kernel": n_warm + steps,
                          "hbm_model_bytes": hbm_model_bytes(B, 12, N, 64, 2, True)}),
              flush=True)
        del q, k, v, do
        torch.cuda.empty_cache()


def cpu_baseline(w, min_seconds=10.0, max_full_n=8192):
    """The oracle as it stands, on this host's cores.  Up to N = max_full_n it
    runs whole heads of the workload (as many as fit in about min_seconds, at
    least one) through the full forward and backward.  Beyond that one head's
    score matrix alone is N^2 doubles (8.6 GB at N = 32768), so it runs the
    oracle's row mode instead: 256 random query rows of one head, each with
    its own softmax and Jacobian (O, lse and dQ for those rows), and the rate
    counts the work those rows do: 4 products of 2*n*d flops per row with n
    allowed keys."""
    import numpy as np
    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    inp = W.make_inputs(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    if w.N <= max_full_n:
        done = 0
        t0 = time.perf_counter()
        for bh in heads:
            oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], w.softmax_scale, w.causal, heads=[bh])
            done += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
        dt = time.perf_counter() - t0
        f_fwd, f_bwd = w.flops()
        flops = (f_fwd + f_bwd) * done / len(heads)
        sample = (f"{done} of {len(heads)} heads of the same workload, full forward + backward in float64 "
                  f"numpy; {dt:.2f} s for {flops / 1e9:.1f} counted GFLOP")
    else:
        rows = np.sort(np.random.default_rng(0).choice(w.N, 256, replace=False))
        b, h = heads[0]
        L = w.N if inp.get("seqlens") is None else int(inp["seqlens"][b])
        x = {n: oracle.to_f64(inp[n][b, h]) for n in ("q", "k", "v", "do")}
        t0 = time.perf_counter()
        oracle.rows_forward_backward(x["q"], x["k"], x["v"], x["do"], w.softmax_scale, rows, w.causal, L)
        dt = time.perf_counter() - t0
        keys = np.minimum(rows + 1, L) if w.causal else np.full(rows.shape, L)
        flops = float(np.sum(np.where(rows < L, keys, 0))) * 4 * 2 * w.d
        sample = (f"256 random query rows of one head (O, lse and dQ of those rows, float64 numpy row mode); "
                  f"{dt:.2f} s for {flops / 1e9:.2f} GFLOP of their products; a whole head would materialise "
                  f"{w.N}^2 scores")
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info() if i.get("user_api") == "blas"}))
    except Exception:
        blas = None
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas, "sample": sample}


def calibrate():
    """Run the fa_calib microbenchmarks (built beside libfa.so) as a child process."""
    import subprocess
    exe = os.path.join(ROOT, "io_aware_exact_07_amd", "fa_calib")
    if not os.path.exists(exe):
        raise SystemExit(f"{exe} is missing: build it with `python -c \"import __graft_entry__ as g; g.build()\"`")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    line = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""
    if r.returncode != 0 or not line.startswith("{"):
        raise SystemExit(f"fa_calib failed (exit {r.returncode}): {r.stdout}{r.stderr}")
    res = json.loads(line)
    res["mfma_frac_of_peak"] = round(res["mfma_bf16_tflops"] / PEAK_BF16_TFLOPS, 4)
    res["hbm_frac_of_peak"] = round(res["hbm_copy_tbs"] * 1000.0 / PEAK_HBM_GBS, 4)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 10 steps and 1 s, so the GPU clocks settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--memory-scaling", action="store_true",
                    help="peak memory of a 12-layer causal attention stack vs the page's model")
    ap.add_argument("--compare-explicit", action="store_true",
                    help="time the tiled path against explicit attention")
    ap.add_argument("--sweep", action="store_true",
                    help="JSON lines: causal H=12 d=64 at N = 1k..32k with B = 16384/N")
    ap.add_argument("--cold", action="store_true",
                    help="also time each step after writing a 512 MB buffer (L2 and the last-level cache "
                         "flushed, outside the timed region); reported under cold_cache")
    ap.add_argument("--calibrate", action="store_true",
                    help="run the calibration microbenchmarks (fa_calib) and print their JSON line")
    ap.add_argument("--workload", default="gpt2_long", choices=sorted(WORKLOAD_KEYS),
                    help="which synthetic workload a step runs (default: the long-context GPT-2 head)")
    ap.add_argument("--head-dim", type=int, default=None,
                    help="override the workload's head dimension (64, 96 or 128)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (asked for --gpus {args.gpus}); "
              f"heads shard across GPUs with no exchange, so per-GPU throughput is the N=1 figure.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.memory_scaling:
        memory_scaling()
        return
    if args.compare_explicit:
        compare_explicit()
        return
    if args.sweep:
        sweep(steps=min(args.steps, 20), warmup=None if args.warmup is None else min(args.warmup, 5))
        return
    if args.calibrate:
        calibrate()
        return

    import torch
    import io_aware_exact_07_amd as fa
    import workloads as W

    w = getattr(W, WORKLOAD_KEYS[args.workload])
    if args.head_dim is not None and args.head_dim != w.d:
        w = dataclasses.replace(w, d=args.head_dim, name=w.name.replace(f"d={w.d}", f"d={args.head_dim}"), scale=None)
    default_workload = args.workload == "gpt2_long" and w.d == W.GPT2_LONG.d
    dev = torch.device("cuda:0")
    inp = W.make_inputs(w)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    sl = None if inp["seqlens"] is None else inp["seqlens"].to(dev)
    slp = None if sl is None else sl.data_ptr()
    B, H, N, d = q.shape
    dt = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_FP32
    causal = 1 if w.causal else 0
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsb = fa.fa_bwd_workspace_bytes(B, H, N, d, dt)
    ws = torch.empty(wsb, device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    scale = w.softmax_scale
    P = [t.data_ptr() for t in (q, k, v, o, lse, dq, dk, dv, do, ws)]

    def step(ev=None):
        st = fa.fa_fwd(P[0], P[1], P[2], P[3], P[4], B, H, N, d, scale, causal, slp, dt, sp)
        if ev is not None:
            ev[0].record(stream)
        st |= fa.fa_bwd_prepare(P[3], P[8], P[4], B, H, N, d, slp, P[9], wsb, dt, sp)
        if ev is not None:
            ev[1].record(stream)
        st |= fa.fa_bwd_dkdv_dq(P[0], P[1], P[2], P[8], P[4], P[5], P[6], P[7], B, H, N, d, scale, causal, slp,
                                P[9], wsb, dt, sp)
        if ev is not None:
            ev[2].record(stream)
        if st != 0:
            raise RuntimeError(f"attention call failed: {st}")

    n_warm = warm_up(step, args.warmup, torch.cuda.synchronize)
    K = args.steps
    mk = lambda: torch.cuda.Event(enable_timing=True)
    # Per-stage events on every SAMPLE_EVERY-th timed step (at least one).
    sampled = list(range(0, K, SAMPLE_EVERY))
    starts = {i: mk() for i in sampled}
    marks = {i: [mk(), mk(), mk()] for i in sampled}
    t_begin, t_end = mk(), mk()
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(K):
        if i in starts:
            starts[i].record(stream)
            step(marks[i])
        else:
            step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_begin.elapsed_time(t_end)
    ms = total_ms / K
    avg = lambda f: sum(f(i) for i in sampled) / len(sampled)
    fwd_ms = avg(lambda i: starts[i].elapsed_time(marks[i][0]))
    prep_ms = avg(lambda i: marks[i][0].elapsed_time(marks[i][1]))
    grads_ms = avg(lambda i: marks[i][1].elapsed_time(marks[i][2]))
    bwd_ms = prep_ms + grads_ms

    cold = None
    if args.cold:
        # Each step starts with its inputs out of every cache: a 512 MB write
        # (twice the last-level cache) runs on the stream before the step's
        # first event, so it is not timed.
        flush = torch.empty(512 << 20, device=dev, dtype=torch.uint8)
        cs = [[mk(), mk(), mk(), mk()] for _ in range(K)]
        for i in range(K):
            flush.fill_(i & 0xFF)
            cs[i][0].record(stream)
            step(cs[i][1:])
        torch.cuda.synchronize()
        med = lambda xs: sorted(xs)[len(xs) // 2]
        cold = {"ms_per_step": round(med([c[0].elapsed_time(c[3]) for c in cs]), 5),
                "fwd_ms": round(med([c[0].elapsed_time(c[1]) for c in cs]), 5),
                "prepare_ms": round(med([c[1].elapsed_time(c[2]) for c in cs]), 5),
                "dkdv_dq_ms": round(med([c[2].elapsed_time(c[3]) for c in cs]), 5),
                "flush_bytes": 512 << 20, "statistic": "median of the timed steps"}
        del flush

    f_fwd, f_bwd = w.flops()
    value = (f_fwd + f_bwd) / (ms * 1e-3) / 1e12
    if cold is not None:
        cold["tflops"] = round((f_fwd + f_bwd) / (cold["ms_per_step"] * 1e-3) / 1e12, 3)
    per_product = f_fwd / 2.0
    launches = {"fwd_kernel": fwd_ms, "bwd_grad_kernel": grads_ms}
    dom = max(launches, key=launches.get)
    achieved = KERNELS[dom][1] * per_product / (launches[dom] * 1e-3) / 1e12
    executed = KERNELS[dom][2] * per_product / (launches[dom] * 1e-3) / 1e12
    e = 2 if w.dtype == "bf16" else 4
    compulsory = e * 4 * B * H * N * d + 4 * B * H * N                 # forward: q, k, v, o + lse
    compulsory += e * 2 * B * H * N * d + 4 * B * H * N                # prepare: o, dO -> D
    compulsory += e * 4 * B * H * N * d + 8 * B * H * N                # gradients: q, k, v, dO, lse2, D in
    compulsory += e * 3 * B * H * N * d                                # dk, dv, dq out
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    traffic = recorded_traffic(dom) if default_workload else None
    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": n_warm,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "key_padding": sl is not None, "fwd_gflop": f_fwd / 1e9, "bwd_gflop": f_bwd / 1e9},
        "fwd_ms": round(fwd_ms, 5),
        "bwd_ms": round(bwd_ms, 5),
        "bwd_stage_ms": {"prepare": round(prep_ms, 5), "dkdv_dq": round(grads_ms, 5)},
        "stage_timing": {"steps_with_events": len(sampled), "one_in": SAMPLE_EVERY},
        **({"cold_cache": cold} if cold is not None else {}),
        "effective_tflops": (round(value * float((sl.double() ** 2).sum()) / (B * N * N), 3) if sl is not None
                             else None),
        "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 3),
        "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 3),
        "pct_peak": round(100.0 * value / peak, 2),
        "compulsory_hbm_gbs": round(compulsory / (ms * 1e-3) / 1e9, 1),
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "algorithmic_gflop_per_launch": round(KERNELS[dom][1] * per_product / 1e9, 3),
            "executed_tflops": round(executed, 3),
            "executed_products_per_score": KERNELS[dom][2],
            "traffic": traffic,
            "traffic_gbs": None if traffic is None else round(traffic / (launches[dom] * 1e-3) / 1e9, 1),
            "avg_launch_ms": round(launches[dom], 5),
            "launches_timed": len(sampled),
        },
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
