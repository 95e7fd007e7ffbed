"""Pins for the fp64 attention oracle, each independent of the oracle's own code.

What fixes each quantity:
  * P rows sum to 1, P >= 0, masked entries exactly 0   (softmax definition)
  * LSE = ln sum exp, recomputed in 50-digit mpmath arithmetic from the raw
    inputs (not from the oracle's scores)
  * closed forms: zero queries give uniform weights, so O is the mean of the
    allowed values (prefix means when causal) and LSE = ln(#allowed keys);
    a row with a single allowed key returns that key's value exactly
  * central finite differences of f = sum(O * dO) for every gradient
  * gradient invariants and metamorphic relations that follow from softmax
    shift invariance
  * an independent library routine (torch's CPU float64 scaled-dot-product
    attention with autograd)
The last test plants plausible mistakes in copies of the oracle and checks
that these pins catch each one.
"""
import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A

MASKS = [("none", False, None), ("causal", True, None), ("padded", False, 5), ("causal+padded", True, 5)]


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def small(N=8, d=4, seed=0, gain=1.0):
    return rnd((N, d), seed, gain), rnd((N, d), seed + 1, gain), rnd((N, d), seed + 2), rnd((N, d), seed + 3)


@pytest.mark.parametrize("name,causal,L", MASKS)
def test_rows_of_P_sum_to_one(name, causal, L):
    q, k, v, _ = small(N=12, d=5, seed=3, gain=2.0)
    O, lse, P = oracle.head_forward(q, k, v, 0.7, causal, L)
    N = q.shape[0]
    Lr = N if L is None else L
    mask = oracle.allowed_mask(N, Lr, causal)
    assert np.all(P >= 0)
    assert np.all(P[~mask] == 0.0)
    for i in range(N):
        if i < Lr:
            assert abs(P[i].sum() - 1.0) < 1e-12
        else:
            assert np.all(P[i] == 0) and np.all(O[i] == 0) and lse[i] == -np.inf


@pytest.mark.parametrize("name,causal,L", MASKS)
def test_lse_equals_log_sum_exp_mpmath(name, causal, L):
    q, k, v, _ = small(N=7, d=3, seed=11, gain=3.0)
    scale = 0.41
    _, lse, _ = oracle.head_forward(q, k, v, scale, causal, L)
    N = q.shape[0]
    Lr = N if L is None else L
    mpmath.mp.dps = 50
    for i in range(N):
        keys = [j for j in range(N) if i < Lr and j < Lr and (not causal or j <= i)]
        if not keys:
            assert lse[i] == -np.inf
            continue
        terms = []
        for j in keys:
            s = mpmath.mpf(0)
            for t in range(q.shape[1]):
                s += mpmath.mpf(float(q[i, t])) * mpmath.mpf(float(k[j, t]))
            terms.append(mpmath.exp(mpmath.mpf(scale) * s))
        ref = mpmath.log(mpmath.fsum(terms))
        assert abs(float(ref) - lse[i]) < 1e-13 * max(1.0, abs(float(ref)))


@pytest.mark.parametrize("name,causal,L", MASKS)
def test_zero_queries_give_uniform_means(name, causal, L):
    N, d = 9, 4
    v = rnd((N, d), 5)
    k = rnd((N, d), 6)
    q = np.zeros((N, d))
    O, lse, _ = oracle.head_forward(q, k, v, 0.5, causal, L)
    Lr = N if L is None else L
    for i in range(N):
        if i >= Lr:
            assert np.all(O[i] == 0) and lse[i] == -np.inf
            continue
        n = (i + 1) if causal else Lr
        n = min(n, Lr)
        assert np.allclose(O[i], v[:n].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[i] - math.log(n)) < 1e-14


def test_single_allowed_key_returns_that_value():
    q, k, v, do = small(N=6, d=4, seed=21, gain=2.0)
    scale = 0.3
    O, lse, _ = oracle.head_forward(q, k, v, scale, causal=True)
    assert np.array_equal(O[0], v[0])
    assert abs(lse[0] - scale * float(q[0] @ k[0])) < 1e-15
    # L = 1: only position 0 is valid
    r = oracle.head_backward(q, k, v, do, scale, causal=False, L=1)
    assert np.array_equal(r["o"][0], v[0])
    assert np.all(r["dq"] == 0) and np.all(r["dk"] == 0)
    assert np.allclose(r["dv"][0], do[0]) and np.all(r["dv"][1:] == 0)


def _f(q, k, v, do, scale, causal, L):
    O, _, _ = oracle.head_forward(q, k, v, scale, causal, L)
    return float((O * do).sum())


@pytest.mark.parametrize("name,causal,L", MASKS)
@pytest.mark.parametrize("jac", ["explicit", "factored"])
def test_gradients_match_central_differences(name, causal, L, jac):
    q, k, v, do = small(N=8, d=3, seed=7, gain=1.5)
    scale = 0.8
    r = oracle.head_backward(q, k, v, do, scale, causal, L, jacobian=jac)
    h = 1e-5
    for gname, X in (("dq", q), ("dk", k), ("dv", v)):
        G = r[gname]
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + h
            fp = _f(q, k, v, do, scale, causal, L)
            X[idx] = old - h
            fm = _f(q, k, v, do, scale, causal, L)
            X[idx] = old
            fd = (fp - fm) / (2 * h)
            assert abs(fd - G[idx]) <= 1e-7 * max(1.0, abs(fd)), (gname, idx, fd, G[idx])


@pytest.mark.parametrize("name,causal,L", MASKS)
def test_gradient_invariants(name, causal, L):
    q, k, v, do = small(N=10, d=6, seed=31, gain=2.0)
    r = oracle.head_backward(q, k, v, do, 0.6, causal, L)
    N = q.shape[0]
    Lr = N if L is None else L
    # rows of dS sum to zero  =>  sum_j dK_j = 0
    assert np.allclose(r["dk"].sum(axis=0), 0.0, atol=1e-12)
    # rows of P sum to one    =>  sum_j dV_j = sum over valid queries of dO_i
    assert np.allclose(r["dv"].sum(axis=0), do[:Lr].sum(axis=0), atol=1e-12)
    # both equal sum(dS * S)/1 up to the scale:  <dQ, Q> = <dK, K>
    assert abs((r["dq"] * q).sum() - (r["dk"] * k).sum()) < 1e-11
    # padded rows and keys carry no gradient
    assert np.all(r["dq"][Lr:] == 0) and np.all(r["dk"][Lr:] == 0) and np.all(r["dv"][Lr:] == 0)
    # D identity used by the recomputing backward: sum_j P_ij dP_ij = dO_i . O_i
    assert np.allclose(r["delta"], (do * r["o"]).sum(axis=1), atol=1e-12)


@pytest.mark.parametrize("name,causal,L", MASKS)
def test_metamorphic_shifts(name, causal, L):
    q, k, v, do = small(N=9, d=4, seed=41, gain=1.5)
    scale = 0.9
    base = oracle.head_backward(q, k, v, do, scale, causal, L)
    c = rnd((4,), 99)
    s = oracle.head_backward(q, k + c, v, do, scale, causal, L)   # every key shifted by the same vector
    Lr = q.shape[0] if L is None else L
    for n in ("o", "dq", "dk", "dv"):
        assert np.allclose(s[n], base[n], atol=1e-11), n
    assert np.allclose(s["lse"][:Lr], base["lse"][:Lr] + scale * (q[:Lr] @ c), atol=1e-11)
    t = oracle.head_backward(q, k, v + c, do, scale, causal, L)    # every value shifted
    assert np.allclose(t["o"][:Lr], base["o"][:Lr] + c, atol=1e-12)
    for n in ("dq", "dk", "dv"):
        assert np.allclose(t[n], base[n], atol=1e-11), n


def test_explicit_and_factored_jacobian_agree():
    q, k, v, do = small(N=64, d=16, seed=51, gain=2.0)
    for causal, L in ((False, None), (True, None), (False, 40), (True, 33)):
        a = oracle.head_backward(q, k, v, do, 0.25, causal, L, jacobian="explicit")
        b = oracle.head_backward(q, k, v, do, 0.25, causal, L, jacobian="factored")
        for n in ("dq", "dk", "dv"):
            assert np.allclose(a[n], b[n], atol=1e-13)


@pytest.mark.parametrize("name,causal,L", MASKS)
def test_independent_library_routine(name, causal, L):
    """torch CPU float64 scaled_dot_product_attention + autograd on valid rows."""
    N, d, scale = 24, 8, 0.35
    q, k, v, do = small(N=N, d=d, seed=61, gain=2.0)
    Lr = N if L is None else 17
    r = oracle.head_backward(q, k, v, do, scale, causal, Lr)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = torch.tensor(oracle.allowed_mask(N, Lr, causal)[:Lr])
    o = torch.nn.functional.scaled_dot_product_attention(tq[None, None, :Lr], tk[None, None], tv[None, None],
                                                         attn_mask=mask, scale=scale)[0, 0]
    (o * torch.tensor(do[:Lr])).sum().backward()
    assert np.allclose(o.detach().numpy(), r["o"][:Lr], atol=1e-12)
    assert np.allclose(tq.grad.numpy(), r["dq"], atol=1e-11)
    assert np.allclose(tk.grad.numpy(), r["dk"], atol=1e-11)
    assert np.allclose(tv.grad.numpy(), r["dv"], atol=1e-11)


def test_row_and_column_subsets_match_full_head():
    N, d = 200, 16
    q, k, v, do = small(N=N, d=d, seed=71, gain=2.0)
    for causal, L in ((True, None), (False, 150), (True, 121)):
        full = oracle.head_backward(q, k, v, do, 0.25, causal, L)
        rows = np.array([0, 1, 57, 120, 121, 150, 199])
        O, lse, dq = oracle.rows_forward_backward(q, k, v, do, 0.25, rows, causal, L)
        assert np.allclose(O, full["o"][rows], atol=1e-13)
        assert np.array_equal(np.isinf(lse), np.isinf(full["lse"][rows]))
        fin = np.isfinite(lse)
        assert np.allclose(lse[fin], full["lse"][rows][fin], atol=1e-13)
        assert np.allclose(dq, full["dq"][rows], atol=1e-13)
        cols = np.array([0, 3, 99, 149, 150, 199])
        dk, dv = oracle.key_columns_backward(q, k, v, do, 0.25, cols, causal, L, chunk=64)
        assert np.allclose(dk, full["dk"][cols], atol=1e-12)
        assert np.allclose(dv, full["dv"][cols], atol=1e-12)


def test_batched_wrappers_follow_seqlens():
    B, H, N, d = 2, 2, 12, 4
    x = [torch.tensor(rnd((B, H, N, d), s)) for s in range(4)]
    seq = np.array([12, 5])
    r = oracle.attention_backward(*x, scale=0.5, causal=True, seqlens=seq)
    for b in range(B):
        for h in range(H):
            one = oracle.head_backward(*(t[b, h].numpy() for t in x), 0.5, True, int(seq[b]))
            for n in ("o", "dq", "dk", "dv"):
                assert np.array_equal(r[n][b, h], one[n])


def _check_batched_forward(fwd, x, seq, causal, scale):
    """Every head of a batched forward against torch's CPU float64
    scaled_dot_product_attention (an independent library routine) with the
    per-sequence mask, and LSE against torch.logsumexp of the masked scores.
    Returns True if every head matches."""
    B, H, N, d = x[0].shape
    O, LSE = fwd(*x[:3], scale=scale, causal=causal, seqlens=seq)
    for b in range(B):
        L = int(seq[b])
        for h in range(H):
            if not (np.all(O[b, h, L:] == 0) and np.all(np.isneginf(LSE[b, h, L:]))):
                return False
            if L == 0:
                continue
            q, k, v = (t[b, h].double() for t in x[:3])
            mask = torch.tensor(oracle.allowed_mask(N, L, causal)[:L])
            o = torch.nn.functional.scaled_dot_product_attention(q[None, None, :L], k[None, None], v[None, None],
                                                                 attn_mask=mask, scale=scale)[0, 0]
            s = (q[:L] @ k.T * scale).masked_fill(~mask, float("-inf"))
            lse = torch.logsumexp(s, dim=1)
            if not (np.allclose(O[b, h, :L], o.numpy(), atol=1e-12, rtol=0)
                    and np.allclose(LSE[b, h, :L], lse.numpy(), atol=1e-12, rtol=0)):
                return False
    return True


@pytest.mark.parametrize("causal", [False, True])
def test_batched_forward_matches_library_routine_per_head(causal):
    """attention_forward over [B, H, N, d] with per-sequence lengths: each head
    uses its own sequence's length (B != H, lengths 12, 5, 1 and 0)."""
    B, H, N, d = 4, 3, 12, 4
    x = [torch.tensor(rnd((B, H, N, d), 10 + s, 1.5)) for s in range(3)]
    seq = np.array([12, 5, 1, 0])
    assert _check_batched_forward(oracle.attention_forward, x, seq, causal, 0.45)
    # the heads argument computes only the listed heads and leaves the rest NaN
    O, LSE = oracle.attention_forward(*x, scale=0.45, causal=causal, seqlens=seq, heads=[(1, 2)])
    full_o, full_lse = oracle.attention_forward(*x, scale=0.45, causal=causal, seqlens=seq)
    assert np.array_equal(O[1, 2], full_o[1, 2]) and np.array_equal(LSE[1, 2], full_lse[1, 2])
    assert np.isnan(O[0, 0]).all() and np.isnan(LSE[3, 1]).all()


def test_batched_forward_pin_catches_a_head_indexed_length():
    """A plausible slip in the batched wrapper, taking the length of sequence h
    instead of sequence b, fails the pin above."""
    def mutant(q, k, v, scale, causal=False, seqlens=None, heads=None):
        q, k, v = oracle.to_f64(q), oracle.to_f64(k), oracle.to_f64(v)
        B, H, N, d = q.shape
        O = np.full((B, H, N, d), np.nan)
        LSE = np.full((B, H, N), np.nan)
        for b in range(B):
            for h in range(H):
                L = int(min(max(int(seqlens[h]), 0), N))
                o, lse, _ = oracle.head_forward(q[b, h], k[b, h], v[b, h], scale, causal, L)
                O[b, h], LSE[b, h] = o, lse
        return O, LSE
    B, H, N, d = 4, 3, 12, 4
    x = [torch.tensor(rnd((B, H, N, d), 10 + s, 1.5)) for s in range(3)]
    seq = np.array([12, 5, 1, 0])
    for causal in (False, True):
        assert not _check_batched_forward(mutant, x, seq, causal, 0.45)


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle must be caught by a pin above.

def _mutant_backward(kind):
    def bwd(q, k, v, do, scale, causal=False, L=None, jacobian="auto"):
        N = q.shape[0]
        L = N if L is None else L
        Am = oracle.allowed_mask(N, L, causal)
        if kind == "causal_off_by_one":
            Am = Am & ~np.eye(N, dtype=bool) if causal else Am
        S = np.where(Am, scale * (q @ k.T), -np.inf)
        P, lse = A._softmax_rows(S, Am)
        dP = do @ v.T
        if kind == "dropped_outer_term":
            dS = np.where(Am, P * dP, 0.0)
        else:
            dS = A._softmax_vjp_factored(P, dP, Am)
        dq = scale * (dS @ k)
        dk = scale * (dS.T @ q)
        dv = P.T @ do
        if kind == "transposed_dk":
            dk = scale * (dS @ q)
        if kind == "missing_scale_dq":
            dq = dS @ k
        if kind == "transposed_dv":
            dv = P @ do
        return dict(o=P @ v, lse=lse, dq=dq, dk=dk, dv=dv)
    return bwd


@pytest.mark.parametrize("kind", ["dropped_outer_term", "transposed_dk", "missing_scale_dq", "transposed_dv",
                                  "causal_off_by_one"])
def test_pins_catch_planted_mistakes(kind):
    q, k, v, do = small(N=8, d=3, seed=7, gain=1.5)
    scale, causal = 0.8, True
    mut = _mutant_backward(kind)(q, k, v, do, scale, causal)
    ref_by_fd = {}
    h = 1e-5
    for gname, X in (("dq", q), ("dk", k), ("dv", v)):
        G = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + h
            fp = _f(q, k, v, do, scale, causal, None)
            X[idx] = old - h
            fm = _f(q, k, v, do, scale, causal, None)
            X[idx] = old
            G[idx] = (fp - fm) / (2 * h)
        ref_by_fd[gname] = G
    fd_ok = all(np.allclose(mut[g], ref_by_fd[g], atol=1e-7) for g in ref_by_fd)
    # the forward closed form: causal row 0 must return v_0 and row 1 must mix v_0, v_1
    closed_ok = np.array_equal(mut["o"][0], v[0]) if kind == "causal_off_by_one" else True
    assert not (fd_ok and closed_ok), f"mutant {kind} slipped through"
