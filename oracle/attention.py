"""Exact scaled-dot-product attention in float64 (TEST INFRASTRUCTURE ONLY).

This is the plain definition the tiled GPU method must reproduce: standard
attention, which materialises the full score and probability matrices
(dmarx anthology record SOTA-087, "Why recomputation is cheaper here than
storing"; Brenndoerfer, "FlashAttention Algorithm > Recomputation Strategy",
opening paragraphs and "Why Recomputation Makes Sense").  Nothing here is
blocked, fused or reordered: scores, probabilities and the softmax Jacobian
are formed explicitly, so each line can be checked against the definition by
eye.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may import this module.

Definitions used (the pages name them but print no formulas, so these are
the textbook ones):
  allowed(i, j) = (i < L) and (j < L) and (not causal or j <= i)
  S_ij  = scale * q_i . k_j            where allowed, -inf elsewhere
  LSE_i = ln sum_j exp(S_ij)           (natural log, includes scale)
  P_ij  = exp(S_ij - LSE_i)            (softmax of row i)
  O_i   = sum_j P_ij v_j
Rows i >= L (padded queries) have no allowed key: O_i = 0, LSE_i = -inf and
every gradient of that row is 0.

Backward of f = sum(O * dO) by the chain rule:
  dV_j  = sum_i P_ij dO_i
  dP_ij = dO_i . v_j
  dS_i  = J_i dP_i,  J_i = diag(P_i) - P_i P_i^T   (softmax Jacobian, allowed
                                                    columns of row i)
  dQ_i  = scale * sum_j dS_ij k_j
  dK_j  = scale * sum_i dS_ij q_i
For long rows J_i (n x n per row) is too large to form; there the same linear
map is applied as J_i x = P_i * x - P_i (P_i . x), which is an identity of the
matrix above, not a different algorithm.
"""
from __future__ import annotations

import numpy as np

EXPLICIT_JACOBIAN_MAX_N = 1024


def to_f64(t):
    """Exact float64 copy of a CPU tensor / array (bf16 values are exact in fp64)."""
    if hasattr(t, "detach"):
        import torch
        return t.detach().to(torch.float64).cpu().numpy()
    return np.asarray(t, dtype=np.float64)


def allowed_mask(N: int, L: int, causal: bool) -> np.ndarray:
    """Boolean [N, N]: key j may be attended by query i."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    a = (i < L) & (j < L)
    if causal:
        a = a & (j <= i)
    return a


def _scores(q, k, scale, A):
    S = scale * (q @ k.T)
    return np.where(A, S, -np.inf)


def _softmax_rows(S, A):
    """(P, LSE) for each row with at least one allowed entry; other rows: P=0, LSE=-inf."""
    has = A.any(axis=1)
    m = np.where(has, np.max(np.where(A, S, -np.inf), axis=1, initial=-np.inf), 0.0)
    E = np.where(A, np.exp(S - m[:, None]), 0.0)
    l = E.sum(axis=1)
    lse = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    P = np.where(A, np.exp(S - np.where(has, lse, 0.0)[:, None]), 0.0)
    return P, lse


def head_forward(q, k, v, scale, causal=False, L=None):
    """One head.  q, k, v float64 [N, d].  Returns (O [N, d], LSE [N], P [N, N])."""
    N = q.shape[0]
    L = N if L is None else int(min(max(L, 0), N))
    A = allowed_mask(N, L, causal)
    S = _scores(q, k, scale, A)
    P, lse = _softmax_rows(S, A)
    O = P @ v
    return O, lse, P


def _softmax_vjp_explicit(P, dP, A):
    """dS_i = J_i dP_i with J_i = diag(p) - p p^T formed over row i's allowed columns."""
    dS = np.zeros_like(P)
    for i in range(P.shape[0]):
        cols = np.nonzero(A[i])[0]
        if cols.size == 0:
            continue
        p = P[i, cols]
        J = np.diag(p) - np.outer(p, p)
        dS[i, cols] = J @ dP[i, cols]
    return dS


def _softmax_vjp_factored(P, dP, A):
    """Same linear map as the explicit Jacobian, applied without forming J_i."""
    dPm = np.where(A, dP, 0.0)
    inner = (P * dPm).sum(axis=1, keepdims=True)
    return np.where(A, P * dPm - P * inner, 0.0)


def head_backward(q, k, v, do, scale, causal=False, L=None, jacobian="auto"):
    """One head.  Returns dict(o, lse, dq, dk, dv, delta) in float64.

    delta_i = sum_j P_ij dP_ij, which equals dO_i . O_i (a diagnostic of the
    identity the tiled backward relies on).
    """
    N = q.shape[0]
    L = N if L is None else int(min(max(L, 0), N))
    A = allowed_mask(N, L, causal)
    O, lse, P = head_forward(q, k, v, scale, causal, L)
    dv = P.T @ do
    dP = do @ v.T
    if jacobian == "auto":
        jacobian = "explicit" if N <= EXPLICIT_JACOBIAN_MAX_N else "factored"
    if jacobian == "explicit":
        dS = _softmax_vjp_explicit(P, dP, A)
    else:
        dS = _softmax_vjp_factored(P, dP, A)
    dq = scale * (dS @ k)
    dk = scale * (dS.T @ q)
    delta = (P * np.where(A, dP, 0.0)).sum(axis=1)
    return dict(o=O, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)


def _seqlen(seqlens, b, N):
    if seqlens is None:
        return N
    return int(min(max(int(seqlens[b]), 0), N))


def attention_forward(q, k, v, scale, causal=False, seqlens=None, heads=None):
    """Batched [B, H, N, d] forward.  heads: optional list of (b, h) to compute.

    Returns (O, LSE); entries of heads not computed are NaN.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, H, N, d = q.shape
    O = np.full((B, H, N, d), np.nan)
    LSE = np.full((B, H, N), np.nan)
    for b, h in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        o, lse, _ = head_forward(q[b, h], k[b, h], v[b, h], scale, causal, _seqlen(seqlens, b, N))
        O[b, h], LSE[b, h] = o, lse
    return O, LSE


def attention_backward(q, k, v, do, scale, causal=False, seqlens=None, heads=None, jacobian="auto"):
    """Batched [B, H, N, d] forward + backward.  Returns dict of float64 arrays
    (o, lse, dq, dk, dv, delta); entries of heads not computed are NaN."""
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, H, N, d = q.shape
    out = {n: np.full((B, H, N, d), np.nan) for n in ("o", "dq", "dk", "dv")}
    out["lse"] = np.full((B, H, N), np.nan)
    out["delta"] = np.full((B, H, N), np.nan)
    for b, h in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        r = head_backward(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, _seqlen(seqlens, b, N), jacobian)
        for n in out:
            out[n][b, h] = r[n]
    return out


def rows_forward_backward(q, k, v, do, scale, rows, causal=False, L=None):
    """One head, selected query rows only: (O, LSE, dQ) for those rows.

    Each row is self-contained (its softmax, its Jacobian), so this is the
    full definition restricted to the chosen rows.  float64 [N, d] inputs.
    """
    N = q.shape[0]
    L = N if L is None else int(min(max(L, 0), N))
    rows = np.asarray(rows)
    A = _mask_rows(rows, N, L, causal)
    S = np.where(A, scale * (q[rows] @ k.T), -np.inf)
    P, lse = _softmax_rows(S, A)
    O = P @ v
    dP = do[rows] @ v.T
    dS = _softmax_vjp_factored(P, dP, A)
    dq = scale * (dS @ k)
    return O, lse, dq


def key_columns_backward(q, k, v, do, scale, cols, causal=False, L=None, chunk=512):
    """One head, selected key rows of dK and dV, streaming all queries in chunks.

    dK_j and dV_j sum over every query, so each chunk of query rows forms its
    full score rows (for its softmax and its Jacobian) and contributes to the
    chosen columns.  Returns (dK[cols], dV[cols]).
    """
    N, d = q.shape
    L = N if L is None else int(min(max(L, 0), N))
    cols = np.asarray(cols)
    dk = np.zeros((cols.size, d))
    dv = np.zeros((cols.size, d))
    for r0 in range(0, N, chunk):
        rows = np.arange(r0, min(N, r0 + chunk))
        A = _mask_rows(rows, N, L, causal)
        S = np.where(A, scale * (q[rows] @ k.T), -np.inf)
        P, _ = _softmax_rows(S, A)
        dP = do[rows] @ v.T
        dS = _softmax_vjp_factored(P, dP, A)
        dk += scale * (dS[:, cols].T @ q[rows])
        dv += P[:, cols].T @ do[rows]
    return dk, dv


def _mask_rows(rows, N, L, causal):
    """allowed_mask restricted to the given query rows (no N x N array)."""
    i = np.asarray(rows)[:, None]
    j = np.arange(N)[None, :]
    a = (i < L) & (j < L)
    if causal:
        a = a & (j <= i)
    return a
