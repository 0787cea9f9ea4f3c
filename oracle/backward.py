"""Gradients of the attention forward pass, in float64 (test infrastructure only).

The robocikowo.com "Flash Attention" page says the backward pass does not keep
the attention matrix: it recomputes it from the saved O and the per-row
logsumexp L (recomputation in place of a stored matrix, trading FLOPs for
memory).  The pages give no formulas, so this oracle is the derivative of the
forward definition (``naive``) written out by the chain rule, for the scalar
loss  sum(dO * O)  whose gradient a training step propagates:

    S  = scale * Q K^T   (causal: S_ij = -inf for j > i)
    P  = softmax(S) row-wise = exp(S - L)
    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij = sum_d dO_id O_id      (the row term of the softmax Jacobian)
    dS = P * (dP - D)                              (elementwise, D broadcast over j)
    dQ = scale * dS K
    dK = scale * dS^T Q

Grouped-query attention (K/V head g serving query heads g*G .. g*G+G-1): dK
and dV of a K/V head are the sums over the query heads of its group.

For large heads, ``dq_rows`` gives dQ of chosen query rows and ``dkdv_cols``
dK, dV of chosen keys, from the same formulas restricted to those rows or
columns of S (each still sees its whole softmax row).

Pins (tests/test_oracle_backward.py): central finite differences of the
forward oracle, closed forms and invariants, planted mistakes; the restricted
forms agree with ``backward_head`` on every row and key.
"""

import numpy as np


def backward_head(q, k, v, do, scale, causal, row_chunk=1024):
    """dQ [N, d], dK [N, d], dV [N, d] of one head (float64 inputs [N, d]).

    Query rows are processed in chunks only to bound memory; every row's
    softmax sees its whole (masked) row.
    """
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    N = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    cols = np.arange(k.shape[0])
    for r0 in range(0, N, row_chunk):
        rows = np.arange(r0, min(r0 + row_chunk, N))
        s = scale * (q[rows] @ k.T)
        if causal:
            s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
        m = s.max(axis=1)
        m = np.where(np.isfinite(m), m, 0.0)
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        p = np.divide(p, l[:, None], out=np.zeros_like(p), where=l[:, None] > 0)
        o = p @ v
        dv += p.T @ do[rows]
        dp = do[rows] @ v.T
        D = np.sum(do[rows] * o, axis=1)
        ds = p * (dp - D[:, None])
        dq[rows] = scale * (ds @ k)
        dk += scale * (ds.T @ q[rows])
    return dq, dk, dv


def attention_backward(q, k, v, do, scale, causal, row_chunk=1024):
    """dQ [B,H,N,d], dK and dV [B,H_kv,N,d] for q, do [B,H,N,d] and k, v [B,H_kv,N,d] (float64)."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if H % H_kv:
        raise ValueError(f"{H} query heads do not split into groups over {H_kv} K/V heads")
    G = H // H_kv
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = h // G
            dq[b, h], dkh, dvh = backward_head(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal, row_chunk)
            dk[b, g] += dkh
            dv[b, g] += dvh
    return dq, dk, dv


def delta_rows(o, do):
    """D = rowsum(dO * O) per query row, the quantity the backward precomputes ([..., N])."""
    return np.sum(np.asarray(o, dtype=np.float64) * np.asarray(do, dtype=np.float64), axis=-1)


def _masked_scores(q, k, scale, causal, rows, cols):
    s = scale * (q[rows] @ k[cols].T)
    if causal:
        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
    return s


def _row_stats(q, k, v, do, scale, causal, rows):
    """Row max m, row sum l (so L = m + log l), O rows and D rows for the given query rows."""
    cols = np.arange(k.shape[0])
    s = _masked_scores(q, k, scale, causal, rows, cols)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = (p / l[:, None]) @ v
    return m, l, o, np.sum(do[rows] * o, axis=1)


def dq_rows(q, k, v, do, scale, causal, rows):
    """dQ [len(rows), d] of one head for the given query rows (float64)."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(k.shape[0])
    s = _masked_scores(q, k, scale, causal, rows, cols)
    m, l, _, D = _row_stats(q, k, v, do, scale, causal, rows)
    p = np.exp(s - m[:, None]) / l[:, None]
    ds = p * (do[rows] @ v.T - D[:, None])
    return scale * (ds @ k)


def dkdv_cols(q, k, v, do, scale, causal, keys, row_chunk=1024):
    """dK, dV [len(keys), d] of one head for the given keys (float64): the
    softmax statistics of every query row, then the keys' columns of P and dS."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    keys = np.asarray(keys, dtype=np.int64)
    N = q.shape[0]
    dk = np.zeros((len(keys), q.shape[1]))
    dv = np.zeros_like(dk)
    for r0 in range(0, N, row_chunk):
        rows = np.arange(r0, min(r0 + row_chunk, N))
        m, l, _, D = _row_stats(q, k, v, do, scale, causal, rows)
        s = _masked_scores(q, k, scale, causal, rows, keys)
        p = np.exp(s - m[:, None]) / l[:, None]
        ds = p * (do[rows] @ v[keys].T - D[:, None])
        dv += p.T @ do[rows]
        dk += scale * (ds.T @ q[rows])
    return dk, dv
