"""Attention by its definition, in float64 (test infrastructure only).

Follows the formula Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V as the
systems-analysis.info page "FlashAttention (PL)" writes it under
"Problematyka standardowego mechanizmu uwagi" and the chipfoundryservices
glossary entry "Flash Attention" writes it in its "Standard attention"
paragraph.  The 1/sqrt(d_k) factor is the ``scale`` argument.  The optional
causal mask is the one the robocikowo.com page names: query i sees key j iff
j <= i.  L is the per-row logsumexp that page says the backward pass keeps,
taken over the scaled scores with the natural logarithm.

The softmax is the standard two-pass form the glossary's "Online Softmax
Trick" paragraph contrasts with the online one: first the row maximum, then
exp and sum over the full row.  Rows are processed in chunks only to bound
memory; each row's softmax always sees the whole row.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def attention_rows(q, k, v, scale, causal, rows=None):
    """O and L for selected query rows of one head.

    q: [N, d] float64 queries, k: [N, d] keys, v: [N, d] values.
    rows: integer indices of the query rows to compute (default: all).
    Returns (O [len(rows), d], L [len(rows)]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if rows is None:
        rows = np.arange(q.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    s = scale * (q[rows] @ k.T)                       # [r, N] scores
    if causal:
        cols = np.arange(k.shape[0])
        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
    m = s.max(axis=1)                                  # pass 1: row maximum
    m_safe = np.where(np.isfinite(m), m, 0.0)          # a fully masked row keeps exp(-inf) = 0
    p = np.exp(s - m_safe[:, None])                    # pass 2: exponentials ...
    l = p.sum(axis=1)                                  # ... and their sum
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (p @ v) / l[:, None]
        lse = m_safe + np.log(l)
    empty = l == 0
    if empty.any():                                    # no visible key: O = 0, L = -inf
        o[empty] = 0.0
        lse[empty] = -np.inf
    return o, lse


def _limit_blas_threads():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except Exception:  # threadpoolctl missing: run with whatever BLAS does
        import contextlib
        return contextlib.nullcontext()


def attention_naive(q, k, v, scale, causal, row_chunk=1024, threads=None):
    """O [B,H,N,d] and L [B,H,N] for float64 tensors q, k, v of shape [B,H,N,d].

    Work is split over (b, h, row chunk) on a thread pool of ``threads``
    workers (default: every core this process may run on), each running
    single-threaded BLAS.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, d), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    tasks = [(b, h, r0) for b in range(B) for h in range(H) for r0 in range(0, N, row_chunk)]

    def run(task):
        b, h, r0 = task
        rows = np.arange(r0, min(r0 + row_chunk, N))
        o[b, h, rows], lse[b, h, rows] = attention_rows(q[b, h], k[b, h], v[b, h], scale, causal, rows)

    threads = threads or len(os.sched_getaffinity(0))
    with _limit_blas_threads():
        if threads <= 1 or len(tasks) == 1:
            for t in tasks:
                run(t)
        else:
            with ThreadPoolExecutor(max_workers=threads) as ex:
                list(ex.map(run, tasks))
    return o, lse
