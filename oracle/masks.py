"""Attention under the non-standard masks: ALiBi linear biases and a
block-sparse mask, in float64 (test infrastructure only).

The robocikowo.com "Flash Attention" page says masks such as ALiBi or
block-sparse patterns need special kernel variants, and the systems-analysis
page lists FlashMask among the literature; neither gives a formula.  Read
here as:

* ALiBi: the score of query i and key j gets the bias -slope_h * |i - j|
  added after scaling, S_ij = scale * q_i . k_j - slope_h * |i - j|, one slope
  per head (under the causal mask only j <= i remain, so the bias is
  -slope_h * (i - j)).
* block-sparse: a boolean matrix over (query block, key block) pairs of
  BLOCK x BLOCK elements; the scores of a pair marked 0 are -inf (never
  computed).  It combines with the causal mask.  A row with no visible key
  has O = 0 and L = -inf.

Both are the plain definition of ``naive`` with the bias added to, or the
mask applied to, the full score matrix.  Pins: tests/test_oracle_masks.py.
"""

import numpy as np

BLOCK = 128


def attention_biased(q, k, v, scale, causal, bias=None, allowed=None, rows=None):
    """O and L of one head with an optional additive bias (added after
    scaling) and an optional boolean mask of allowed scores.  q, k, v [N, d];
    rows: the query rows to compute (default all); bias and allowed are
    [len(rows), N], the rows' lines of the full N x N matrices."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    N = len(rows)
    s = scale * (q[rows] @ k.T)
    if bias is not None:
        s = s + bias
    keep = np.ones((N, k.shape[0]), dtype=bool) if allowed is None else np.asarray(allowed, dtype=bool)
    if causal:
        keep &= np.arange(k.shape[0])[None, :] <= rows[:, None]
    s = np.where(keep, s, -np.inf)
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m_safe[:, None])
    l = p.sum(axis=1)
    o = np.zeros((N, v.shape[1]))
    lse = np.full(N, -np.inf)
    seen = l > 0
    o[seen] = (p[seen] @ v) / l[seen, None]
    lse[seen] = m_safe[seen] + np.log(l[seen])
    return o, lse


def alibi_bias(N, slope, rows=None):
    """-slope * |i - j| for an N x N score matrix (or its given rows)."""
    idx = np.arange(N, dtype=np.float64)
    ri = idx if rows is None else np.asarray(rows, dtype=np.float64)
    return -float(slope) * np.abs(ri[:, None] - idx[None, :])


def attention_alibi(q, k, v, scale, causal, slopes):
    """O [B,H,N,d], L [B,H,N] with ALiBi biases, slopes [H] (float64 inputs)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, H, N, _ = q.shape
    o = np.empty(q.shape)
    lse = np.empty((B, H, N))
    for h in range(H):
        bias = alibi_bias(N, slopes[h])
        for b in range(B):
            o[b, h], lse[b, h] = attention_biased(q[b, h], k[b, h], v[b, h], scale, causal, bias=bias)
    return o, lse


def expand_block_mask(block_mask, N, block=BLOCK, rows=None):
    """Boolean [N, N] (or its given rows) from a block mask [ceil(N/block), ceil(N/block)]."""
    bm = np.asarray(block_mask, dtype=bool)
    idx = np.arange(N) // block
    ridx = idx if rows is None else np.asarray(rows, dtype=np.int64) // block
    return bm[ridx[:, None], idx[None, :]]


def attention_blocksparse(q, k, v, scale, causal, block_mask):
    """O [B,H,N,d], L [B,H,N] under a block mask [B, H, nb, nb] (float64 inputs)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, H, N, _ = q.shape
    o = np.empty(q.shape)
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            allowed = expand_block_mask(block_mask[b, h], N)
            o[b, h], lse[b, h] = attention_biased(q[b, h], k[b, h], v[b, h], scale, causal, allowed=allowed)
    return o, lse
