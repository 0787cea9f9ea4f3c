"""Grouped-query (and multi-query) attention by its definition (test infrastructure only).

The systems-analysis.info page "FlashAttention (PL)", section
"FlashAttention-2 (2023)", lists Multi-Query Attention among the architectures
FlashAttention-2 extended its support to.  Read here with grouped-query
attention as the general case: the H query heads are split into H_kv
consecutive groups of G = H / H_kv heads, and every query head of group g
attends over K/V head g (MQA is H_kv = 1, ordinary multi-head attention is
H_kv = H).  Each query head's result is then exactly the plain attention of
that head against its group's K and V, so the oracle repeats every K/V head G
times and applies the plain definition of ``naive``.
"""

import numpy as np

from .naive import attention_naive


def expand_kv(x, H):
    """[B, H_kv, N, d] -> [B, H, N, d]: K/V head g repeated for query heads g*G .. g*G+G-1."""
    H_kv = x.shape[1]
    if H % H_kv:
        raise ValueError(f"{H} query heads do not split into groups over {H_kv} K/V heads")
    return np.repeat(x, H // H_kv, axis=1)


def attention_gqa(q, k, v, scale, causal, **kw):
    """O [B,H,N,d] and L [B,H,N] for q [B,H,N,d] and k, v [B,H_kv,N,d] (float64)."""
    H = q.shape[1]
    return attention_naive(q, expand_kv(np.asarray(k), H), expand_kv(np.asarray(v), H), scale, causal, **kw)
