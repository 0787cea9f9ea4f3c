"""Decode-shaped attention and the logsumexp merge of key-split partials, in
float64 (test infrastructure only).

Decode shape: N_q query rows against N_k >= N_q keys, the queries being the
last N_q positions of the sequence.  Under the causal mask query i (0-based
among the N_q) sits at position N_k - N_q + i and sees keys j <= N_k - N_q + i
(with N_q = N_k this is the square mask of ``naive``).  The pages cite
sequence parallelism (systems-analysis.info "FlashAttention (PL)", section
"FlashAttention-2 (2023)") and decoding work (its literature list); they
give no formula for either, so this is the plain definition of attention
over the keys each query sees.

Key split: the keys are cut into ranges; over each range r the attention of
a row is O_r (normalised over that range) with logsumexp L_r.  Since
softmax over the union is exp(S - L) with L = log(sum_r exp(L_r)), the full
result is O = sum_r exp(L_r - L) * O_r.  ``merge_partials`` applies that
identity; a range a row does not see has L_r = -inf and O_r = 0 and drops out.

Pins (tests/test_oracle_decode.py): equality with the square oracle when
N_q = N_k and with the last rows of a square causal problem, a plain-loop
brute force, merged partials of random key splits against the whole, and
planted mistakes.
"""

import numpy as np


def _decode_scores(q, k, scale, causal, key_lo=0, key_hi=None):
    """Scaled scores of q [N_q, d] against keys [key_lo, key_hi) of k [N_k, d],
    with invisible keys at -inf."""
    N_q, N_k = q.shape[0], k.shape[0]
    key_hi = N_k if key_hi is None else key_hi
    cols = np.arange(key_lo, key_hi)
    s = scale * (q @ k[key_lo:key_hi].T)
    if causal:
        pos = N_k - N_q + np.arange(N_q)
        s = np.where(cols[None, :] > pos[:, None], -np.inf, s)
    return s


def _softmax_rows(s, v):
    """O = softmax(s) v row by row and L = logsumexp(s); rows with no finite score give O = 0, L = -inf."""
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m_safe[:, None])
    l = p.sum(axis=1)
    o = np.zeros((s.shape[0], v.shape[1]))
    lse = np.full(s.shape[0], -np.inf)
    seen = l > 0
    o[seen] = (p[seen] @ v) / l[seen, None]
    lse[seen] = m_safe[seen] + np.log(l[seen])
    return o, lse


def attention_decode(q, k, v, scale, causal):
    """O [N_q, d] and L [N_q] of one head: q [N_q, d], k and v [N_k, d], N_q <= N_k."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    if q.shape[0] > k.shape[0]:
        raise ValueError("decode shape needs N_q <= N_k")
    return _softmax_rows(_decode_scores(q, k, scale, causal), v)


def partial_over_keys(q, k, v, scale, causal, key_lo, key_hi):
    """(O_r, L_r) of one head over keys [key_lo, key_hi): attention normalised over
    that range alone (the causal alignment still refers to all N_k keys)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    return _softmax_rows(_decode_scores(q, k, scale, causal, key_lo, key_hi), v[key_lo:key_hi])


def merge_partials(o_parts, lse_parts):
    """O [rows, d], L [rows] from partials o_parts [S, rows, d], lse_parts [S, rows]."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_parts - m_safe[None, :])            # [S, rows]; -inf parts weigh 0
    tot = w.sum(axis=0)
    o = np.zeros(o_parts.shape[1:])
    lse = np.full(o_parts.shape[1], -np.inf)
    seen = tot > 0
    o[seen] = np.einsum("sr,srd->rd", w[:, seen], o_parts[:, seen]) / tot[seen, None]
    lse[seen] = m_safe[seen] + np.log(tot[seen])
    return o, lse


def attention_decode_gqa(q, k, v, scale, causal):
    """O [B, H, N_q, d], L [B, H, N_q] for q [B, H, N_q, d] and k, v [B, H_kv, N_k, d];
    query head h reads K/V head h // (H / H_kv)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, H, N_q, d = q.shape
    H_kv = k.shape[1]
    if H % H_kv:
        raise ValueError(f"{H} query heads do not split into groups over {H_kv} K/V heads")
    G = H // H_kv
    o = np.empty((B, H, N_q, d))
    lse = np.empty((B, H, N_q))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attention_decode(q[b, h], k[b, h // G], v[b, h // G], scale, causal)
    return o, lse
