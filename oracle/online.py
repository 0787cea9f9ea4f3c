"""Blockwise online-softmax attention in float64 (test infrastructure only).

Written from the method's description, independently of ``naive``:

* Q is cut into row blocks of ``block_rows`` rows and K, V into column blocks
  of ``block_cols`` rows (chipfoundryservices glossary "Flash Attention",
  "Tiling Algorithm" step 1; the robocikowo.com page's B_r x d and B_c x d
  blocks).
* Each Q block is visited once and iterates over the K/V blocks (step 2).
* The block scores S = scale * Q_i K_j^T are formed (step 3).
* A running row maximum m and running row sum l are kept (step 4; the
  systems-analysis.info page "FlashAttention (PL)", "Obliczanie Softmax w
  trybie online"): when a block raises m, the earlier partial output and sum
  are multiplied by exp(m_old - m_new) -- the robocikowo page's
  rescale(O_prev, m_old, m_new) -- and the block adds exp(S - m_new) V_j
  (step 5).
* After the last block the accumulated output is divided by l once (step 6).

Under the causal mask, column blocks that lie entirely to the right of the
block's last row are skipped (they contribute exp(-inf) = 0 to every row), and
inside a block S[r, c] = -inf where key c > query r.
"""

import numpy as np


def _one_head(q, k, v, scale, causal, br, bc):
    N, d = q.shape
    out = np.zeros((N, d), dtype=np.float64)
    lse = np.zeros(N, dtype=np.float64)
    for r0 in range(0, N, br):
        r1 = min(r0 + br, N)
        qi = q[r0:r1]
        m = np.full(r1 - r0, -np.inf)
        l = np.zeros(r1 - r0)
        acc = np.zeros((r1 - r0, d))
        for c0 in range(0, N, bc):
            if causal and c0 > r1 - 1:
                break                                   # this and all later blocks are fully masked
            c1 = min(c0 + bc, N)
            s = scale * (qi @ k[c0:c1].T)
            if causal:
                rr = np.arange(r0, r1)[:, None]
                cc = np.arange(c0, c1)[None, :]
                s = np.where(cc > rr, -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            base = np.where(np.isfinite(m_new), m_new, 0.0)   # keeps -inf - (-inf) out
            alpha = np.exp(m - base)                          # exp(-inf) = 0 on the first block
            p = np.exp(s - base[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[c0:c1]
            m = m_new
        with np.errstate(invalid="ignore", divide="ignore"):
            out[r0:r1] = acc / l[:, None]
            lse[r0:r1] = m + np.log(l)
        dead = l == 0
        out[r0:r1][dead] = 0.0
        lse[r0:r1][dead] = -np.inf
    return out, lse


def attention_online(q, k, v, scale, causal, block_rows=64, block_cols=64):
    """O and L via the blockwise recurrence; q, k, v are [N, d] or [B, H, N, d] float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim == 2:
        return _one_head(q, k, v, scale, causal, block_rows, block_cols)
    B, H, N, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = _one_head(q[b, h], k[b, h], v[b, h], scale, causal, block_rows, block_cols)
    return o, lse
