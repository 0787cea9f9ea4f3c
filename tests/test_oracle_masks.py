"""Pins of the masked-attention oracle (oracle/masks.py) against things other
than itself: the plain oracle, causal ALiBi as plain attention on augmented
vectors, a plain-loop brute force, block-diagonal independence, and planted
mistakes."""

import math

import numpy as np
import pytest

from oracle import attention_rows
from oracle.masks import BLOCK, alibi_bias, attention_alibi, attention_biased, attention_blocksparse, expand_block_mask

SCALE = 0.35


def _rand(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def _bruteforce(q, k, v, scale, causal, slope=0.0, allowed=None, rows=None):
    """Plain loops and math.fsum, one row at a time (the given rows, default all)."""
    N, d = q.shape
    rows = list(range(N)) if rows is None else list(rows)
    o = np.zeros((len(rows), v.shape[1]))
    lse = np.full(len(rows), -np.inf)
    for r, i in enumerate(rows):
        vis = [j for j in range(k.shape[0]) if (not causal or j <= i) and (allowed is None or allowed[i][j])]
        if not vis:
            continue
        s = [scale * math.fsum(q[i][c] * k[j][c] for c in range(d)) - slope * abs(i - j) for j in vis]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        l = math.fsum(e)
        o[r] = [math.fsum(e[t] * v[j][c] for t, j in enumerate(vis)) / l for c in range(v.shape[1])]
        lse[r] = m + math.log(l)
    return o, lse


def _alibi_pins_hold(fn):
    ok = True
    q, k, v = _rand(1, 2, 11, 4, seed=1), _rand(1, 2, 11, 4, seed=2), _rand(1, 2, 11, 4, seed=3)
    for causal in (False, True):
        # slope 0 is plain attention
        o, l = fn(q, k, v, SCALE, causal, np.zeros(2))
        for h in range(2):
            o2, l2 = attention_rows(q[0, h], k[0, h], v[0, h], SCALE, causal)
            ok &= np.allclose(o[0, h], o2, rtol=0, atol=1e-13) and np.allclose(l[0, h], l2, rtol=0, atol=1e-13)
        # brute force with real slopes
        slopes = np.array([0.25, 1.5])
        o, l = fn(q, k, v, SCALE, causal, slopes)
        for h in range(2):
            ob, lb = _bruteforce(q[0, h], k[0, h], v[0, h], SCALE, causal, slopes[h])
            ok &= np.allclose(o[0, h], ob, rtol=0, atol=1e-12) and np.allclose(l[0, h], lb, rtol=0, atol=1e-12)
    # causal: the bias -m(i - j) is +m*j up to a per-row constant, i.e. plain
    # attention on q' = [q, m/scale] and k' = [k, j]; L differs by -m*i
    N, m = 23, 0.7
    q1, k1, v1 = _rand(N, 5, seed=4), _rand(N, 5, seed=5), _rand(N, 5, seed=6)
    qa = np.concatenate([q1, np.full((N, 1), m / SCALE)], axis=1)
    ka = np.concatenate([k1, np.arange(N, dtype=np.float64)[:, None]], axis=1)
    o2, l2 = attention_rows(qa, ka, v1, SCALE, True)
    o, l = fn(q1[None, None], k1[None, None], v1[None, None], SCALE, True, np.array([m]))
    ok &= np.allclose(o[0, 0], o2, rtol=0, atol=1e-11) and np.allclose(l[0, 0], l2 - m * np.arange(N), rtol=0,
                                                                        atol=1e-11)
    return bool(ok)


def _sparse_pins_hold(fn):
    ok = True
    N = 2 * BLOCK + 37
    nb = 3
    rng = np.random.default_rng(7)
    q, k, v = rng.standard_normal((1, 1, N, 4)), rng.standard_normal((1, 1, N, 4)), rng.standard_normal((1, 1, N, 4))
    for causal in (False, True):
        # all blocks allowed: plain attention
        o, l = fn(q, k, v, SCALE, causal, np.ones((1, 1, nb, nb), dtype=np.uint8))
        o2, l2 = attention_rows(q[0, 0], k[0, 0], v[0, 0], SCALE, causal)
        ok &= np.allclose(o[0, 0], o2, rtol=0, atol=1e-13) and np.allclose(l[0, 0], l2, rtol=0, atol=1e-13)
        # block-diagonal: every row block is its own attention problem
        o, l = fn(q, k, v, SCALE, causal, np.eye(nb, dtype=np.uint8)[None, None])
        for r in range(nb):
            sl = slice(r * BLOCK, min(N, (r + 1) * BLOCK))
            o2, l2 = attention_rows(q[0, 0, sl], k[0, 0, sl], v[0, 0, sl], SCALE, causal)
            ok &= np.allclose(o[0, 0, sl], o2, rtol=0, atol=1e-13) and np.allclose(l[0, 0, sl], l2, rtol=0,
                                                                                    atol=1e-13)
    # an irregular pattern against the brute force on sampled rows, including an empty row block
    bm = np.array([[0, 1, 0], [1, 0, 1], [0, 0, 0]], dtype=np.uint8)
    allowed = expand_block_mask(bm, N)
    for causal in (False, True):
        o, l = fn(q, k, v, SCALE, causal, bm[None, None])
        rows = [0, 5, BLOCK - 1, BLOCK, 200, N - 1]
        ob, lb = _bruteforce(q[0, 0], k[0, 0], v[0, 0], SCALE, causal, allowed=allowed.tolist(), rows=rows)
        ok &= np.allclose(o[0, 0, rows], ob, rtol=0, atol=1e-12) and np.allclose(l[0, 0, rows], lb, rtol=0, atol=1e-12)
        ok &= bool(np.all(o[0, 0, 2 * BLOCK:] == 0) and np.all(np.isneginf(l[0, 0, 2 * BLOCK:])))
    return bool(ok)


def test_alibi_pins_accept_oracle():
    assert _alibi_pins_hold(attention_alibi)


def test_sparse_pins_accept_oracle():
    assert _sparse_pins_hold(attention_blocksparse)


def test_alibi_bias_matrix():
    b = alibi_bias(4, 0.5)
    assert b[0, 0] == 0 and b[3, 0] == -1.5 and b[0, 3] == -1.5 and np.array_equal(b, b.T)


def test_expand_block_mask_ragged():
    bm = np.array([[1, 0], [0, 1]], dtype=np.uint8)
    m = expand_block_mask(bm, BLOCK + 5)
    assert m.shape == (BLOCK + 5, BLOCK + 5)
    assert m[0, 0] and not m[0, BLOCK] and m[BLOCK, BLOCK + 4] and not m[BLOCK + 4, BLOCK - 1]


def _alibi_mutant(kind):
    def fn(q, k, v, scale, causal, slopes):
        B, H, N, _ = q.shape
        o = np.empty(q.shape)
        lse = np.empty((B, H, N))
        for h in range(H):
            idx = np.arange(N, dtype=np.float64)
            if kind == "signed":
                bias = -slopes[h] * (idx[:, None] - idx[None, :])
            elif kind == "unscaled_order":
                bias = -slopes[h] * np.abs(idx[:, None] - idx[None, :]) / scale
            else:   # "positive"
                bias = slopes[h] * np.abs(idx[:, None] - idx[None, :])
            for b in range(B):
                o[b, h], lse[b, h] = attention_biased(q[b, h], k[b, h], v[b, h], scale, causal, bias=bias)
        return o, lse
    return fn


@pytest.mark.parametrize("kind", ["signed", "unscaled_order", "positive"])
def test_alibi_pins_reject_planted_mistakes(kind):
    assert not _alibi_pins_hold(_alibi_mutant(kind))


def _sparse_mutant(kind):
    def fn(q, k, v, scale, causal, block_mask):
        B, H, N, _ = q.shape
        o = np.empty(q.shape)
        lse = np.empty((B, H, N))
        for b in range(B):
            for h in range(H):
                bm = block_mask[b, h].T if kind == "transposed" else block_mask[b, h]
                blk = BLOCK + 1 if kind == "block_off_by_one" else BLOCK
                allowed = expand_block_mask(bm, N, blk)
                o[b, h], lse[b, h] = attention_biased(q[b, h], k[b, h], v[b, h], scale, causal, allowed=allowed)
        return o, lse
    return fn


@pytest.mark.parametrize("kind", ["transposed", "block_off_by_one"])
def test_sparse_pins_reject_planted_mistakes(kind):
    assert not _sparse_pins_hold(_sparse_mutant(kind))


@pytest.mark.parametrize("causal", [False, True])
def test_restricted_rows_agree_with_whole_matrix(causal):
    rng = np.random.default_rng(31)
    N = BLOCK + 50
    q, k, v = (rng.standard_normal((N, 5)) for _ in range(3))
    rows = np.array([0, 3, BLOCK - 1, BLOCK, N - 1])
    bias = alibi_bias(N, 0.3)
    o, l = attention_biased(q, k, v, SCALE, causal, bias=bias)
    o2, l2 = attention_biased(q, k, v, SCALE, causal, bias=alibi_bias(N, 0.3, rows), rows=rows)
    assert np.allclose(o2, o[rows], rtol=0, atol=1e-13) and np.allclose(l2, l[rows], rtol=0, atol=1e-13)
    bm = np.array([[1, 0], [1, 1]], dtype=np.uint8)
    o, l = attention_biased(q, k, v, SCALE, causal, allowed=expand_block_mask(bm, N))
    o2, l2 = attention_biased(q, k, v, SCALE, causal, allowed=expand_block_mask(bm, N, rows=rows), rows=rows)
    assert np.allclose(o2, o[rows], rtol=0, atol=1e-13) and np.allclose(l2, l[rows], rtol=0, atol=1e-13)
