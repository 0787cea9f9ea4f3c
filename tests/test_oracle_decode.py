"""Pins of the decode-shaped oracle and the key-split merge (oracle/decode.py)
against things other than themselves: the square oracle, a plain-loop brute
force, and the merge identity checked against attention over all keys."""

import math

import numpy as np
import pytest

from oracle import attention_rows
from oracle.decode import attention_decode, attention_decode_gqa, merge_partials, partial_over_keys

SCALE = 0.3


def _rand(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def _bruteforce_row(q_row, k, v, scale, visible):
    """One row in plain Python loops: softmax over the visible keys, math.fsum sums."""
    s = [scale * math.fsum(a * b for a, b in zip(q_row, k[j])) for j in visible]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    l = math.fsum(e)
    o = [math.fsum(e[t] * v[j][c] for t, j in enumerate(visible)) / l for c in range(len(v[0]))]
    return o, m + math.log(l)


def _pins_hold(decode, merge):
    ok = True
    # square problem: decode equals the square oracle
    q, k, v = _rand(9, 4, seed=1), _rand(9, 4, seed=2), _rand(9, 4, seed=3)
    for causal in (False, True):
        o, l = decode(q, k, v, SCALE, causal)
        o2, l2 = attention_rows(q, k, v, SCALE, causal)
        ok &= np.allclose(o, o2, rtol=0, atol=1e-13) and np.allclose(l, l2, rtol=0, atol=1e-13)
    # the last N_q rows of a square causal problem
    N_k, N_q = 13, 3
    qf, k, v = _rand(N_k, 5, seed=4), _rand(N_k, 5, seed=5), _rand(N_k, 5, seed=6)
    o, l = decode(qf[N_k - N_q:], k, v, SCALE, True)
    o2, l2 = attention_rows(qf, k, v, SCALE, True, rows=np.arange(N_k - N_q, N_k))
    ok &= np.allclose(o, o2, rtol=0, atol=1e-13) and np.allclose(l, l2, rtol=0, atol=1e-13)
    # brute force, one query against all keys
    q1 = _rand(1, 5, seed=7)
    o, l = decode(q1, k, v, SCALE, False)
    ob, lb = _bruteforce_row(list(q1[0]), k.tolist(), v.tolist(), SCALE, list(range(N_k)))
    ok &= np.allclose(o[0], ob, rtol=0, atol=1e-13) and abs(l[0] - lb) < 1e-13
    # merged partials of a key split equal the whole
    q, k, v = _rand(4, 6, seed=8), _rand(37, 6, seed=9), _rand(37, 6, seed=10)
    for causal in (False, True):
        for cuts in ([0, 37], [0, 10, 37], [0, 1, 2, 20, 35, 37], [0, 0, 16, 16, 37]):
            parts = [partial_over_keys(q, k, v, SCALE, causal, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
            o, l = merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
            o2, l2 = decode(q, k, v, SCALE, causal)
            ok &= np.allclose(o, o2, rtol=0, atol=1e-12) and np.allclose(l, l2, rtol=0, atol=1e-12)
    return bool(ok)


def test_pins_accept_oracle():
    assert _pins_hold(attention_decode, merge_partials)


def test_merge_ignores_empty_parts_and_order():
    rng = np.random.default_rng(12)
    o_parts = rng.standard_normal((4, 5, 3))
    l_parts = rng.standard_normal((4, 5))
    l_parts[2, :] = -np.inf                       # a part no row sees
    o_parts[2, :] = 0.0
    o, l = merge_partials(o_parts, l_parts)
    o2, l2 = merge_partials(o_parts[[3, 0, 1]], l_parts[[3, 0, 1]])
    assert np.allclose(o, o2, rtol=0, atol=1e-14) and np.allclose(l, l2, rtol=0, atol=1e-14)
    o1, l1 = merge_partials(o_parts[:1], l_parts[:1])
    assert np.array_equal(o1, o_parts[0]) and np.allclose(l1, l_parts[0], rtol=0, atol=1e-15)


def test_causal_decode_rows_see_a_growing_prefix():
    # query i of N_q sees N_k - N_q + i + 1 keys: with V = key index, O is a weighted index below that bound
    N_k, N_q = 20, 4
    q, k = _rand(N_q, 3, seed=13), _rand(N_k, 3, seed=14)
    v = np.tile(np.arange(N_k, dtype=np.float64)[:, None], (1, 2))
    o, _ = attention_decode(q, k, v, SCALE, True)
    for i in range(N_q):
        assert o[i, 0] <= N_k - N_q + i + 1e-12
    # a query that sees one key more than the previous: zero query gives the plain prefix mean
    o0, l0 = attention_decode(np.zeros((N_q, 3)), k, v, SCALE, True)
    for i in range(N_q):
        n = N_k - N_q + i + 1
        assert abs(o0[i, 0] - (n - 1) / 2) < 1e-12 and abs(l0[i] - math.log(n)) < 1e-12


def test_gqa_decode_matches_per_head():
    q = _rand(2, 6, 3, 4, seed=15)
    k, v = _rand(2, 2, 11, 4, seed=16), _rand(2, 2, 11, 4, seed=17)
    o, l = attention_decode_gqa(q, k, v, SCALE, True)
    for b in range(2):
        for h in range(6):
            o2, l2 = attention_decode(q[b, h], k[b, h // 3], v[b, h // 3], SCALE, True)
            assert np.allclose(o[b, h], o2, rtol=0, atol=1e-15) and np.allclose(l[b, h], l2, rtol=0, atol=1e-15)


def _mutant_decode(kind):
    def fn(q, k, v, scale, causal):
        N_q, N_k = q.shape[0], k.shape[0]
        s = scale * (q @ k.T)
        if causal:
            off = 0 if kind == "top_left" else N_k - N_q
            s = np.where(np.arange(N_k)[None, :] > (off + np.arange(N_q))[:, None], -np.inf, s)
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        return (p @ v) / p.sum(axis=1)[:, None], m + np.log(p.sum(axis=1))
    return fn


def _mutant_merge(kind):
    def fn(o_parts, lse_parts):
        if kind == "plain_mean":
            return o_parts.mean(axis=0), np.log(np.exp(lse_parts).sum(axis=0))
        w = np.exp(lse_parts)
        if kind == "max_only":
            return o_parts[np.argmax(lse_parts, axis=0), np.arange(o_parts.shape[1])], lse_parts.max(axis=0)
        # "unnormalised": weights not divided by their sum
        return np.einsum("sr,srd->rd", w, o_parts), np.log(w.sum(axis=0))
    return fn


@pytest.mark.parametrize("kind", ["top_left"])
def test_pins_reject_wrong_alignment(kind):
    assert not _pins_hold(_mutant_decode(kind), merge_partials)


@pytest.mark.parametrize("kind", ["plain_mean", "max_only", "unnormalised"])
def test_pins_reject_wrong_merge(kind):
    assert not _pins_hold(attention_decode, _mutant_merge(kind))
