"""Pins of the backward oracle (oracle/backward.py) against things other than itself.

* central finite differences of the forward oracle (oracle.naive / oracle.gqa)
  on tiny shapes: an independent route to the same derivative;
* invariants that hold exactly: the rows of dS sum to zero (so the keys' dK
  sum to zero and dQ does not change when a constant vector is added to every
  key), the rows of P sum to one (so the keys' dV sum to the queries' dO);
* planted mistakes that the finite-difference pin must reject.
"""

import numpy as np
import pytest

from oracle import attention_gqa
from oracle.backward import attention_backward, backward_head, delta_rows, dkdv_cols, dq_rows

SCALE = 0.7


def _loss(q, k, v, do, causal):
    o, _ = attention_gqa(q, k, v, SCALE, causal, threads=1)
    return float(np.sum(do * o))


def _fd(q, k, v, do, causal, eps=1e-5):
    grads = []
    for which in range(3):
        xs = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(xs[which])
        for idx in np.ndindex(*g.shape):
            orig = xs[which][idx]
            xs[which][idx] = orig + eps
            fp = _loss(*xs, do, causal)
            xs[which][idx] = orig - eps
            fm = _loss(*xs, do, causal)
            xs[which][idx] = orig
            g[idx] = (fp - fm) / (2 * eps)
        grads.append(g)
    return grads


def _tiny(H, H_kv, N=5, d=3, seed=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, H, N, d))
    k = rng.standard_normal((1, H_kv, N, d))
    v = rng.standard_normal((1, H_kv, N, d))
    do = rng.standard_normal((1, H, N, d))
    return q, k, v, do


def _bwd_pins_hold(fn, causal):
    ok = True
    for H, H_kv in ((2, 2), (4, 2)):
        q, k, v, do = _tiny(H, H_kv)
        got = fn(q, k, v, do, SCALE, causal)
        for g, f in zip(got, _fd(q, k, v, do, causal)):
            ok &= g.shape == f.shape and np.max(np.abs(g - f)) < 1e-7
    return bool(ok)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(2, 2), (4, 2), (3, 1)])
def test_backward_matches_finite_differences(causal, H, H_kv):
    q, k, v, do = _tiny(H, H_kv, seed=H * 10 + H_kv)
    got = attention_backward(q, k, v, do, SCALE, causal)
    for name, g, f in zip("qkv", got, _fd(q, k, v, do, causal)):
        assert np.max(np.abs(g - f)) < 1e-7, name


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    rng = np.random.default_rng(11)
    B, H, H_kv, N, d = 2, 4, 2, 37, 8
    q, do = (rng.standard_normal((B, H, N, d)) for _ in range(2))
    k, v = (rng.standard_normal((B, H_kv, N, d)) for _ in range(2))
    dq, dk, dv = attention_backward(q, k, v, do, SCALE, causal, row_chunk=16)
    G = H // H_kv
    for b in range(B):
        for g in range(H_kv):
            # rows of dS sum to zero -> sum over keys of dK is zero
            assert np.max(np.abs(dk[b, g].sum(axis=0))) < 1e-12
            # rows of P sum to one -> sum over keys of dV = sum over the group's queries of dO
            assert np.allclose(dv[b, g].sum(axis=0), do[b, g * G:(g + 1) * G].sum(axis=(0, 1)), rtol=0, atol=1e-12)
    # a constant added to every key moves no probability: all gradients are unchanged
    u = rng.standard_normal(d)
    dq2, dk2, dv2 = attention_backward(q, k + u, v, do, SCALE, causal)
    assert np.max(np.abs(dq2 - dq)) < 1e-11 and np.max(np.abs(dk2 - dk)) < 1e-11 and np.max(np.abs(dv2 - dv)) < 1e-11
    # no upstream gradient, no gradient
    z = attention_backward(q, k, v, np.zeros_like(do), SCALE, causal)
    assert all(np.all(t == 0) for t in z)


def test_constant_values_leave_no_score_gradient():
    # every value row equal: O does not depend on Q or K at all
    rng = np.random.default_rng(2)
    q, k, do = (rng.standard_normal((1, 2, 9, 4)) for _ in range(3))
    v = np.broadcast_to(rng.standard_normal(4), (1, 2, 9, 4)).copy()
    dq, dk, _ = attention_backward(q, k, v, do, SCALE, True)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13


def test_delta_is_the_softmax_row_term():
    rng = np.random.default_rng(4)
    q, k, v, do = (rng.standard_normal((1, 1, 6, 3)) for _ in range(4))
    o, _ = attention_gqa(q, k, v, SCALE, False, threads=1)
    s = SCALE * q[0, 0] @ k[0, 0].T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose(delta_rows(o, do)[0, 0], np.sum(p * (do[0, 0] @ v[0, 0].T), axis=1), rtol=0, atol=1e-13)


def test_pins_accept_oracle():
    for causal in (False, True):
        assert _bwd_pins_hold(lambda q, k, v, do, s, c: attention_backward(q, k, v, do, s, c), causal)


def _mutant(kind):
    """attention_backward with one planted mistake in the per-head formulas."""
    def head(q, k, v, do, scale, causal):
        N = q.shape[0]
        s = scale * (q @ k.T)
        if causal and kind != "mask_off":
            s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ v
        dp = do @ v.T
        D = np.sum(do * o, axis=1)
        ds = {"d_sign": p * (dp + D[:, None]), "no_d": p * dp}.get(kind, p * (dp - D[:, None]))
        dq = (1.0 if kind == "no_scale" else scale) * (ds @ k)
        dk = scale * ((p if kind == "dk_uses_p" else ds).T @ q)
        dv = (p @ do) if kind == "dv_untransposed" else (p.T @ do)
        return dq, dk, dv

    def fn(q, k, v, do, scale, causal):
        B, H = q.shape[:2]
        G = H // k.shape[1]
        dq, dk, dv = np.empty_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(H):
                a, bb, c = head(q[b, h], k[b, h // G], v[b, h // G], do[b, h], scale, causal)
                dq[b, h] = a
                dk[b, h // G] += bb
                dv[b, h // G] += c
        return dq, dk, dv
    return fn


@pytest.mark.parametrize("kind", ["d_sign", "no_d", "no_scale", "dk_uses_p", "dv_untransposed", "mask_off"])
def test_pins_reject_planted_mistakes(kind):
    assert not (_bwd_pins_hold(_mutant(kind), False) and _bwd_pins_hold(_mutant(kind), True))


def test_backward_head_rows_in_chunks_equal_whole():
    rng = np.random.default_rng(8)
    q, k, v, do = (rng.standard_normal((50, 8)) for _ in range(4))
    a = backward_head(q, k, v, do, 0.3, True, row_chunk=7)
    b = backward_head(q, k, v, do, 0.3, True, row_chunk=1024)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_restricted_forms_agree_with_whole_head(causal):
    rng = np.random.default_rng(21)
    N, d = 45, 6
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    dq, dk, dv = backward_head(q, k, v, do, 0.4, causal)
    rows = np.array([0, 1, 7, 30, 44])
    assert np.allclose(dq_rows(q, k, v, do, 0.4, causal, rows), dq[rows], rtol=0, atol=1e-12)
    keys = np.array([0, 3, 22, 44])
    a, b = dkdv_cols(q, k, v, do, 0.4, causal, keys, row_chunk=8)
    assert np.allclose(a, dk[keys], rtol=0, atol=1e-12) and np.allclose(b, dv[keys], rtol=0, atol=1e-12)
