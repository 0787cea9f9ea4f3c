"""Pins for the float64 oracle: facts the pages and the mathematics fix.

None of these re-types the oracle's formula.  They check it against
  * the pages' statement that the blockwise online softmax gives the identical
    (exact) result (dexblog.ro table row "Softmax online"; robocikowo.com
    closing paragraph "Exact attention") -> naive == online for any blocking;
  * a 50-digit brute force written with mpmath in plain Python loops;
  * closed forms: V = 1, Q = 0 (mean / prefix mean, L = ln n), causal row 0,
    N = 1, a two-token example solved by hand;
  * invariances: shifting every key by u, permuting keys/values jointly,
    permuting queries;
  * the logsumexp identity sum_j exp(S_ij - L_i) = 1, summed with math.fsum.
A last group plants plausible mistakes (wrong sign, missing scale, swapped
operands, mask off or shifted, L without the log) into copies of the oracle
and checks that the pins catch every one.
"""

import itertools
import math

import mpmath
import numpy as np
import pytest

from oracle import attention_gqa, attention_naive, attention_online, attention_rows


def rand_qkv(N, d, seed, B=None, H=None, scale_inputs=1.0):
    rng = np.random.default_rng(seed)
    shape = (N, d) if B is None else (B, H, N, d)
    return tuple(scale_inputs * rng.standard_normal(shape) for _ in range(3))


def brute_mp(q, k, v, scale, causal, dps=50):
    """O and L for one head by the definition, in mpmath at ``dps`` digits, plain loops."""
    mpmath.mp.dps = dps
    N, d = len(q), len(q[0])
    O, L = [], []
    for i in range(N):
        js = [j for j in range(N) if not (causal and j > i)]
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[i][t]) * mpmath.mpf(k[j][t]) for t in range(d)) for j in js]
        w = [mpmath.exp(x) for x in s]
        z = mpmath.fsum(w)
        O.append([mpmath.fsum(w[a] * mpmath.mpf(v[j][t]) for a, j in enumerate(js)) / z for t in range(d)])
        L.append(mpmath.log(z))
    return (np.array([[float(x) for x in row] for row in O]), np.array([float(x) for x in L]))


# ---------------------------------------------------------------- naive == online
@pytest.mark.parametrize("N", [1, 7, 100, 257])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("br,bc", [(1, 1), (3, 5), (16, 16), (64, 64), (None, None)])
def test_naive_equals_online(N, causal, br, bc):
    q, k, v = rand_qkv(N, 16, seed=N * 7 + causal)
    br = br or N
    bc = bc or N
    o1, l1 = attention_rows(q, k, v, 0.25, causal)
    o2, l2 = attention_online(q, k, v, 0.25, causal, br, bc)
    assert np.linalg.norm(o1 - o2) <= 1e-12 * np.linalg.norm(o1)
    assert np.max(np.abs(l1 - l2)) <= 1e-12 * max(1.0, np.max(np.abs(l1)))


def test_naive_4d_matches_rows_and_threads():
    q, k, v = rand_qkv(70, 8, seed=3, B=2, H=3)
    o, l = attention_naive(q, k, v, 0.3, True, row_chunk=16, threads=4)
    for b, h in itertools.product(range(2), range(3)):
        o1, l1 = attention_rows(q[b, h], k[b, h], v[b, h], 0.3, True)
        assert np.array_equal(o[b, h], o1) and np.array_equal(l[b, h], l1)
    o4, l4 = attention_online(q, k, v, 0.3, True, 8, 24)
    assert np.max(np.abs(o4 - o)) < 1e-12


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("N,d,causal", [(1, 3, False), (5, 4, True), (9, 8, False), (16, 8, True), (16, 5, False)])
def test_mpmath_bruteforce(N, d, causal):
    q, k, v = rand_qkv(N, d, seed=100 + N + d, scale_inputs=2.0)
    scale = 1.0 / math.sqrt(d)
    o_ref, l_ref = brute_mp(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    for o, l in (attention_rows(q, k, v, scale, causal), attention_online(q, k, v, scale, causal, 3, 2)):
        assert np.max(np.abs(o - o_ref)) < 1e-13
        assert np.max(np.abs(l - l_ref)) < 1e-13


def test_lse_identity_fsum():
    q, k, v = rand_qkv(40, 6, seed=9, scale_inputs=3.0)
    for causal in (False, True):
        _, L = attention_rows(q, k, v, 0.5, causal)
        for i in range(40):
            terms = []
            for j in range(40 if not causal else i + 1):
                s = 0.5 * math.fsum(float(q[i, t]) * float(k[j, t]) for t in range(6))
                terms.append(math.exp(s - float(L[i])))
            assert abs(math.fsum(terms) - 1.0) < 1e-13


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_v_all_ones_gives_ones(causal):
    q, k, _ = rand_qkv(130, 32, seed=11, scale_inputs=1.5)
    v = np.ones((130, 32))
    for o, _ in (attention_rows(q, k, v, 0.2, causal), attention_online(q, k, v, 0.2, causal, 32, 48)):
        assert np.max(np.abs(o - 1.0)) < 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_gives_mean_and_log_count(causal):
    N = 97
    _, k, v = rand_qkv(N, 12, seed=12)
    q = np.zeros((N, 12))
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = np.cumsum(v, axis=0) / counts[:, None] if causal else np.broadcast_to(v.mean(axis=0), (N, 12))
    for o, l in (attention_rows(q, k, v, 0.7, causal), attention_online(q, k, v, 0.7, causal, 10, 13)):
        assert np.max(np.abs(o - mean)) < 1e-13
        assert np.max(np.abs(l - np.log(counts))) < 1e-13


def test_causal_row0_is_v0():
    q, k, v = rand_qkv(50, 16, seed=13, scale_inputs=4.0)
    for o, l in (attention_rows(q, k, v, 0.25, True), attention_online(q, k, v, 0.25, True, 16, 16)):
        assert np.array_equal(o[0], v[0])
        assert abs(l[0] - 0.25 * float(q[0] @ k[0])) < 1e-13


def test_single_token():
    q, k, v = rand_qkv(1, 64, seed=14)
    for causal in (False, True):
        o, l = attention_rows(q, k, v, 0.125, causal)
        assert np.array_equal(o, v)
        assert abs(l[0] - 0.125 * float(q[0] @ k[0])) < 1e-13


def test_two_token_worked_example():
    # d = 1, scale = 1, q = [1, 1], k = [0, ln 3], v = [0, 1].  Scores for either
    # query are [0, ln 3], so the weights are [1/4, 3/4]: O = 3/4, L = ln 4.
    # Under the causal mask query 0 sees only key 0: O = 0, L = 0.
    q = np.array([[1.0], [1.0]])
    k = np.array([[0.0], [math.log(3.0)]])
    v = np.array([[0.0], [1.0]])
    o, l = attention_rows(q, k, v, 1.0, False)
    assert np.allclose(o[:, 0], [0.75, 0.75], atol=1e-15, rtol=0)
    assert np.allclose(l, [math.log(4.0)] * 2, atol=1e-15, rtol=0)
    o, l = attention_rows(q, k, v, 1.0, True)
    assert np.allclose(o[:, 0], [0.0, 0.75], atol=1e-15, rtol=0)
    assert np.allclose(l, [0.0, math.log(4.0)], atol=1e-15, rtol=0)


# ---------------------------------------------------------------- invariances
@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance_with_huge_scores(causal):
    N, d = 64, 16
    q, k, v = rand_qkv(N, d, seed=15)
    u = np.full(d, 40.0)          # scores move by ~hundreds: exp without the max would overflow
    o0, l0 = attention_rows(q, k, v, 1.0, causal)
    for o1, l1 in (attention_rows(q, k + u, v, 1.0, causal), attention_online(q, k + u, v, 1.0, causal, 16, 8)):
        assert np.all(np.isfinite(o1))
        assert np.max(np.abs(o1 - o0)) < 1e-11
        assert np.max(np.abs(l1 - (l0 + q @ u))) < 1e-10


def test_permutations():
    N, d = 45, 8
    q, k, v = rand_qkv(N, d, seed=16)
    perm = np.random.default_rng(0).permutation(N)
    o0, l0 = attention_rows(q, k, v, 0.4, False)
    o1, l1 = attention_rows(q, k[perm], v[perm], 0.4, False)
    assert np.max(np.abs(o1 - o0)) < 1e-14 and np.max(np.abs(l1 - l0)) < 1e-13
    o2, l2 = attention_rows(q[perm], k, v, 0.4, False)
    assert np.max(np.abs(o2 - o0[perm])) < 1e-14 and np.max(np.abs(l2 - l0[perm])) < 1e-13


def test_selected_rows_equal_full():
    q, k, v = rand_qkv(80, 8, seed=17)
    rows = np.array([0, 5, 79, 33])
    o, l = attention_rows(q, k, v, 0.3, True)
    os_, ls_ = attention_rows(q, k, v, 0.3, True, rows)
    assert np.array_equal(os_, o[rows]) and np.array_equal(ls_, l[rows])


# ---------------------------------------------------------------- planted mistakes
def _pins_hold(fn):
    """A compact battery of the pins above, for an arbitrary (q,k,v,scale,causal)->(O,L)."""
    ok = True
    q, k, v = rand_qkv(9, 4, seed=21, scale_inputs=2.0)
    for causal in (False, True):
        o_ref, l_ref = brute_mp(q.tolist(), k.tolist(), v.tolist(), 0.5, causal, dps=30)
        o, l = fn(q, k, v, 0.5, causal)
        ok &= np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(l - l_ref)) < 1e-12
    q0 = np.zeros_like(q)
    o, l = fn(q0, k, v, 0.5, True)
    ok &= np.max(np.abs(l - np.log(np.arange(1, 10)))) < 1e-12
    o, l = fn(q, k, v, 0.5, True)
    ok &= np.array_equal(o[0], v[0])
    return bool(ok)


def test_pins_accept_oracle():
    assert _pins_hold(lambda q, k, v, s, c: attention_rows(q, k, v, s, c))
    assert _pins_hold(lambda q, k, v, s, c: attention_online(q, k, v, s, c, 2, 3))


@pytest.mark.parametrize("mutant", [
    "sign", "no_scale", "swap_kv", "mask_off", "mask_shift", "lse_no_log", "no_normalise", "transpose_q",
])
def test_pins_reject_planted_mistakes(mutant):
    def shifted_mask(q, k, v, s, c):
        if not c:
            return attention_rows(q, k, v, s, c)
        # sees keys j <= i + 1 instead of j <= i
        N = len(q)
        o = np.empty_like(v); l = np.empty(N)
        for i in range(N):
            js = np.arange(min(i + 2, N))
            oi, li = attention_rows(q[i:i + 1], k[js], v[js], s, False)
            o[i], l[i] = oi[0], li[0]
        return o, l

    def transpose_q(q, k, v, s, c):
        n, d = q.shape
        qq = np.resize(q.T.copy(), (n, d))       # operand read in the wrong order
        return attention_rows(qq, k, v, s, c)

    fns = {
        "sign": lambda q, k, v, s, c: attention_rows(q, k, v, -s, c),
        "no_scale": lambda q, k, v, s, c: attention_rows(q, k, v, 1.0, c),
        "swap_kv": lambda q, k, v, s, c: attention_rows(q, v, k, s, c),
        "mask_off": lambda q, k, v, s, c: attention_rows(q, k, v, s, False),
        "mask_shift": shifted_mask,
        "lse_no_log": lambda q, k, v, s, c: (lambda o, l: (o, np.exp(l)))(*attention_rows(q, k, v, s, c)),
        "no_normalise": lambda q, k, v, s, c: (lambda o, l: (o * np.exp(l)[:, None], l))(*attention_rows(q, k, v, s, c)),
        "transpose_q": transpose_q,
    }
    assert not _pins_hold(fns[mutant])


# ---------------------------------------------------------------- grouped-query attention
def _gqa_pins_hold(fn):
    """Pins of the grouping rule for an arbitrary (q, k, v, scale, causal) -> (O, L) over
    q [B,H,N,d] and k, v [B,H_kv,N,d]: query head h must read K/V head h // (H / H_kv)."""
    ok = True
    rng = np.random.default_rng(5)
    B, H, H_kv, N, d = 2, 6, 3, 7, 4
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H_kv, N, d))
    # closed form: V constant per K/V head (value = 10*b + g + 1) -> every output row of a
    # query head equals its own group's constant, whatever the weights
    v = np.empty((B, H_kv, N, d))
    for b in range(B):
        for g in range(H_kv):
            v[b, g] = 10 * b + g + 1
    for causal in (False, True):
        o, _ = fn(q, k, v, 0.7, causal)
        for b in range(B):
            for h in range(H):
                ok &= np.max(np.abs(o[b, h] - (10 * b + h // (H // H_kv) + 1))) < 1e-12
    # each query head against its group's K/V, by the single-head definition
    v = rng.standard_normal((B, H_kv, N, d))
    o, l = fn(q, k, v, 0.7, True)
    for b in range(B):
        for h in range(H):
            g = h // (H // H_kv)
            oh, lh = attention_rows(q[b, h], k[b, g], v[b, g], 0.7, True)
            ok &= np.max(np.abs(o[b, h] - oh)) < 1e-12 and np.max(np.abs(l[b, h] - lh)) < 1e-12
    return bool(ok)


def test_gqa_pins_accept_oracle():
    assert _gqa_pins_hold(lambda q, k, v, s, c: attention_gqa(q, k, v, s, c, threads=1))


def test_gqa_with_all_heads_is_mha_and_mqa_shares_one_head():
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((1, 4, 9, 8)) for _ in range(3))
    o1, l1 = attention_gqa(q, k, v, 0.4, True, threads=1)
    o2, l2 = attention_naive(q, k, v, 0.4, True, threads=1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o, l = attention_gqa(q, k[:, :1], v[:, :1], 0.4, False, threads=1)     # MQA
    for h in range(4):
        oh, lh = attention_rows(q[0, h], k[0, 0], v[0, 0], 0.4, False)
        assert np.allclose(o[0, h], oh, rtol=0, atol=1e-13) and np.allclose(l[0, h], lh, rtol=0, atol=1e-13)
    with pytest.raises(ValueError):
        attention_gqa(q, k[:, :3], v[:, :3], 0.4, False)


@pytest.mark.parametrize("mutant", ["interleaved", "last_group", "swap_kv"])
def test_gqa_pins_reject_planted_mistakes(mutant):
    def interleaved(q, k, v, s, c):               # h -> h % H_kv instead of h // G
        H, H_kv = q.shape[1], k.shape[1]
        idx = np.arange(H) % H_kv
        return attention_naive(q, k[:, idx], v[:, idx], s, c, threads=1)

    def last_group(q, k, v, s, c):                # every head reads the last K/V head
        H, H_kv = q.shape[1], k.shape[1]
        idx = np.full(H, H_kv - 1)
        return attention_naive(q, k[:, idx], v[:, idx], s, c, threads=1)

    fns = {"interleaved": interleaved, "last_group": last_group,
           "swap_kv": lambda q, k, v, s, c: attention_gqa(q, v, k, s, c, threads=1)}
    assert not _gqa_pins_hold(fns[mutant])
