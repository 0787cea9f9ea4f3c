"""Where the backward tolerance comes from (CPU).

The pages fix no tolerance for the gradients.  This float64 model repeats the
chain-rule formulas of ``oracle.backward`` with the kernels' rounding points
applied -- O rounded to bf16 before D = rowsum(dO * O), L to float32,
P = exp(S - L) to float32 and then to bf16 as the dV operand, and
dS = P * (dP - D) to bf16 as the dQ and dK operand; everything else in
float64 -- and measures each gradient's relative L2 error against the exact
oracle on the shapes and scales the GPU tests use.

The GPU backward tests hold every gradient to relative L2 <= 5e-3 (<= 1e-2
where scale * sqrt(d) > 3, i.e. nearly one-hot softmax rows where the bf16
rounding of dS dominates).  This test asserts that the modelled error of the
kernels' rounding scheme sits below those bounds with at least a factor 1.5
of margin, so the bounds are neither arbitrary nor tight enough to fail on
correct kernels.  It also checks that the model is a model of rounding only:
with every rounding removed it reproduces the oracle to float64 accuracy.
"""

import numpy as np
import pytest

from oracle.backward import backward_head
from workloads import bf16_bits_from_f32, bf16_bits_to_f64, by_name, make_grad_output, make_inputs


def bf(x):
    return bf16_bits_to_f64(bf16_bits_from_f32(np.asarray(x, dtype=np.float32)))


def f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def modelled_head(q, k, v, do, scale, causal, rounded=True):
    """dQ, dK, dV with the kernels' rounding points (identity maps when not rounded)."""
    rb = bf if rounded else (lambda a: a)
    rf = f32 if rounded else (lambda a: a)
    N = q.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = rb((p / l[:, None]) @ v)                    # the forward's bf16 output
    L = rf(m + np.log(l))                           # the forward's float32 lse
    p32 = rf(np.exp(s - L[:, None]))
    dv = rb(p32).T @ do
    D = np.sum(do * o, axis=1)
    dsb = rb(p32 * (do @ v.T - D[:, None]))
    return scale * (dsb @ k), scale * (dsb.T @ q), dv


# (N, d, causal, scale, bound the GPU tests hold the gradients to)
CASES = [(333, 64, True, None, 5e-3), (1000, 128, True, None, 5e-3), (700, 128, False, None, 5e-3),
         (200, 64, True, 0.9, 1e-2), (200, 128, True, 0.9, 1e-2), (200, 128, True, -0.3, 5e-3),
         (333, 256, True, None, 5e-3), (300, 256, False, None, 5e-3), (200, 256, True, 0.9, 1e-2)]


def _head_inputs(N, d, causal):
    w = by_name("gpt2s_causal_bf16_b8h12n1024d64").with_(B=1, H=2, N=N, d=d, causal=causal, seed=77)
    x = make_inputs(w)
    do = bf16_bits_to_f64(make_grad_output(w))
    return w, x, do


@pytest.mark.parametrize("N,d,causal,scale,bound", CASES)
def test_modelled_error_below_bound(N, d, causal, scale, bound):
    w, x, do = _head_inputs(N, d, causal)
    sc = w.softmax_scale if scale is None else scale
    for h in range(w.H):
        q, k, v = x.f64("q", 0, h), x.f64("k", 0, h), x.f64("v", 0, h)
        ex = backward_head(q, k, v, do[0, h], sc, causal)
        mo = modelled_head(q, k, v, do[0, h], sc, causal)
        for name, a, b in zip(("dq", "dk", "dv"), mo, ex):
            rel = np.linalg.norm(a - b) / np.linalg.norm(b)
            assert rel * 1.5 <= bound, f"N={N} d={d} scale={sc:.3g} head {h} {name}: modelled {rel:.2e}"


def test_model_without_rounding_is_the_oracle():
    w, x, do = _head_inputs(97, 64, True)
    q, k, v = x.f64("q", 0, 0), x.f64("k", 0, 0), x.f64("v", 0, 0)
    ex = backward_head(q, k, v, do[0, 0], w.softmax_scale, True)
    mo = modelled_head(q, k, v, do[0, 0], w.softmax_scale, True, rounded=False)
    for a, b in zip(mo, ex):
        assert np.linalg.norm(a - b) <= 1e-12 * np.linalg.norm(b)
