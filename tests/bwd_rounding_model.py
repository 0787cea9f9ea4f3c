"""Float64 model of the backward kernels' roundings, from which the backward
tolerance is derived (run by hand: ``python tests/bwd_rounding_model.py``).

It repeats the chain-rule formulas of ``oracle.backward`` with the kernel's
rounding points applied: O rounded to bf16 before D = rowsum(dO * O), L to
float32, P = exp(S - L) to float32 and then to bf16 as the dV operand, and
dS = P * (dP - D) to bf16 as the dQ and dK operand; everything else in
float64.  It prints the relative L2 error of each gradient against the exact
oracle for the shapes and scales the GPU tests use.
"""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from oracle.backward import backward_head  # noqa: E402
from workloads import bf16_bits_from_f32, bf16_bits_to_f64, by_name, make_grad_output, make_inputs  # noqa: E402


def bf(x):
    return bf16_bits_to_f64(bf16_bits_from_f32(np.asarray(x, dtype=np.float32)))


def modelled_head(q, k, v, do, scale, causal):
    N = q.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = bf((p / l[:, None]) @ v)
    L = (m + np.log(l)).astype(np.float32).astype(np.float64)
    p32 = np.exp(s - L[:, None]).astype(np.float32).astype(np.float64)
    dv = bf(p32).T @ do
    D = np.sum(do * o, axis=1)
    dsb = bf(p32 * (do @ v.T - D[:, None]))
    return scale * (dsb @ k), scale * (dsb.T @ q), dv


def main():
    for N, d, causal, scale in [(333, 64, True, None), (1000, 128, True, None), (700, 128, False, None),
                                (200, 64, True, 0.9), (200, 128, True, 0.9), (200, 128, True, -0.3)]:
        w = by_name("gpt2s_causal_bf16_b8h12n1024d64").with_(B=1, H=2, N=N, d=d, causal=causal, seed=77)
        sc = w.softmax_scale if scale is None else scale
        x = make_inputs(w)
        do = bf16_bits_to_f64(make_grad_output(w))
        for h in range(w.H):
            q, k, v = x.f64("q", 0, h), x.f64("k", 0, h), x.f64("v", 0, h)
            ex = backward_head(q, k, v, do[0, h], sc, causal)
            mo = modelled_head(q, k, v, do[0, h], sc, causal)
            rel = [np.linalg.norm(a - b) / np.linalg.norm(b) for a, b in zip(mo, ex)]
            print(f"N={N} d={d} causal={causal} scale={sc:.4g} head {h}: "
                  + " ".join(f"{n} {r:.2e}" for n, r in zip(("dq", "dk", "dv"), rel)))


if __name__ == "__main__":
    main()
