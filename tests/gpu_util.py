"""Helpers shared by the GPU parity tests: move seeded inputs to the device, run
the HIP path through the C ABI binding, and compute oracle references."""

import numpy as np
import torch

from oracle import attention_rows
from workloads import make_inputs
from workloads.gen import AttnInputs

# tolerances stated for this path: bf16 (and the fp32 split path) and fp8
TOL = {
    "bf16": {"max_abs": 2e-2, "rel_l2": 5e-3, "lse_max": 1e-3},
    "f32": {"max_abs": 2e-2, "rel_l2": 5e-3, "lse_max": 1e-3},
    "fp8": {"rel_l2": 5e-2},
}


def to_device(x: AttnInputs):
    dt = x.workload.dtype
    if dt == "f32":
        conv = lambda a: torch.from_numpy(a).cuda()
    elif dt == "bf16":
        conv = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        conv = lambda a: torch.from_numpy(a).cuda().view(torch.float8_e4m3fn)
    return conv(x.q), conv(x.k), conv(x.v)


def run_gpu(x: AttnInputs, stream=None, scale=None):
    import exact_io_aware_48_amd as fa
    w = x.workload
    q, k, v = to_device(x)
    scale = w.softmax_scale if scale is None else scale
    if w.kv_heads != w.H:                         # grouped-query attention
        if w.dtype == "fp8":
            o, lse = fa.fa_fwd_gqa_fp8(q, k, v, *x.descale, scale=scale, causal=w.causal, stream=stream)
        else:
            o, lse = fa.fa_fwd_gqa(q, k, v, scale=scale, causal=w.causal, stream=stream)
    elif w.dtype == "fp8":
        o, lse = fa.fa_fwd_fp8(q, k, v, *x.descale, scale=scale, causal=w.causal, stream=stream)
    else:
        o, lse = fa.fa_fwd(q, k, v, scale=scale, causal=w.causal, stream=stream)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle_full(x: AttnInputs, scale=None):
    w = x.workload
    scale = w.softmax_scale if scale is None else scale
    o = np.empty((w.B, w.H, w.N, w.d))
    l = np.empty((w.B, w.H, w.N))
    for b in range(w.B):
        for h in range(w.H):
            g = h // w.group                         # the K/V head of query head h
            o[b, h], l[b, h] = attention_rows(x.f64("q", b, h), x.f64("k", b, g), x.f64("v", b, g), scale, w.causal)
    return o, l


def oracle_threads():
    """Threads for the float64 oracle: every core in the affinity mask, capped
    by the CPU share the job is granted (OMP_NUM_THREADS when set)."""
    import os
    cores = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    return min(cores, int(share)) if share.isdigit() and int(share) > 0 else cores


def oracle_all(x, scale=None):
    """The float64 oracle over every element of the workload, threaded over
    (batch, head, row chunk)."""
    from oracle import attention_gqa
    w = x.workload
    scale = w.softmax_scale if scale is None else scale
    return attention_gqa(x.f64("q"), x.f64("k"), x.f64("v"), scale, w.causal, threads=oracle_threads())


def sample_rows(N, bc=64, br=128, count=48, seed=0):
    """Query rows worth checking: both ends, tile and row-block edges, and random ones."""
    rng = np.random.default_rng(seed)
    edges = {0, 1, N - 1, N - 2}
    for base in (bc, br):
        for m in range(base, N, base * max(1, N // (base * 6))):
            edges.update({m - 1, m})
    rows = sorted(r for r in edges if 0 <= r < N)
    extra = rng.choice(N, size=min(N, count), replace=False)
    return np.unique(np.concatenate([rows, extra])).astype(np.int64)


def check(errs, dtype, what=""):
    tol = TOL[dtype]
    bad = {k: (errs[k], tol[k]) for k in tol if k in errs and not errs[k] <= tol[k]}
    assert not bad, f"{what}: errors {errs} exceed tolerances {tol}"
