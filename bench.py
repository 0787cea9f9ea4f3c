#!/usr/bin/env python3
"""Benchmark of the FlashAttention forward (and backward) pass on one MI355X.

A step is one call of the C-ABI entry point over one batch of the workload:
the whole hot path (tile scheduling, Q/K/V loads, both MFMA products, online
softmax, masking, normalisation, O and logsumexp stores) runs in that one
kernel launch.  Inputs are seeded synthetic tensors (``workloads``) made
resident in HBM before the timed region.

The K timed steps are K back-to-back launches of the entry point, bracketed by
device synchronisation and one HIP event pair on the launch stream
(``--graph``: captured once into a HIP graph and replayed).

Prints one JSON line.  The headline workload is the largest configuration of
the metric's N = 1K-16K range (B=2, H=8, N=16384, d=256, bf16).  ``value`` is
whole-job throughput in TFLOP/s by the convention 4*B*H*N^2*d (halved for the
causal mask) over the K timed steps on the host clock.  ``roofline.achieved``
is the same FLOP count per launch over the mean launch duration from the HIP
event pair around the timed region (divided by K; it includes whatever gap the
GPU leaves between launches).  ``kernel_ms_p10_p50_p90`` comes from a separate
untimed pass with an event pair around each launch, which itself adds dispatch
latency.  ``traffic`` is the HBM bytes per launch measured with rocprofv3 PMC
counters (FETCH_SIZE + WRITE_SIZE, scaled by the factor the same counters give
for a plain copy of known size), read from profiles/ and only when the kernel
sources are unchanged since that measurement.

``other_workloads`` times every other forward workload the same way and gives
each its own ``roofline`` block.  The bound is the lower of the two ceilings:
MFMA (the dense peak of the type the products use) or HBM at the compulsory
traffic (Q, K, V read once, O and L written once).  An HBM-bound workload's
block is in GB/s of compulsory bytes against 8 TB/s; its TFLOP/s and share of
the dense peak are given beside it.

The line also carries ``backward``: the mean time of one fa_bwd call (its
launches back to back) on the long-context,
grouped-query, GPT-2-small and BERT-large workloads, in TFLOP/s by the usual
convention of 2.5 x the forward's FLOPs.

It also carries ``variants``: ALiBi on the long-context and GPT-2-small
workloads (TFLOP/s by the plain convention) and a block-sparse sliding
window with one global block (TFLOP/s over the allowed query/key pairs,
and the speed-up over the dense kernel).  And ``decode``: one fa_fwd_split call (split kernel and merge) on
the decode workloads (fa_fwd_split_fp8 for the one with an fp8 K/V cache), as
HBM bandwidth over the compulsory bytes (K and V read once) against the 8 TB/s peak.  ``cold``: the GPT-2- and BERT-shaped
forward workloads (whose inputs fit in the 256 MiB MALL) timed with a 512 MiB
device write before every launch, p10/p50/p90 of single launches.  ``gpu``:
the device name, architecture and compute units, and the current clock
levels from the amdgpu kernel driver's sysfs files right after the headline's timed region.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--only-headline]
    python bench.py --backward-only --workload NAME   time only fa_bwd on NAME (for profiling runs)
    python bench.py --copy-calibration ...     also run a 256 MiB device copy (for PMC scaling)
    python bench.py --summarize-pmc DIR_FETCH DIR_WRITE --workload NAME
                                               write profiles/traffic_<NAME>.json from two PMC runs
    python bench.py --summarize-counters DIR... --workload NAME
                                               write profiles/counters_<NAME>.txt from SQ counter passes
    python bench.py --timeline NAME...         per-workgroup phase timeline of one launch (diagnostic build)
    python bench.py --issue-probes             MFMA / FMA / exp / LDS-read issue microbenchmarks (probe library)
"""

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEADLINE = "wide_bf16_b2h8n16384d256"
METRIC = "attention fwd TFLOP/s and % of MI355X dense MFMA peak at N=1K–16K, 1 GPU"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 2516.6, "fp8": 5033.2}   # dense MFMA peaks of the type the products use
HBM_GBPS = 8000.0
# forward workloads whose inputs fit in the 256 MiB MALL: also timed cold
COLD_WORKLOADS = ["gpt2s_causal_bf16_b8h12n1024d64", "bertl_bf16_b16h16n512d64"]
BWD_WORKLOADS = ["long_causal_bf16_b1h32n8192d128", "gqa_causal_bf16_b1h32kv8n8192d128",
                 "gpt2s_causal_bf16_b8h12n1024d64", "bertl_bf16_b16h16n512d64", "wide_bf16_b2h8n16384d256"]
# forward workloads also timed with ALiBi biases
ALIBI_WORKLOADS = ["long_causal_bf16_b1h32n8192d128", "gpt2s_causal_bf16_b8h12n1024d64", "wide_fp8_b2h8n16384d256"]
KERNEL_SOURCES = ["exact_io_aware_48_amd/csrc/fa_common.hpp", "exact_io_aware_48_amd/csrc/fa_tile.hpp",
                  "exact_io_aware_48_amd/csrc/fa_fwd_kernel.hpp", "exact_io_aware_48_amd/csrc/fa_pipe_kernel.hpp",
                  "exact_io_aware_48_amd/csrc/fa_host.hpp", "exact_io_aware_48_amd/csrc/fa_launch.hpp",
                  "exact_io_aware_48_amd/csrc/fa_api.hip", "include/fa_fwd.h"]
# sources of the backward kernels (hashed into the backward trace summaries)
BWD_KERNEL_SOURCES = ["exact_io_aware_48_amd/csrc/fa_common.hpp", "exact_io_aware_48_amd/csrc/fa_host.hpp",
                      "exact_io_aware_48_amd/csrc/fa_bwd_kernel.hpp", "exact_io_aware_48_amd/csrc/fa_bwd_api.hip",
                      "include/fa_bwd.h"]
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash(sources=None):
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload_name):
    path = os.path.join(PROFILES, f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t["hbm_bytes_per_launch"]


# ------------------------------------------------------------------ GPU timing
def device_inputs(w):
    import numpy as np
    import torch
    from workloads import make_inputs
    x = make_inputs(w)
    if w.dtype == "f32":
        conv = lambda a: torch.from_numpy(a).cuda()
    elif w.dtype == "bf16":
        conv = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        conv = lambda a: torch.from_numpy(a).cuda().view(torch.float8_e4m3fn)
    return x, conv(x.q), conv(x.k), conv(x.v)


def time_workload(w, steps, warmup, settle_s=0.25, graph=False):
    """Time exactly `steps` launches of the forward on workload w (see time_launch).

    graph=False (default): `steps` eager launches back to back with one event
    pair on the launch stream around all of them; the per-launch time is that
    pair's time / steps.  A separate untimed pass brackets single launches with
    their own event pairs for the spread (p10/p50/p90).
    graph=True: the `steps` launches are captured once into a HIP graph and the
    timed region is one replay of it; the per-launch time is the replay's event
    time / steps, which includes the gap between dependent kernels.
    """
    import torch
    import exact_io_aware_48_amd as fa
    x, q, k, v = device_inputs(w)
    out_dtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=out_dtype, device="cuda")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    # stream=None: the current stream at call time (the capture stream while capturing)
    gqa = w.kv_heads != w.H
    if w.dtype == "fp8":
        f = fa.fa_fwd_gqa_fp8 if gqa else fa.fa_fwd_fp8
        launch = lambda: f(q, k, v, *x.descale, o=o, lse=lse, scale=w.softmax_scale, causal=w.causal)
    else:
        f = fa.fa_fwd_gqa if gqa else fa.fa_fwd
        launch = lambda: f(q, k, v, o=o, lse=lse, scale=w.softmax_scale, causal=w.causal)
    return time_launch(launch, steps, warmup, settle_s, graph)


def backward_inputs(w):
    """Device tensors for one backward step of workload w (bf16): q, k, v, the
    forward's o and lse (computed here by fa_fwd_gqa), dO, the float32
    gradient outputs and the statistics workspace."""
    import numpy as np
    import torch
    import exact_io_aware_48_amd as fa
    from workloads import make_grad_output
    _, q, k, v = device_inputs(w)
    do = torch.from_numpy(make_grad_output(w).view(np.int16)).cuda().view(torch.bfloat16)
    o, lse = fa.fa_fwd_gqa(q, k, v, scale=w.softmax_scale, causal=w.causal)
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.H, w.kv_heads, w.N, w.d), dtype=torch.uint8, device="cuda")
    return q, k, v, o, lse, do, dq, dk, dv, ws


def time_backward(w, steps, warmup, settle_s=0.25, graph=False):
    """Time exactly `steps` calls of fa_bwd (dQ with the statistics, then dK/dV) on workload w."""
    import exact_io_aware_48_amd as fa
    q, k, v, o, lse, do, dq, dk, dv, ws = backward_inputs(w)
    launch = lambda: fa.fa_bwd(q, k, v, o, do, lse, scale=w.softmax_scale, causal=w.causal, dq=dq, dk=dk, dv=dv,
                               workspace=ws)
    return time_launch(launch, steps, warmup, settle_s, graph)


def time_decode(w, steps, warmup, settle_s=0.25, graph=False):
    """Time exactly `steps` calls of fa_fwd_split, or fa_fwd_split_fp8 on fp8 inputs (split
    kernel + merge), on decode workload w."""
    import torch
    import exact_io_aware_48_amd as fa
    x, q, k, v = device_inputs(w)
    fp8 = w.dtype == "fp8"
    splits, nbytes = fa.fa_fwd_split_plan(w.B, w.H, w.kv_heads, w.q_rows, w.N, w.d, 0, fp8=fp8)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, w.q_rows), dtype=torch.float32, device="cuda")
    if fp8:
        launch = lambda: fa.fa_fwd_split_fp8(q, k, v, *x.descale, scale=w.softmax_scale, causal=w.causal, o=o,
                                             lse=lse, workspace=ws)
    else:
        launch = lambda: fa.fa_fwd_split(q, k, v, scale=w.softmax_scale, causal=w.causal, o=o, lse=lse,
                                         workspace=ws)
    t = time_launch(launch, steps, warmup, settle_s, graph)
    t["splits"] = splits
    return t


def alibi_slopes(H):
    """The geometric slopes 2^(-8 (h + 1) / H) of the ALiBi paper."""
    return [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]


def time_alibi(w, steps, warmup, settle_s=0.25, graph=False):
    import torch
    import exact_io_aware_48_amd as fa
    x, q, k, v = device_inputs(w)
    slopes = torch.tensor(alibi_slopes(w.H), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    if w.dtype == "fp8":
        o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
        launch = lambda: fa.fa_fwd_alibi_fp8(q, k, v, slopes, *x.descale, o=o, lse=lse, scale=w.softmax_scale,
                                             causal=w.causal)
    else:
        o = torch.empty_like(q)
        launch = lambda: fa.fa_fwd_alibi(q, k, v, slopes, o=o, lse=lse, scale=w.softmax_scale, causal=w.causal)
    return time_launch(launch, steps, warmup, settle_s, graph)


def local_global_mask(N, window=1):
    """Block mask [nb, nb]: each query block sees its neighbours within `window`
    blocks and the first block (a sliding window with one global block)."""
    import numpy as np
    nb = (N + 127) // 128
    m = np.zeros((nb, nb), dtype=np.uint8)
    for i in range(nb):
        m[i, max(0, i - window):i + window + 1] = 1
        m[i, 0] = 1
    return m


def blocksparse_flops(w, bm):
    """4*d per allowed (query, key) pair, counted per block pair (ragged edges, causal)."""
    nb = bm.shape[-1]
    size = lambda i: min(128, w.N - 128 * i)
    pairs = 0
    for i in range(nb):
        for j in range(nb):
            if not bm[i, j] or (w.causal and j > i):
                continue
            r, c = size(i), size(j)
            pairs += r * (r + 1) // 2 if (w.causal and i == j) else r * c
    return 4.0 * w.d * pairs * w.B * w.H


def time_blocksparse(w, bm, steps, warmup, settle_s=0.25, graph=False):
    import torch
    import exact_io_aware_48_amd as fa
    _, q, k, v = device_inputs(w)
    m = torch.from_numpy(bm).cuda()
    o, lse = torch.empty_like(q), torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    launch = lambda: fa.fa_fwd_blocksparse(q, k, v, m, o=o, lse=lse, scale=w.softmax_scale, causal=w.causal)
    return time_launch(launch, steps, warmup, settle_s, graph)


def backward_flops(w):
    """Backward matmul FLOPs by the usual convention: 2.5 x the forward's (five
    N x N x d products against the forward's two)."""
    return 2.5 * w.flops


MIN_TIMED_MS = 200.0       # each timed region covers at least this long (auto step counts)
AUTO_STEPS = (20, 5000)    # bounds of an automatic step count


def time_launch(launch, steps, warmup, settle_s=0.25, graph=False):
    """steps=None: as many steps as fill MIN_TIMED_MS, from the mean of the
    last settling round (within AUTO_STEPS)."""
    import torch
    # untimed: let the clocks settle on this very step, then the W warmup steps
    torch.cuda.synchronize()
    t_end = time.perf_counter() + settle_s
    round_ms = None
    while True:
        r0 = time.perf_counter()
        for _ in range(8):
            launch()
        torch.cuda.synchronize()
        round_ms = (time.perf_counter() - r0) * 1e3 / 8
        if time.perf_counter() >= t_end:
            break
    if steps is None:
        steps = int(min(AUTO_STEPS[1], max(AUTO_STEPS[0], math.ceil(MIN_TIMED_MS / max(round_ms, 1e-3)))))
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                launch()
        g.replay()                      # untimed: the first replay uploads the graph
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        per = a.elapsed_time(b) / steps
        return {"wall_ms_per_step": (t1 - t0) * 1e3 / steps, "kernel_ms_mean": per, "kernel_ms_median": per,
                "kernel_ms_p10": None, "kernel_ms_p90": None, "steps": steps,
                "timing": f"one HIP graph replay of {steps} launches"}
    # the timed region: exactly `steps` back-to-back launches, one event pair on
    # the launch stream around them and the host clock outside
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        launch()
    b.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    mean = a.elapsed_time(b) / steps
    # untimed: the spread of single launches, each bracketed by its own event pair
    # (the pairs add dispatch latency between launches, so they time only the spread)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(steps, 50))]
    for x, y in ev:
        x.record(stream)
        launch()
        y.record(stream)
    torch.cuda.synchronize()
    kms = sorted(x.elapsed_time(y) for x, y in ev)
    return {
        "wall_ms_per_step": (t1 - t0) * 1e3 / steps,
        "kernel_ms_mean": mean,
        "kernel_ms_median": kms[len(kms) // 2],
        "kernel_ms_p10": kms[len(kms) // 10],
        "kernel_ms_p90": kms[(9 * len(kms)) // 10],
        "steps": steps,
        "timing": "eager back-to-back launches, one event pair around the timed region; "
                  "p10/p50/p90 from a separate untimed pass with an event pair around each launch",
    }


def time_cold(w, iters=30, scratch_bytes=512 * 2**20):
    """Cold-cache series: before each launch a 512 MiB scratch write evicts the
    L2s and the 256 MiB MALL (the GPT-2- and BERT-shaped inputs fit in the
    MALL), then one event pair on the launch stream times the launch alone."""
    import torch
    import exact_io_aware_48_amd as fa
    x, q, k, v = device_inputs(w)
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    f = fa.fa_fwd_gqa if w.kv_heads != w.H else fa.fa_fwd
    launch = lambda: f(q, k, v, o=o, lse=lse, scale=w.softmax_scale, causal=w.causal)
    scratch = torch.empty(scratch_bytes // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):                  # untimed warmup
        scratch.fill_(0.0)
        launch()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i, (a, b) in enumerate(ev):
        scratch.fill_(float(i))
        a.record(stream)
        launch()
        b.record(stream)
    torch.cuda.synchronize()
    kms = sorted(a.elapsed_time(b) for a, b in ev)
    med = kms[len(kms) // 2]
    return {"kernel_ms_p10_p50_p90": [round(kms[len(kms) // 10], 5), round(med, 5), round(kms[(9 * len(kms)) // 10], 5)],
            "tflops_at_median": round(w.flops / (med * 1e-3) / 1e12, 1),
            "iterations": iters, "eviction": f"{scratch_bytes >> 20} MiB device write before each launch"}


def read_clocks(kinds=("sclk", "mclk")):
    """Current clock levels from the amdgpu kernel driver's sysfs files
    (pp_dpm_sclk / pp_dpm_mclk of each card it exposes).  Plain file reads:
    nothing is spawned from this GPU-initialised process."""
    clocks = {}
    for kind in kinds:
        for path in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{kind}"))[:8]:
            try:
                with open(path) as f:
                    levels = f.read().splitlines()
            except OSError:
                continue
            cur = [ln.split(":", 1)[-1].replace("*", "").strip() for ln in levels if ln.rstrip().endswith("*")]
            clocks[f"{path.split('/')[4]}/{kind}"] = cur[0] if cur else None
    return clocks if clocks else "no readable /sys/class/drm/card*/device/pp_dpm_sclk"


def gpu_info():
    """The GPU model (from the runtime) and the current clock levels, read
    right after the headline's timed region."""
    import torch
    pr = torch.cuda.get_device_properties(0)
    info = {"name": pr.name, "arch": getattr(pr, "gcnArchName", None), "compute_units": pr.multi_processor_count,
            "memory_gib": round(pr.total_memory / 2**30, 1)}
    info["clocks"] = read_clocks()
    return info


def copy_calibration(nbytes=256 * 2**20, reps=3):
    """A plain device copy of known size, so PMC byte counters can be scaled."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ CPU oracle baseline
def cpu_share():
    """The CPU threads this job may use: every core in the affinity mask, capped
    by the CPU share the scheduler grants the job (OMP_NUM_THREADS when set;
    one GPU's share on the GPU hosts)."""
    cores = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS")
    if share and share.isdigit() and int(share) > 0:
        cores = min(cores, int(share))
    return cores


def blas_name():
    import numpy as np
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:
        return "unknown"


def cpu_baseline(w, min_seconds=10.0, max_seconds=30.0):
    """The float64 oracle, as it stands, on a bounded sample of the workload:
    whole heads (every query row against every key), one head after another in
    the workload's order, until ``min_seconds`` of wall time have passed or the
    workload is exhausted; TFLOP/s over the sample's own FLOPs."""
    from oracle import attention_naive
    from workloads import make_inputs
    x = make_inputs(w)
    threads = cpu_share()
    import numpy as np
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    head_flops = w.flops / len(heads)
    # heads per oracle call: enough 1024-row chunks to keep every thread busy
    per_call = max(1, math.ceil(2 * threads * 1024 / w.N))
    done, t0 = 0, time.perf_counter()
    for i in range(0, len(heads), per_call):
        chunk = heads[i:i + per_call]
        stack = lambda which, kv: np.stack([x.f64(which, b, h // w.group if kv else h) for b, h in chunk])[None]
        attention_naive(stack("q", False), stack("k", True), stack("v", True), w.softmax_scale, w.causal,
                        threads=threads)
        done += len(chunk)
        el = time.perf_counter() - t0
        if el >= min_seconds or el + el * len(chunk) / done > max_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done * head_flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "blas": blas_name(),
            "sample": f"{done} of the {len(heads)} heads of the workload (N={w.N}, d={w.d}, "
                      f"{'causal' if w.causal else 'full'}, every row of each), float64 numpy oracle on "
                      f"{threads} threads, {dt:.2f} s wall; FLOPs by the same convention as value"}


# ------------------------------------------------------------------ PMC summary
def is_forward_kernel(name):
    """The forward attention kernels (fa_fwd_kernel and the software-pipelined fa_fwd_pipe_kernel)."""
    return "fa_fwd_kernel" in name or "fa_fwd_pipe_kernel" in name


def _read_counter_csv(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    rows = []
    for fn in files:
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    return rows


def summarize_pmc(dir_fetch, dir_write, workload_name, command=""):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the attention kernel, scaled by a copy kernel."""
    from workloads import by_name
    w = by_name(workload_name)
    out = {}
    for counter, d in (("FETCH_SIZE", dir_fetch), ("WRITE_SIZE", dir_write)):
        rows = [r for r in _read_counter_csv(d) if r.get("Counter_Name") == counter]
        fa_vals = [float(r["Counter_Value"]) for r in rows if is_forward_kernel(r["Kernel_Name"])]
        cp_vals = [float(r["Counter_Value"]) for r in rows if not is_forward_kernel(r["Kernel_Name"])
                   and "opy" in r["Kernel_Name"]]
        if not fa_vals:
            raise SystemExit(f"no forward-kernel dispatch with {counter} in {d}")
        copy_kib = max(cp_vals) if cp_vals else None
        out[counter] = {"kib_per_dispatch_mean": sum(fa_vals) / len(fa_vals), "dispatches": len(fa_vals),
                        "copy_kib": copy_kib}
    known_kib = 256 * 1024.0                  # the calibration copy reads and writes 256 MiB
    f_fetch = known_kib / out["FETCH_SIZE"]["copy_kib"] if out["FETCH_SIZE"]["copy_kib"] else 1.0
    f_write = known_kib / out["WRITE_SIZE"]["copy_kib"] if out["WRITE_SIZE"]["copy_kib"] else 1.0
    fetch_b = out["FETCH_SIZE"]["kib_per_dispatch_mean"] * 1024 * f_fetch
    write_b = out["WRITE_SIZE"]["kib_per_dispatch_mean"] * 1024 * f_write
    res = {
        "workload": workload_name,
        "kernel_source_sha": kernel_source_hash(),
        "fetch_kib_per_dispatch": out["FETCH_SIZE"]["kib_per_dispatch_mean"],
        "write_kib_per_dispatch": out["WRITE_SIZE"]["kib_per_dispatch_mean"],
        "copy_scale_fetch": f_fetch,
        "copy_scale_write": f_write,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "compulsory_bytes": w.compulsory_bytes,
        "traffic_over_compulsory": (fetch_b + write_b) / w.compulsory_bytes,
        "command": command,
    }
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"traffic_{workload_name}.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


# per-instruction FLOPs of the MFMAs the forward issues (32x32x16 bf16, 32x32x64 fp8)
MFMA_FLOPS = {"bf16": 2 * 32 * 32 * 16, "fp8": 2 * 32 * 32 * 64}
SIMDS = 256 * 4
SPEC_CLOCK_GHZ = 2.4


def summarize_counters(dirs, workload_name, command=""):
    """SQ counters of the forward kernel (one rocprofv3 --pmc pass per
    directory), averaged over its dispatches, with derived ratios: instructions
    per MFMA, LDS bank conflicts per LDS instruction, and the MFMA busy
    fraction over all SIMDs for the kernel's mean duration in
    profiles/kernel_trace_<workload>.txt at the 2.4 GHz spec clock."""
    from workloads import by_name
    w = by_name(workload_name)
    vals = {}
    for d in dirs:
        for r in _read_counter_csv(d):
            if is_forward_kernel(r["Kernel_Name"]):
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no forward-kernel dispatch in {dirs}")
    mean = {k: sum(v) / len(v) for k, v in sorted(vals.items())}
    lines = [f"# SQ counters of the forward kernel: {workload_name}", "",
             f"command (one pass per counter set): {command}",
             f"kernel sources sha: {kernel_source_hash()}", "",
             "counter                          dispatches   mean per dispatch"]
    lines += [f"{k:32s} {len(vals[k]):10d}   {mean[k]:18.1f}" for k in mean]
    mf = mean.get("SQ_INSTS_MFMA")
    derived = []
    if mf:
        for k, label in (("SQ_INSTS_VALU", "VALU instructions per MFMA (the count includes the MFMAs)"),
                         ("SQ_INSTS_VALU_TRANS_F32", "transcendental (exp) instructions per MFMA"),
                         ("SQ_INSTS_LDS", "LDS instructions per MFMA"),
                         ("SQ_INSTS_SALU", "scalar instructions per MFMA")):
            if k in mean:
                derived.append(f"{label}: {mean[k] / mf:.2f}")
        flops = mf * MFMA_FLOPS["fp8" if w.dtype == "fp8" else "bf16"]
        derived.append(f"MFMA FLOPs counted / FLOPs by the metric convention: {flops / w.flops:.3f}")
    if "SQ_LDS_BANK_CONFLICT" in mean and mean.get("SQ_INSTS_LDS"):
        derived.append(f"LDS bank conflict cycles per LDS instruction: {mean['SQ_LDS_BANK_CONFLICT'] / mean['SQ_INSTS_LDS']:.4f}")
    trace = os.path.join(PROFILES, f"kernel_trace_{workload_name}.txt")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and os.path.exists(trace):
        with open(trace) as f:
            row = next((ln for ln in f if ln.startswith("fa::fa_fwd_kernel") or ln.startswith("fa::fa_fwd_pipe_kernel")),
                       None)
        if row:
            avg_us = float(row.split()[-4])
            busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * avg_us * 1e3 * SPEC_CLOCK_GHZ)
            derived.append(f"MFMA busy fraction over {SIMDS} SIMDs at {SPEC_CLOCK_GHZ} GHz for the traced mean "
                           f"duration {avg_us:.2f} us: {busy:.3f}")
    lines += ["", "derived:"] + [f"- {d}" for d in derived]
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"counters_{workload_name}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(trace_dir, workload_name, command, prefix="kernel_trace"):
    """Write profiles/<prefix>_<workload>.txt from a rocprofv3 --kernel-trace --stats run."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {trace_dir}")
    rows = []
    for fn in files:
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    backward = prefix.startswith("kernel_trace_backward")
    lines = [f"rocprofv3 kernel statistics: {workload_name}",
             f"command: {command}",
             (f"backward kernel sources sha: {kernel_source_hash(BWD_KERNEL_SOURCES)}" if backward else
              f"kernel sources sha: {kernel_source_hash()}"),
             "",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'share%':>7s}"]
    for r in rows:
        name = r["Name"].replace("void ", "")[:60]
        lines.append(f"{name:60s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.2f} "
                     f"{float(r['MinNs'])/1e3:10.2f} {float(r['MaxNs'])/1e3:10.2f} {float(r['Percentage']):7.2f}")
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"{prefix}_{workload_name}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ------------------------------------------------------------------ main
def roofline_block(w, t):
    """The roofline of one forward workload from its mean launch time.

    Ceilings: the dense MFMA peak of the type the products use, and HBM at
    the compulsory traffic (AI * 8 TB/s, AI = metric FLOPs / compulsory
    bytes).  Whichever is lower bounds the kernel: an MFMA-bound block is in
    TFLOP/s against the peak, an HBM-bound one in GB/s of compulsory bytes
    against 8 TB/s."""
    peak = PEAK_TFLOPS[w.dtype]
    sec = t["kernel_ms_mean"] * 1e-3
    tflops = w.flops / sec / 1e12
    ai = w.flops / w.compulsory_bytes
    hbm_ceiling = ai * HBM_GBPS / 1e3
    common = {"traffic": traffic_for(w.name), "kernel_ms_mean": round(t["kernel_ms_mean"], 5),
              "tflops": round(tflops, 1), "pct_of_dense_peak": round(100 * tflops / peak, 2),
              "arith_intensity_flop_per_compulsory_byte": round(ai, 1),
              "ceilings_tflops": {"mfma": peak, "hbm": round(hbm_ceiling, 1)}}
    if hbm_ceiling < peak:
        gbs = w.compulsory_bytes / sec / 1e9
        blk = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_GBPS, "unit": "GB/s",
               "frac": round(gbs / HBM_GBPS, 4), "algorithmic_bytes_per_launch": w.compulsory_bytes}
    else:
        blk = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
               "frac": round(tflops / peak, 4), "algorithmic_flops_per_launch": w.flops}
    blk.update(common)
    return blk


# ------------------------------------------------------------------ issue probes
ROLE_PROBES = [(1, "MFMA waves only (8 MFMA per iteration)"), (2, "FMA waves only (64 FMA per iteration)"),
               (3, "MFMA waves + FMA waves"), (6, "exp waves only (64 exp per iteration)"),
               (7, "MFMA waves + exp waves")]


def issue_probes(iters=2000, reps=40, settle_launches=400):
    """Run the issue-rate microbenchmarks of libfa_probe.so (csrc/fa_issue_probe.hip)
    and return their table as text lines: per configuration the launch time, the
    time per wave-iteration, for mixed work the sum of its parts timed alone at
    the same waves per SIMD, and the sclk level right after it.  A settling run
    (about 0.2 s of the MFMA + exp mix) comes first, so that the first rows do
    not meet a clock still ramping up from idle."""
    import ctypes
    import torch
    from exact_io_aware_48_amd import _lib
    lib = _lib.load_probe()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    ms = ctypes.c_float()

    def run(fn, i):
        st = fn(i, out.data_ptr(), out.numel(), iters, reps, ctypes.byref(ms))
        if st != 0:
            raise RuntimeError(f"probe {i}: status {st}")
        return ms.value

    if lib.fa_probe_mixed(4, out.data_ptr(), out.numel(), iters, settle_launches, ctypes.byref(ms)) != 0:
        raise RuntimeError("probe settling run failed")

    def sclk():
        c = read_clocks(("sclk",))
        return ", ".join(f"{v}" for v in c.values()) if isinstance(c, dict) else "?"

    rows, alone = [], {}
    for i in range(lib.fa_probe_mixed_count()):
        wk = (ctypes.c_int * 5)()
        lib.fa_probe_mixed_work(i, wk)
        wps, mf, fma, ex, lds = list(wk)
        t = run(lib.fa_probe_mixed, i)
        if (mf > 0) + (fma > 0) + (ex > 0) + (lds > 0) == 1:
            alone[(wps, mf, fma, ex, lds)] = t
        # mixed work without LDS reads: the sum of its MFMA, FMA and exp parts where each was timed alone
        parts = [alone.get(key) for n, key in ((mf, (wps, mf, 0, 0, 0)), (fma, (wps, 0, fma, 0, 0)),
                                               (ex, (wps, 0, 0, ex, 0))) if n]
        summed = len(parts) > 1 and lds == 0 and None not in parts
        rows.append(f"{lib.fa_probe_mixed_name(i).decode():58s} {t:8.3f} ms  {t * 1e6 / iters:7.1f} ns/iter"
                    + f"  sclk {sclk():>8s}" + (f"  parts alone {sum(parts):.3f} ms" if summed else ""))
    for role, name in ROLE_PROBES:
        t = run(lib.fa_probe_roles, role)
        rows.append(f"{'split roles: ' + name:58s} {t:8.3f} ms  {t * 1e6 / iters:7.1f} ns/iter  sclk {sclk():>8s}")
    return [f"issue probes: {cus} workgroups (one per CU), {iters} iterations, mean of {reps} launches after "
            f"{reps // 2 + 1} warm-up launches, following a {settle_launches}-launch settling run", ""] + rows


# ------------------------------------------------------------------ timeline
def timeline_summary(w, lib, launches=200):
    """Per-workgroup phases of one forward launch on workload w, from the
    diagnostic timeline build (fa_timeline_read): where the time goes between
    the workgroups' Q/first-tile loads, main loops and O stores, how the work
    spreads over CUs and XCDs, and how workgroups that share a CU progress.
    Times in microseconds (100 MHz s_memrealtime stamps)."""
    import collections
    import ctypes
    import numpy as np
    import torch
    x, q, k, v = device_inputs(w)
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, o, lse)]
    code = {"f32": 0, "bf16": 1, "fp8": 2}[w.dtype]
    if w.dtype == "fp8":
        call = lambda: lib.fa_fwd_gqa_fp8(*ptrs, w.B, w.H, w.kv_heads, w.N, w.d, w.softmax_scale, *x.descale,
                                          int(w.causal), s)
    else:
        call = lambda: lib.fa_fwd_gqa(*ptrs, w.B, w.H, w.kv_heads, w.N, w.d, w.softmax_scale, int(w.causal), code, s)
    for _ in range(launches):                 # warm caches and clocks; the last launch is the one read
        assert call() == 0
    torch.cuda.synchronize()
    grid = ctypes.c_int64()
    i32 = ctypes.c_int
    assert lib.fa_plan(w.B, w.H, w.N, w.d, int(w.causal), code, ctypes.byref(i32()), ctypes.byref(i32()),
                       ctypes.byref(grid), ctypes.byref(i32()), ctypes.byref(i32()), ctypes.byref(ctypes.c_int64())) == 0
    nwg = grid.value
    buf = np.zeros(nwg * 6, dtype=np.uint64)
    assert lib.fa_timeline_read(buf.ctypes.data, buf.nbytes) == 0
    t = buf.reshape(nwg, 6).astype(np.int64)
    t0 = t[:, 0].min()
    st, pro, lp, en = ((t[:, i] - t0) / 100.0 for i in range(4))
    hw, xcc = t[:, 4] & 0xFFFFFFFF, t[:, 4] >> 32
    cu_key = list(zip(xcc.tolist(), ((hw >> 13) & 7).tolist(), ((hw >> 12) & 1).tolist(), ((hw >> 8) & 15).tolist()))
    pct = lambda a: [round(float(v), 2) for v in np.percentile(a, [0, 10, 50, 90, 100])]
    cus = collections.defaultdict(list)
    for i, key in enumerate(cu_key):
        cus[key].append(i)
    gaps, rank = [], np.zeros(nwg, dtype=int)
    for ids in cus.values():
        ids.sort(key=lambda i: st[i])
        for r, i in enumerate(ids):
            rank[i] = r
        # idle time between a workgroup's end and the start of the next on
        # the CU (only where they ran one after another)
        gaps += [st[b] - en[a] for a, b in zip(ids, ids[1:]) if st[b] >= en[a]]
    loop = lp - pro
    per_cu_loop = np.array([loop[ids].sum() for ids in cus.values()])
    per_cu_end = np.array([en[ids].max() for ids in cus.values()])
    xcds = {}
    for xc in sorted(set(xcc.tolist())):
        keys = [k for k in cus if k[0] == xc]
        ids = np.array([i for k in keys for i in cus[k]])
        xcds[int(xc)] = {"loop_sum_per_cu_mean": round(float(np.mean([loop[cus[k]].sum() for k in keys])), 2),
                         "last_end": round(float(max(en[cus[k]].max() for k in keys)), 2),
                         # main-loop median by start rank: whether an XCD's pace changes once others finish
                         "loop_p50_by_rank": [round(float(np.median(loop[ids[rank[ids] == r]])), 2)
                                              for r in range(rank[ids].max() + 1)]}
    return {
        "workload": w.name, "workgroups": int(nwg), "span_us": round(float(en.max()), 2),
        "percentiles": "p0 p10 p50 p90 p100",
        "start_offset": pct(st), "prologue": pct(pro - st), "main_loop": pct(loop), "o_store": pct(en - lp),
        "end": pct(en),
        "cus": len(cus), "workgroups_per_cu": dict(collections.Counter(len(v) for v in cus.values())),
        "loop_sum_per_cu": pct(per_cu_loop), "last_end_per_cu": pct(per_cu_end),
        "gap_between_sequential_workgroups_on_a_cu": pct(np.array(gaps)) if gaps else None,
        "by_start_rank_on_cu": {int(r): {"main_loop_p50": round(float(np.median(loop[rank == r])), 2),
                                         "end_p50": round(float(np.median(en[rank == r])), 2)}
                                for r in range(rank.max() + 1)},
        "xcd": xcds,
    }



def summarize_timelines(path, command="", out=None):
    """Write profiles/timeline_forward_workloads.txt from the JSON lines of
    ``bench.py --timeline`` (one per workload)."""
    lines = ["Per-workgroup timelines of one forward launch per workload (diagnostic build, "
             "s_memrealtime at 100 MHz; microseconds)",
             f"command: {command}", f"kernel sources sha: {kernel_source_hash()}",
             "phases per workgroup: start offset (dispatch), prologue (Q and first K/V tiles), main loop, "
             "O store (incl. a workgroup barrier); percentiles p0 p10 p50 p90 p100"]
    with open(path) as f:
        recs = [json.loads(ln) for ln in f if ln.startswith("{")]
    if not recs:
        raise SystemExit(f"no timeline record in {path}")
    for r in recs:
        wpc = {str(k): v for k, v in r["workgroups_per_cu"].items()}
        lines += ["", f"== {r['workload']}: {r['workgroups']} workgroups on {r['cus']} CUs {wpc}, span {r['span_us']}"]
        for k in ("start_offset", "prologue", "main_loop", "o_store", "end", "loop_sum_per_cu", "last_end_per_cu"):
            lines.append(f"  {k:34s} {r[k]}")
        gap = r.get("gap_between_sequential_workgroups_on_a_cu")
        lines.append("  gap_between_sequential_workgroups_on_a_cu "
                     + (str(gap) if gap else "  (none: the CU's workgroups ran side by side)"))
        lines.append("  by start rank on a CU: " + ", ".join(
            f"{k}: loop {v['main_loop_p50']} end {v['end_p50']}" for k, v in r["by_start_rank_on_cu"].items()))
        lines.append("  per XCD (loop sum per CU mean / last end): " + ", ".join(
            f"{k}: {v['loop_sum_per_cu_mean']}/{v['last_end']}" for k, v in r["xcd"].items()))
        if all("loop_p50_by_rank" in v for v in r["xcd"].values()):
            lines.append("  per XCD main loop p50 by start rank on a CU: " + ", ".join(
                f"{k}: {v['loop_p50_by_rank']}" for k, v in r["xcd"].items()))
    out = out or os.path.join(PROFILES, "timeline_forward_workloads.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60,
                    help="timed launches of the headline workload (the default covers about 0.2 s)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true", help="skip timing the other workloads")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--settle", type=float, default=0.25, help="seconds of untimed clock-settling steps")
    ap.add_argument("--graph", action="store_true",
                    help="time one HIP graph replay of the K launches instead of eager launches")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward workloads")
    ap.add_argument("--no-decode", action="store_true", help="skip timing the split-KV decode workloads")
    ap.add_argument("--no-variants", action="store_true", help="skip timing the ALiBi and block-sparse variants")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache series")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only fa_bwd on --workload and print its line (for profiling runs)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="write profiles/counters_<NAME>.txt from rocprofv3 --pmc passes over --workload")
    ap.add_argument("--summarize-timelines", metavar="JSONL",
                    help="write profiles/timeline_forward_workloads.txt from the output of --timeline")
    ap.add_argument("--command", default="", help="the profiling command, recorded in the summary")
    ap.add_argument("--summary-prefix", default="kernel_trace", help="file name prefix of --summarize-trace")
    ap.add_argument("--timeline", nargs="+", metavar="NAME",
                    help="per-workgroup phase timeline of one forward launch of each workload, from the "
                         "diagnostic build (python -m exact_io_aware_48_amd.build --timeline); one JSON line each")
    ap.add_argument("--issue-probes", action="store_true",
                    help="the issue-rate microbenchmarks (python -m exact_io_aware_48_amd.build --probes): MFMA, "
                         "FMA, exp and LDS reads in one wave or in different waves; writes profiles/issue_probes.txt")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, args.command)
        return 0
    if args.summarize_timelines:
        summarize_timelines(args.summarize_timelines, args.command)
        return 0
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload, args.command)
        return 0
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.workload, args.command, args.summary_prefix)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this benchmark runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the attention forward shards over (batch, head) with no communication, so N GPUs would run "
              "N independent copies of this kernel on 1/N of the heads", file=sys.stderr)
        return 2

    import torch
    from workloads import WORKLOADS, by_name
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.issue_probes:
        lines = issue_probes()
        lines.insert(1, "command: python bench.py --issue-probes")
        os.makedirs(PROFILES, exist_ok=True)
        with open(os.path.join(PROFILES, "issue_probes.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines), flush=True)
        return 0
    if args.timeline:
        from exact_io_aware_48_amd import _lib
        tl = _lib.load_timeline()
        for name in args.timeline:
            print(json.dumps(timeline_summary(by_name(name), tl)), flush=True)
        return 0

    w = by_name(args.workload)
    if args.copy_calibration:
        copy_calibration()
    if args.backward_only:
        bt = time_backward(w, args.steps, args.warmup, args.settle, graph=args.graph)
        print(json.dumps({"backward": w.name, "ms_per_call": round(bt["kernel_ms_mean"], 5),
                          "tflops_2p5x_convention": round(backward_flops(w) / (bt["kernel_ms_mean"] * 1e-3) / 1e12, 1),
                          "timing": bt["timing"]}), flush=True)
        return 0
    t = time_workload(w, args.steps, args.warmup, args.settle, graph=args.graph)
    gpu = gpu_info()                    # clocks as the headline's timed region left them
    peak = PEAK_TFLOPS[w.dtype]
    value = w.flops / (t["wall_ms_per_step"] * 1e-3) / 1e12
    roof = roofline_block(w, t)
    roof["kernel_ms_p10_p50_p90"] = None if t["kernel_ms_p10"] is None else \
        [round(t["kernel_ms_p10"], 5), round(t["kernel_ms_median"], 5), round(t["kernel_ms_p90"], 5)]
    roof["timing"] = t["timing"]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["wall_ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1) Q/K/V, resident in HBM before timing",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "scale": w.softmax_scale, "parallelism": "single GPU"},
        "pct_of_dense_peak": round(100 * value / peak, 2),
        "roofline": roof,
        "sclk_after": read_clocks(("sclk",)),
    }
    if not args.only_headline:
        others = {}
        for ow in WORKLOADS:
            if ow.name == w.name:
                continue
            ot = time_workload(ow, None, max(3, args.warmup // 2), args.settle,
                               graph=args.graph)
            rb = roofline_block(ow, ot)
            others[ow.name] = {"tflops_kernel": rb["tflops"], "pct_of_dense_peak": rb["pct_of_dense_peak"],
                               "kernel_ms_mean": rb["kernel_ms_mean"],
                               "kernel_ms_p50_single_launch": round(ot["kernel_ms_median"], 5),
                               "steps": ot["steps"], "dtype": ow.dtype, "roofline": rb,
                               "sclk_after": read_clocks(("sclk",))}
        line["other_workloads"] = others
    if not args.no_cold and not args.only_headline:
        line["cold"] = {name: time_cold(by_name(name)) for name in COLD_WORKLOADS}
    if not args.no_backward:
        bwd = {}
        for name in BWD_WORKLOADS:
            bw = by_name(name)
            bt = time_backward(bw, None, max(3, args.warmup // 2), args.settle, graph=args.graph)
            tf = backward_flops(bw) / (bt["kernel_ms_mean"] * 1e-3) / 1e12
            bwd[name] = {"ms_per_call": round(bt["kernel_ms_mean"], 4), "tflops": round(tf, 1), "steps": bt["steps"],
                         "pct_of_dense_peak": round(100 * tf / PEAK_TFLOPS["bf16"], 2),
                         "flops": "2.5 x forward (five N x N x d products)",
                         "launches": "dQ (with the statistics), dK/dV (+ reduction for split grouped heads)"}
        line["backward"] = bwd
    if not args.no_variants:
        var = {}
        for name in ALIBI_WORKLOADS:
            vw = by_name(name)
            at = time_alibi(vw, None, max(3, args.warmup // 2), args.settle, graph=args.graph)
            tf = vw.flops / (at["kernel_ms_mean"] * 1e-3) / 1e12
            var["alibi:" + name] = {"ms_per_call": round(at["kernel_ms_mean"], 4), "tflops": round(tf, 1),
                                    "pct_of_dense_peak": round(100 * tf / PEAK_TFLOPS[vw.dtype], 2)}
        sw = by_name("long_causal_bf16_b1h32n8192d128").with_(causal=False)
        bm = local_global_mask(sw.N)
        bt = time_blocksparse(sw, bm, None, max(3, args.warmup // 2), args.settle,
                              graph=args.graph)
        dt = time_workload(sw, None, max(3, args.warmup // 2), args.settle, graph=args.graph)
        tf = blocksparse_flops(sw, bm) / (bt["kernel_ms_mean"] * 1e-3) / 1e12
        var["blocksparse:local_global_b1h32n8192d128"] = {
            "ms_per_call": round(bt["kernel_ms_mean"], 4), "tflops_effective": round(tf, 1),
            "pct_of_dense_peak": round(100 * tf / PEAK_TFLOPS["bf16"], 2),
            "density": round(float(bm.mean()), 4), "dense_ms": round(dt["kernel_ms_mean"], 4),
            "speedup_vs_dense": round(dt["kernel_ms_mean"] / bt["kernel_ms_mean"], 2),
            "pattern": "each 128-query block sees its neighbours (window 1) and the first key block; non-causal"}
        line["variants"] = var
    if not args.no_decode:
        from workloads import DECODE_WORKLOADS
        dec = {}
        for dw in DECODE_WORKLOADS:
            dt = time_decode(dw, None, max(5, args.warmup), args.settle, graph=args.graph)
            gbs = dw.compulsory_bytes / (dt["kernel_ms_mean"] * 1e-3) / 1e9
            dec[dw.name] = {"us_per_call": round(dt["kernel_ms_mean"] * 1e3, 1), "splits": dt["splits"], "dtype": dw.dtype,
                            "hbm_gbs": round(gbs, 0), "frac_of_hbm_peak": round(gbs / HBM_GBPS, 4),
                            "compulsory_bytes": dw.compulsory_bytes,
                            "launches": "split kernel, merge"}
        line["decode"] = dec
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    line["gpu"] = gpu
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
