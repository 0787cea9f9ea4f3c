"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Inputs are the same seeded bytes on both sides (``workloads``).  Reduced-size
cases are compared element by element over the whole output; they span
several K/V tiles and query blocks and end on a ragged tail.  Full-size
workloads are compared on every element, in the same launch configuration
the benchmark times, against the threaded float64 oracle.
"""

import numpy as np
import pytest
import torch

from oracle import attention_rows, errors
from workloads import WORKLOADS, by_name, make_inputs
from workloads.gen import from_f32

from gpu_util import TOL, check, oracle_all, oracle_full, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _print_case(*a):
    print("CASE", *a, flush=True)


# ---------------------------------------------------------------- reduced sizes, every element
REDUCED = [
    # (base workload, B, H, N)
    ("tiny_f32_b1h2n256d64", 1, 2, 256),
    ("tiny_f32_b1h2n256d64", 1, 1, 300),
    ("gpt2s_causal_bf16_b8h12n1024d64", 2, 3, 333),
    ("bertl_bf16_b16h16n512d64", 2, 2, 300),
    ("long_causal_bf16_b1h32n8192d128", 1, 2, 1000),
    ("wide_bf16_b2h8n16384d256", 1, 2, 700),
    ("wide_fp8_b2h8n16384d256", 1, 2, 700),
]
# grouped-query: (base workload, B, H, H_kv, N)
REDUCED_GQA = [
    ("gqa_causal_bf16_b1h32kv8n8192d128", 1, 8, 2, 700),     # groups of 4
    ("gqa_causal_bf16_b1h32kv8n8192d128", 2, 6, 3, 333),     # groups of 2, two batches
    ("gqa_causal_bf16_b1h32kv8n8192d128", 1, 4, 1, 300),     # MQA
    ("gqa_causal_bf16_b1h32kv8n8192d128", 1, 16, 8, 257),    # 8 K/V heads: one per XCD
]


@pytest.mark.parametrize("name,B,H,N", REDUCED)
def test_reduced_workloads_all_elements(name, B, H, N):
    w = by_name(name).with_(B=B, H=H, N=N)
    _print_case(name, B, H, N)
    x = make_inputs(w)
    o, l = run_gpu(x)
    o_ref, l_ref = oracle_full(x)
    e = errors(o, o_ref, l, l_ref)
    check(e, w.dtype, f"{name} B={B} H={H} N={N}")


@pytest.mark.parametrize("name,B,H,H_kv,N", REDUCED_GQA)
@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("bf16", 64, False), ("bf16", 256, False),
                                            ("fp8", 128, True), ("f32", 64, True)])
def test_gqa_all_elements(name, B, H, H_kv, N, dtype, d, causal):
    w = by_name(name).with_(B=B, H=H, H_kv=H_kv, N=N, d=d, dtype=dtype, causal=causal)
    _print_case("gqa", name, B, H, H_kv, N, dtype, d, causal)
    x = make_inputs(w)
    o, l = run_gpu(x)
    o_ref, l_ref = oracle_full(x)
    check(errors(o, o_ref, l, l_ref), dtype, f"gqa B={B} H={H} H_kv={H_kv} N={N} {dtype} d={d} causal={causal}")


# ---------------------------------------------------------------- edge shapes
EDGE = [(N, d, c, dt) for dt in ("bf16",) for d in (64, 128, 256) for N in (1, 7, 100, 257, 1000)
        for c in (False, True)]
EDGE += [(N, d, c, "f32") for d in (64, 128, 256) for N in (1, 100, 257) for c in (False, True)]
# fp32 at d = 256 runs its largest (spilling) instance: ragged causal diagonals at several sizes
EDGE += [(N, 256, True, "f32") for N in (333, 1000, 1313)]
EDGE += [(N, d, c, "fp8") for d in (64, 128, 256) for N in (1, 100, 257) for c in (False, True)]


@pytest.mark.parametrize("N,d,causal,dtype", EDGE)
def test_edge_shapes(N, d, causal, dtype):
    w = by_name("bertl_bf16_b16h16n512d64").with_(B=1, H=2, N=N, d=d, causal=causal, dtype=dtype, seed=1000 + N + d)
    _print_case("edge", N, d, causal, dtype)
    x = make_inputs(w)
    o, l = run_gpu(x)
    o_ref, l_ref = oracle_full(x)
    check(errors(o, o_ref, l, l_ref), dtype, f"edge N={N} d={d} causal={causal} {dtype}")


# ---------------------------------------------------------------- full-size workloads
# Every element of every workload at its full size, in the launch configuration
# the benchmark times, against the threaded float64 oracle (the largest, the
# two N = 16384, d = 256 workloads, take about 4.4e12 float64 FLOPs each).
@pytest.mark.parametrize("name", [w.name for w in WORKLOADS])
def test_full_size_workloads(name):
    w = by_name(name)
    _print_case("full", name)
    x = make_inputs(w)
    o, l = run_gpu(x)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    o_ref, l_ref = oracle_all(x)
    check(errors(o, o_ref, l, l_ref), w.dtype, name + " (every element)")


# ---------------------------------------------------------------- structured inputs
@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("f32", 64), ("fp8", 256)])
@pytest.mark.parametrize("causal", [False, True])
def test_v_all_ones(dtype, d, causal):
    w = by_name("bertl_bf16_b16h16n512d64").with_(B=1, H=2, N=300, d=d, dtype=dtype, causal=causal)
    base = make_inputs(w.with_(dtype="f32"))
    x = from_f32(w, base.q * 2, base.k, np.ones_like(base.v))
    _print_case("v_ones", dtype, d, causal)
    o, _ = run_gpu(x)
    # fp8: P is rounded to e4m3, whose half-ulp is 2**-4 of the value
    tol = 2e-2 if dtype != "fp8" else 2.0**-4
    assert np.max(np.abs(o - 1.0)) <= tol


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("f32", 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_mean_and_log_count(dtype, d, causal):
    N = 257
    w = by_name("bertl_bf16_b16h16n512d64").with_(B=1, H=1, N=N, d=d, dtype=dtype, causal=causal)
    base = make_inputs(w.with_(dtype="f32"))
    x = from_f32(w, np.zeros_like(base.q), base.k, base.v)
    _print_case("q_zero", dtype, d, causal)
    o, l = run_gpu(x)
    v = x.f64("v")[0, 0]
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = np.cumsum(v, axis=0) / counts[:, None] if causal else np.broadcast_to(v.mean(axis=0), v.shape)
    check(errors(o[0, 0], mean, l[0, 0], np.log(counts)), dtype, "q_zero")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_causal_row0_is_v0_bitwise(d):
    w = by_name("gpt2s_causal_bf16_b8h12n1024d64").with_(B=1, H=2, N=200, d=d)
    x = make_inputs(w)
    _print_case("row0", d)
    o, l = run_gpu(x)
    assert np.array_equal(o[:, :, 0], x.f64("v")[:, :, 0])
    s0 = w.softmax_scale * np.einsum("bhd,bhd->bh", x.f64("q")[:, :, 0], x.f64("k")[:, :, 0])
    assert np.max(np.abs(l[:, :, 0] - s0)) < 1e-4


def test_large_scores_from_shifted_keys():
    # every key shifted by 16 in every dim: scores reach tens, so the running max moves a lot
    w = by_name("bertl_bf16_b16h16n512d64").with_(B=1, H=1, N=320, d=64)
    base = make_inputs(w.with_(dtype="f32"))
    x = from_f32(w, base.q, base.k + np.float32(16.0), base.v)
    _print_case("shift")
    o, l = run_gpu(x)
    ref, lref = oracle_full(x)
    assert np.max(np.abs(lref)) > 20
    check(errors(o, ref, l, lref), "bf16", "shifted keys")


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("f32", 64), ("fp8", 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_running_max_grows_at_row_dependent_rates(dtype, d, causal):
    """Scores rise along the keys at a different rate for every query row, so
    the running maximum grows by more than the rescale threshold on many
    tiles, by different amounts in neighbouring rows (the rescale of O and l
    must use each row's own factor)."""
    N = 400
    w = by_name("bertl_bf16_b16h16n512d64").with_(B=1, H=2, N=N, d=d, dtype=dtype, causal=causal)
    base = make_inputs(w.with_(dtype="f32"))
    rate = (np.arange(N) % 7).astype(np.float32)[None, None, :, None] * np.float32(0.25)
    ramp = (np.arange(N) / N).astype(np.float32)[None, None, :, None] * np.float32(4.0)
    q = base.q * np.float32(0.5) + rate
    k = base.k * np.float32(0.5) + ramp
    x = from_f32(w, q, k, base.v)
    _print_case("row-rates", dtype, d, causal)
    o, l = run_gpu(x)
    ref, lref = oracle_full(x)
    check(errors(o, ref, l, lref), dtype, f"row-dependent growth {dtype} d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_scores_jump_after_the_first_tiles(d, causal):
    """From key J on, every score rises by a row-dependent amount, up to about
    18 (natural units; 26 in log2 units) above the earlier keys: tiles after
    a row's first take the exponentials against a base far below their
    maximum, their lane sums pass the bound, and the tile is redone against a
    new base for the rows that grew by more than the lag (others keep
    theirs).  J differs per head so the jump falls at different tile phases."""
    N = 700
    w = by_name("bertl_bf16_b16h16n512d64").with_(B=1, H=3, N=N, d=d, causal=causal)
    base = make_inputs(w.with_(dtype="f32"))
    rng = np.random.default_rng(17)
    u = rng.standard_normal(d).astype(np.float32)
    u /= np.linalg.norm(u)
    q = base.q * np.float32(0.5)
    k = base.k * np.float32(0.5)
    beta = np.linspace(0.0, 1.5, N, dtype=np.float32)              # per query row
    alpha = np.float32(12.0 / (1.5 * w.softmax_scale))               # score rise 12 * beta: up to 18
    for h, J in enumerate((70, 200, 333)):
        q[0, h] += beta[:, None] * u[None, :] * np.float32(1.5)
        k[0, h, J:] += alpha * u[None, :]
    x = from_f32(w, q, k, base.v)
    _print_case("jump", d, causal)
    o, l = run_gpu(x)
    ref, lref = oracle_full(x)
    check(errors(o, ref, l, lref), "bf16", f"score jump d={d} causal={causal}")


# ---------------------------------------------------------------- maximum sizes
def _edge_rows(N, extra, seed):
    rng = np.random.default_rng(seed)
    edges = [0, 1, 63, 64, 255, 256, N // 2, N - 257, N - 256, N - 2, N - 1]
    return np.unique(np.concatenate([edges, rng.choice(N, extra, replace=False)])).astype(np.int64)


def test_long_context_n131072_sampled_rows():
    """N = 131072 keys, causal, d = 128 (the largest context the tests run):
    seeded inputs, sampled rows of both heads against the float64 oracle."""
    w = by_name("long_causal_bf16_b1h32n8192d128").with_(H=2, N=131072, seed=131)
    _print_case("long-context", w.N)
    x = make_inputs(w)
    o, l = run_gpu(x)
    rows = _edge_rows(w.N, 40, 5)
    for h in range(2):
        o_ref, l_ref = attention_rows(x.f64("q", 0, h), x.f64("k", 0, h), x.f64("v", 0, h), w.softmax_scale, True,
                                      rows)
        check(errors(o[0, h, rows], o_ref, l[0, h, rows], l_ref), "bf16", f"N=131072 head {h}")


def test_offsets_beyond_2_31_elements():
    """B=1, H=72, N=131072, d=256 (2.4e9 elements per tensor, 4.5 GiB each):
    head 64 starts exactly at element 2^31 and the later heads past it.  Q = 0 makes every score 0, so query i
    sees its visible keys uniformly: O_i is the mean of V over keys j <= i and
    L_i = log(i + 1) (a property that holds at any size).  V is a pattern with
    values k/16, k = (7j + 3c + 5h) mod 17, exact in bf16, built on the device;
    sampled rows of sampled heads are compared with the float64 prefix means."""
    import exact_io_aware_48_amd as fa
    B, H, N, d = 1, 72, 131072, 256
    assert 64 * N * d == 2**31
    _print_case("offsets>2^31", B, H, N, d)
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros_like(q)
    v = torch.empty_like(q)
    j = torch.arange(N, device="cuda", dtype=torch.int64)[:, None]
    c = torch.arange(d, device="cuda", dtype=torch.int64)[None, :]
    for h in range(H):
        v[0, h] = (((7 * j + 3 * c + 5 * h) % 17).to(torch.float32) / 16).to(torch.bfloat16)
    del j, c
    o, lse = fa.fa_fwd(q, k, v, scale=1.0 / 16, causal=True)
    torch.cuda.synchronize()
    del q, k, v
    rows = _edge_rows(N, 24, 6)
    rows_t = torch.from_numpy(rows).cuda()
    jj = np.arange(N, dtype=np.int64)[:, None]
    cc = np.arange(d, dtype=np.int64)[None, :]
    for h in (0, 40, 63, 64, 71):
        got_o = o[0, h].index_select(0, rows_t).float().cpu().numpy().astype(np.float64)
        got_l = lse[0, h].index_select(0, rows_t).cpu().numpy().astype(np.float64)
        vals = ((7 * jj + 3 * cc + 5 * h) % 17).astype(np.float64) / 16
        prefix = np.cumsum(vals, axis=0)[rows] / (rows[:, None] + 1)
        check(errors(got_o, prefix, got_l, np.log(rows + 1.0)), "bf16", f"offsets>2^31 head {h}")


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.3])
def test_other_scales(scale):
    w = by_name("bertl_bf16_b16h16n512d64").with_(B=1, H=2, N=190, d=64, causal=True)
    x = make_inputs(w)
    _print_case("scale", scale)
    o, l = run_gpu(x, scale=scale)
    ref, lref = oracle_full(x, scale=scale)
    check(errors(o, ref, l, lref), "bf16", f"scale={scale}")


# ---------------------------------------------------------------- runtime behaviour
def test_deterministic_and_stream():
    w = by_name("long_causal_bf16_b1h32n8192d128").with_(B=1, H=8, N=1500)
    x = make_inputs(w)
    _print_case("determinism")
    a = run_gpu(x)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_gpu(x, stream=s)
    c = run_gpu(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[0], c[0])
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[1], c[1])


def test_error_paths_raise():
    import exact_io_aware_48_amd as fa
    q = torch.zeros((1, 1, 16, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as ei:
        fa.fa_fwd(q, q, q)
    assert ei.value.status == 3
    q = torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as ei:
        fa.fa_fwd(q, q, q, scale=float("inf"))
    assert ei.value.status == 5
    q8 = torch.zeros((1, 1, 16, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FaError) as ei:
        fa.fa_fwd_fp8(q8, q8, q8, 1.0, 0.0, 1.0)
    assert ei.value.status == 5
