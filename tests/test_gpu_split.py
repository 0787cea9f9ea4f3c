"""GPU parity of split-KV decode attention (fa_fwd_split, fa_fwd_split_fp8)
and of the merge (fa_lse_merge) against the float64 oracle (oracle/decode.py).

Inputs are the seeded bf16 or e4m3 bytes of ``workloads`` (the oracle takes
the dequantised e4m3 values).  O is compared element by element at the
forward's tolerances (bf16: max abs 2e-2, relative L2 5e-3; fp8: relative L2
5e-2), lse within 1e-3 for both; the merge alone is compared on partials the
oracle made from a real key split.
"""

import numpy as np
import pytest
import torch

from oracle import attention_decode_gqa, errors, merge_partials, partial_over_keys
from workloads import DECODE_WORKLOADS, by_name, make_inputs

from gpu_util import TOL, check, to_device

pytestmark = pytest.mark.gpu
BASE = "decode_gqa_bf16_b8h32kv8q1n32768d128"


def _print_case(*a):
    print("CASE split", *a, flush=True)


def run_split(x, splits=0, scale=None):
    import exact_io_aware_48_amd as fa
    w = x.workload
    q, k, v = to_device(x)
    o, lse = fa.fa_fwd_split(q, k, v, scale=w.softmax_scale if scale is None else scale, causal=w.causal,
                             num_splits=splits)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle(x, scale=None):
    w = x.workload
    return attention_decode_gqa(x.f64("q"), x.f64("k"), x.f64("v"), w.softmax_scale if scale is None else scale,
                                w.causal)


CASES = [
    # (B, H, H_kv, N_q, N_k, d, causal, splits)
    (2, 8, 2, 1, 1000, 128, True, 0),
    (1, 32, 8, 1, 4096, 128, False, 0),
    (1, 4, 1, 3, 777, 64, True, 5),
    (2, 6, 3, 16, 2048, 64, True, 0),
    (1, 8, 8, 1, 100, 128, False, 1),
    (1, 2, 2, 64, 64, 128, True, 2),          # square: the forward's causal mask
    (1, 4, 2, 1, 20, 64, True, 0),            # fewer keys than one tile
    (1, 16, 2, 8, 500, 128, True, 3),         # 64 rows per K/V head: two row blocks
    (1, 2, 1, 1, 100, 64, True, 1000),        # more splits asked than tiles
    (3, 4, 4, 2, 3000, 64, False, 7),
    (2, 8, 2, 1, 1000, 256, True, 0),         # d = 256: 32-key tiles, 64 KiB ring
    (1, 16, 2, 8, 3001, 256, True, 3),
    (1, 4, 4, 1, 20, 256, False, 1),
    (2, 4, 1, 5, 2048, 256, False, 0),
    (1, 4, 2, 1, 4000, 128, True, 100),       # more than 64 splits: the merge forms the weights again
]


@pytest.mark.parametrize("B,H,H_kv,N_q,N_k,d,causal,splits", CASES)
def test_split_all_elements(B, H, H_kv, N_q, N_k, d, causal, splits):
    _print_case(B, H, H_kv, N_q, N_k, d, causal, splits)
    w = by_name(BASE).with_(B=B, H=H, H_kv=H_kv, N_q=N_q, N=N_k, d=d, causal=causal, seed=100 + N_k)
    x = make_inputs(w)
    o, l = run_split(x, splits)
    o_ref, l_ref = oracle(x)
    check(errors(o, o_ref, l, l_ref), "bf16", f"split B={B} H={H}/{H_kv} N_q={N_q} N_k={N_k} d={d} S={splits}")


def run_split_fp8(x, splits=0, scale=None):
    import exact_io_aware_48_amd as fa
    w = x.workload
    q, k, v = to_device(x)
    o, lse = fa.fa_fwd_split_fp8(q, k, v, *x.descale, scale=w.softmax_scale if scale is None else scale,
                                 causal=w.causal, num_splits=splits)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_fp8(o, l, o_ref, l_ref, what):
    """fp8: O to the fp8 forward's relative L2 bound (P is rounded to e4m3).  The
    scores are exact products of the e4m3 values summed in fp32 and the row sums
    use the unrounded probabilities, so L keeps the bf16 path's bound."""
    errs = errors(o, o_ref, l, l_ref)
    check(errs, "fp8", what)
    assert errs["lse_max"] <= TOL["bf16"]["lse_max"], f"{what}: lse error {errs['lse_max']}"


FP8_CASES = [
    # (B, H, H_kv, N_q, N_k, d, causal, splits): 64-key tiles at every d
    (2, 8, 2, 1, 1000, 128, True, 0),
    (1, 32, 8, 1, 4096, 128, False, 0),
    (1, 4, 1, 3, 777, 64, True, 5),
    (2, 6, 3, 16, 2048, 64, True, 0),
    (1, 4, 2, 1, 20, 64, True, 0),            # fewer keys than one tile
    (1, 16, 2, 8, 500, 128, True, 3),         # 64 rows per K/V head: two row blocks
    (1, 2, 2, 64, 64, 128, True, 2),          # square: the forward's causal mask; more splits than tiles
    (2, 8, 2, 1, 1000, 256, True, 0),         # d = 256: 64 KiB ring
    (1, 16, 2, 8, 3001, 256, True, 3),
    (1, 4, 4, 1, 20, 256, False, 1),
    (3, 4, 4, 2, 3000, 64, False, 7),
]


@pytest.mark.parametrize("B,H,H_kv,N_q,N_k,d,causal,splits", FP8_CASES)
def test_split_fp8_all_elements(B, H, H_kv, N_q, N_k, d, causal, splits):
    _print_case("fp8", B, H, H_kv, N_q, N_k, d, causal, splits)
    w = by_name(BASE).with_(B=B, H=H, H_kv=H_kv, N_q=N_q, N=N_k, d=d, causal=causal, dtype="fp8", seed=200 + N_k)
    x = make_inputs(w)
    o, l = run_split_fp8(x, splits)
    o_ref, l_ref = oracle(x)
    check_fp8(o, l, o_ref, l_ref, f"split fp8 B={B} H={H}/{H_kv} N_q={N_q} N_k={N_k} d={d} S={splits}")


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_split_fp8_other_scales(scale):
    _print_case("fp8 scale", scale)
    w = by_name(BASE).with_(B=1, H=8, H_kv=2, N_q=4, N=900, d=128, dtype="fp8", seed=6)
    x = make_inputs(w)
    o, l = run_split_fp8(x, 0, scale)
    o_ref, l_ref = oracle(x, scale)
    check_fp8(o, l, o_ref, l_ref, f"fp8 scale {scale}")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.7])
def test_split_other_scales(scale):
    _print_case("scale", scale)
    w = by_name(BASE).with_(B=1, H=8, H_kv=2, N_q=4, N=900, d=128, seed=5)
    x = make_inputs(w)
    o, l = run_split(x, 0, scale)
    o_ref, l_ref = oracle(x, scale)
    check(errors(o, o_ref, l, l_ref), "bf16", f"scale {scale}")


def test_split_count_changes_only_rounding_and_repeats_bitwise():
    _print_case("splits")
    w = by_name(BASE).with_(B=1, H=8, H_kv=2, N_q=2, N=5000, d=128, seed=6)
    x = make_inputs(w)
    o_ref, l_ref = oracle(x)
    runs = {}
    for s in (1, 4, 0, 40):
        runs[s] = run_split(x, s)
        check(errors(*runs[s][:1], o_ref, runs[s][1], l_ref), "bf16", f"splits {s}")
    again = run_split(x, 4)
    assert np.array_equal(again[0], runs[4][0]) and np.array_equal(again[1], runs[4][1])


@pytest.mark.parametrize("w", DECODE_WORKLOADS, ids=lambda w: w.name)
def test_split_full_size_all_elements(w):
    _print_case("full", w.name)
    x = make_inputs(w)
    o_ref, l_ref = oracle(x)
    if w.dtype == "fp8":
        check_fp8(*run_split_fp8(x), o_ref, l_ref, w.name)
    else:
        o, l = run_split(x)
        check(errors(o, o_ref, l, l_ref), "bf16", w.name)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_merge_entry_point(out_dtype):
    import exact_io_aware_48_amd as fa
    _print_case("merge", out_dtype)
    rng = np.random.default_rng(9)
    rows, d, N_k = 24, 96, 300
    q, k, v = rng.standard_normal((rows, d)), rng.standard_normal((N_k, d)), rng.standard_normal((N_k, d))
    cuts = [0, 7, 7, 150, 299, 300]                    # one empty part, one single key
    parts = [partial_over_keys(q, k, v, 0.1, True, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    o_parts = np.stack([p[0] for p in parts]).astype(np.float32)
    l_parts = np.stack([p[1] for p in parts]).astype(np.float32)
    o_ref, l_ref = merge_partials(o_parts.astype(np.float64), l_parts.astype(np.float64))
    o, l = fa.fa_lse_merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(l_parts).cuda(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    l = l.cpu().numpy().astype(np.float64)
    tol = 1e-5 if out_dtype == torch.float32 else 8e-3
    assert np.max(np.abs(o - o_ref)) <= tol * max(1.0, np.max(np.abs(o_ref)))
    assert np.max(np.abs(l - l_ref)) <= 1e-5 * max(1.0, np.max(np.abs(l_ref)))
    # a row no part sees merges to O = 0, L = -inf
    l_parts[:, 3] = -np.inf
    o2, l2 = fa.fa_lse_merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(l_parts).cuda(),
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.isneginf(l2.cpu().numpy()[3]) and np.all(o2.cpu().numpy()[3] == 0)


@pytest.mark.parametrize("num_parts,d", [(13, 200), (70, 64), (130, 40)])
def test_merge_many_parts(num_parts, d):
    """Part counts off the merge's batches of eight and past 64 (weights formed
    again from L_s), head dims off its 64-column steps, rows off its four per
    block, and an empty part; fp32 output against the float64 merge."""
    import exact_io_aware_48_amd as fa
    _print_case("merge many", num_parts, d)
    rng = np.random.default_rng(num_parts)
    rows, N_k = 37, 10 * num_parts
    q, k, v = rng.standard_normal((rows, d)), rng.standard_normal((N_k, d)), rng.standard_normal((N_k, d))
    cuts = np.linspace(0, N_k, num_parts + 1).astype(int)
    cuts[3] = cuts[2]                                  # part 2 is empty
    parts = [partial_over_keys(q, k, v, 0.1, False, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    o_parts = np.stack([p[0] for p in parts]).astype(np.float32)
    l_parts = np.stack([p[1] for p in parts]).astype(np.float32)
    o_ref, l_ref = merge_partials(o_parts.astype(np.float64), l_parts.astype(np.float64))
    o, l = fa.fa_lse_merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(l_parts).cuda(),
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    o = o.cpu().numpy().astype(np.float64)
    l = l.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(o - o_ref)) <= 1e-5 * max(1.0, np.max(np.abs(o_ref)))
    assert np.max(np.abs(l - l_ref)) <= 1e-5 * max(1.0, np.max(np.abs(l_ref)))
