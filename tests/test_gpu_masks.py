"""GPU parity of the ALiBi and block-sparse forward variants (fa_fwd_alibi,
fa_fwd_blocksparse and their FP8 forms through the C ABI) against the float64
oracle (oracle/masks.py), element by element, at the forward's tolerances for
each input dtype (bf16, f32, fp8) and head dim (64, 128, 256).
Rows that see no key (block-sparse) must come back as O = 0, lse = -inf
exactly."""

import numpy as np
import pytest
import torch

from oracle import attention_alibi, attention_blocksparse, errors
from oracle.masks import alibi_bias, attention_biased, expand_block_mask
from workloads import by_name, make_inputs

from gpu_util import check, to_device

pytestmark = pytest.mark.gpu
BASE = "gpt2s_causal_bf16_b8h12n1024d64"


def _print_case(*a):
    print("CASE masks", *a, flush=True)


def alibi_slopes(H):
    """The geometric slopes 2^(-8 (h + 1) / H) of the ALiBi paper."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)


def run_alibi(x, slopes, scale=None):
    import exact_io_aware_48_amd as fa
    w = x.workload
    q, k, v = to_device(x)
    sl = torch.from_numpy(slopes).cuda()
    scale = w.softmax_scale if scale is None else scale
    if w.dtype == "fp8":
        o, lse = fa.fa_fwd_alibi_fp8(q, k, v, sl, *x.descale, scale=scale, causal=w.causal)
    else:
        o, lse = fa.fa_fwd_alibi(q, k, v, sl, scale=scale, causal=w.causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def run_sparse(x, bm):
    import exact_io_aware_48_amd as fa
    w = x.workload
    q, k, v = to_device(x)
    m = torch.from_numpy(bm).cuda()
    if w.dtype == "fp8":
        o, lse = fa.fa_fwd_blocksparse_fp8(q, k, v, m, *x.descale, scale=w.softmax_scale, causal=w.causal)
    else:
        o, lse = fa.fa_fwd_blocksparse(q, k, v, m, scale=w.softmax_scale, causal=w.causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_with_empty_rows(o, l, o_ref, l_ref, what, dtype="bf16"):
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l), empty), f"{what}: rows with no visible key differ"
    assert np.all(o[empty] == 0), f"{what}: O of rows with no visible key is not 0"
    seen = ~empty
    if seen.any():
        check(errors(o[seen], o_ref[seen], l[seen], l_ref[seen]), dtype, what)


ALIBI_CASES = [(B, H, N, d, c, "bf16") for (B, H, N) in ((1, 4, 333), (2, 2, 1000), (1, 2, 1))
               for d in (64, 128, 256) for c in (False, True)]
# fp32 inputs: d = 64 and 128 (d = 256 has no variant instance)
ALIBI_CASES += [(1, 2, 333, d, c, dt) for dt in ("f32", "fp8") for d in (64, 128, 256) for c in (False, True)
                if not (dt == "f32" and d == 256)]
ALIBI_CASES += [(2, 3, 1000, 256, True, "fp8"), (1, 2, 1, 128, True, "fp8"), (1, 2, 1, 64, False, "f32")]


@pytest.mark.parametrize("B,H,N,d,causal,dtype", ALIBI_CASES)
def test_alibi_all_elements(B, H, N, d, causal, dtype):
    _print_case("alibi", B, H, N, d, causal, dtype)
    w = by_name(BASE).with_(B=B, H=H, N=N, d=d, causal=causal, dtype=dtype, seed=300 + N + d)
    x = make_inputs(w)
    slopes = alibi_slopes(H)
    o, l = run_alibi(x, slopes)
    o_ref, l_ref = attention_alibi(x.f64("q"), x.f64("k"), x.f64("v"), w.softmax_scale, causal,
                                   slopes.astype(np.float64))
    check(errors(o, o_ref, l, l_ref), dtype, f"alibi B={B} H={H} N={N} d={d} causal={causal} {dtype}")


def test_f32_variants_at_d256_are_refused():
    import exact_io_aware_48_amd as fa
    w = by_name(BASE).with_(B=1, H=2, N=64, d=256, causal=True, dtype="f32", seed=1)
    q, k, v = to_device(make_inputs(w))
    with pytest.raises(fa.FaError, match="UNSUPPORTED"):
        fa.fa_fwd_alibi(q, k, v, torch.ones(2, device="cuda"))
    with pytest.raises(fa.FaError, match="UNSUPPORTED"):
        fa.fa_fwd_blocksparse(q, k, v, torch.ones((1, 1), dtype=torch.uint8, device="cuda"))


def test_alibi_fp8_descales():
    """Per-tensor descales that are not 1: they scale the dot products, not the bias."""
    import exact_io_aware_48_amd as fa
    _print_case("alibi-fp8-descales")
    w = by_name(BASE).with_(B=1, H=2, N=400, d=128, causal=True, dtype="fp8", seed=71)
    x = make_inputs(w)
    assert all(s != 1.0 for s in x.descale)
    slopes = alibi_slopes(w.H)
    o, l = run_alibi(x, slopes)
    o_ref, l_ref = attention_alibi(x.f64("q"), x.f64("k"), x.f64("v"), w.softmax_scale, True,
                                   slopes.astype(np.float64))
    check(errors(o, o_ref, l, l_ref), "fp8", "alibi fp8 descales")
    # the same bytes through fa_fwd_alibi (unit descales) see the undescaled values
    q, k, v = to_device(x)
    o1, l1 = fa.fa_fwd_alibi(q, k, v, torch.from_numpy(slopes).cuda(), scale=w.softmax_scale, causal=True)
    torch.cuda.synchronize()
    qu, ku, vu = (x.f64(n) / s for n, s in zip(("q", "k", "v"), x.descale))
    o_ref1, l_ref1 = attention_alibi(qu, ku, vu, w.softmax_scale, True, slopes.astype(np.float64))
    check(errors(o1.float().cpu().numpy().astype(np.float64), o_ref1, l1.cpu().numpy().astype(np.float64),
                 l_ref1), "fp8", "alibi fp8 unit descales")


@pytest.mark.parametrize("scale,slopes", [(-0.1, (0.5, 0.02)), (0.3, (4.0, 0.0)), (0.0, (0.1, 1.0))])
def test_alibi_scales_and_slopes(scale, slopes):
    _print_case("alibi-scale", scale, slopes)
    w = by_name(BASE).with_(B=1, H=2, N=300, d=128, causal=True, seed=44)
    x = make_inputs(w)
    sl = np.array(slopes, dtype=np.float32)
    o, l = run_alibi(x, sl, scale)
    o_ref, l_ref = attention_alibi(x.f64("q"), x.f64("k"), x.f64("v"), scale, True, sl.astype(np.float64))
    check(errors(o, o_ref, l, l_ref), "bf16", f"alibi scale={scale} slopes={slopes}")


def test_alibi_full_gpt2s_shape():
    w = by_name(BASE)
    _print_case("alibi-full", w.name)
    x = make_inputs(w)
    slopes = alibi_slopes(w.H)
    o, l = run_alibi(x, slopes)
    o_ref, l_ref = attention_alibi(x.f64("q"), x.f64("k"), x.f64("v"), w.softmax_scale, True,
                                   slopes.astype(np.float64))
    check(errors(o, o_ref, l, l_ref), "bf16", "alibi gpt2s")


def _patterns(B, H, nb, seed):
    rng = np.random.default_rng(seed)
    local = np.zeros((nb, nb), dtype=np.uint8)
    for i in range(nb):
        local[i, max(0, i - 1):i + 2] = 1
        local[i, 0] = 1                       # a global first block
    empty_row = rng.integers(0, 2, (nb, nb)).astype(np.uint8)
    empty_row[nb // 2] = 0                    # a row block that sees nothing
    return {
        "random": rng.integers(0, 2, (B, H, nb, nb)).astype(np.uint8),
        "local_global": np.broadcast_to(local, (B, H, nb, nb)).copy(),
        "empty_row": np.broadcast_to(empty_row, (B, H, nb, nb)).copy(),
        "all": np.ones((B, H, nb, nb), dtype=np.uint8),
        "none": np.zeros((B, H, nb, nb), dtype=np.uint8),
    }


SPARSE_CASES = [(B, H, N, d, c, pat, "bf16") for (B, H, N) in ((1, 2, 700), (2, 2, 300)) for d in (64, 128, 256)
                for c in (False, True) for pat in ("random", "local_global", "empty_row")]
SPARSE_CASES += [(1, 2, 513, 128, True, "all", "bf16"), (1, 2, 200, 64, False, "none", "bf16"),
                 (1, 1, 1, 64, True, "all", "bf16"), (1, 2, 300, 256, True, "none", "bf16")]
SPARSE_CASES += [(1, 2, 700, d, c, pat, dt) for dt in ("f32", "fp8") for d in (64, 128, 256) for c in (False, True)
                 for pat in ("random", "empty_row") if not (dt == "f32" and d == 256)]
SPARSE_CASES += [(1, 1, 1, 256, False, "all", "fp8"), (1, 2, 200, 128, True, "none", "f32")]


@pytest.mark.parametrize("B,H,N,d,causal,pattern,dtype", SPARSE_CASES)
def test_blocksparse_all_elements(B, H, N, d, causal, pattern, dtype):
    _print_case("sparse", B, H, N, d, causal, pattern, dtype)
    w = by_name(BASE).with_(B=B, H=H, N=N, d=d, causal=causal, dtype=dtype, seed=400 + N + d)
    x = make_inputs(w)
    nb = (N + 127) // 128
    bm = _patterns(B, H, nb, seed=N + d + (1 if causal else 0))[pattern]
    o, l = run_sparse(x, bm)
    o_ref, l_ref = attention_blocksparse(x.f64("q"), x.f64("k"), x.f64("v"), w.softmax_scale, causal, bm)
    check_with_empty_rows(o, l, o_ref, l_ref, f"sparse B={B} H={H} N={N} d={d} causal={causal} {pattern} {dtype}",
                          dtype)


def test_blocksparse_shared_masks():
    """A [H, nb, nb] mask shared by the batch and an [nb, nb] mask shared by all heads."""
    import exact_io_aware_48_amd as fa
    _print_case("sparse-shared")
    w = by_name(BASE).with_(B=2, H=3, N=400, d=64, causal=False, seed=9)
    x = make_inputs(w)
    q, k, v = to_device(x)
    nb = 4
    rng = np.random.default_rng(5)
    for shape in ((3, nb, nb), (nb, nb)):
        bm = rng.integers(0, 2, shape).astype(np.uint8)
        o, l = fa.fa_fwd_blocksparse(q, k, v, torch.from_numpy(bm).cuda(), scale=w.softmax_scale, causal=False)
        torch.cuda.synchronize()
        full = np.broadcast_to(bm, (2, 3, nb, nb))
        o_ref, l_ref = attention_blocksparse(x.f64("q"), x.f64("k"), x.f64("v"), w.softmax_scale, False, full)
        check_with_empty_rows(o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64),
                              o_ref, l_ref, f"shared mask {shape}")


def _sample_rows(N, seed):
    rng = np.random.default_rng(seed)
    edges = [0, 1, 127, 128, 255, 256, N // 2, N - 2, N - 1]
    return np.unique(np.concatenate([edges, rng.choice(N, 20, replace=False)]))


def test_alibi_full_long_causal_sampled():
    """The long-context causal workload with ALiBi, as the benchmark times it:
    sampled rows of sampled heads."""
    w = by_name("long_causal_bf16_b1h32n8192d128")
    _print_case("alibi-long", w.name)
    x = make_inputs(w)
    slopes = alibi_slopes(w.H)
    o, l = run_alibi(x, slopes)
    rows = _sample_rows(w.N, 1)
    for h in (0, 17, 31):
        o_ref, l_ref = attention_biased(x.f64("q", 0, h), x.f64("k", 0, h), x.f64("v", 0, h), w.softmax_scale, True,
                                        bias=alibi_bias(w.N, float(slopes[h]), rows), rows=rows)
        check(errors(o[0, h, rows], o_ref, l[0, h, rows], l_ref), "bf16", f"alibi long head {h}")


def test_blocksparse_full_sliding_window_sampled():
    """N = 8192, d = 128, 32 heads, non-causal, each 128-query block seeing its
    neighbours and the first key block (the benchmark's pattern): sampled rows."""
    w = by_name("long_causal_bf16_b1h32n8192d128").with_(causal=False)
    _print_case("sparse-long")
    x = make_inputs(w)
    nb = w.N // 128
    bm = np.zeros((nb, nb), dtype=np.uint8)
    for i in range(nb):
        bm[i, max(0, i - 1):i + 2] = 1
        bm[i, 0] = 1
    o, l = run_sparse(x, bm)
    rows = _sample_rows(w.N, 2)
    for h in (0, 31):
        o_ref, l_ref = attention_biased(x.f64("q", 0, h), x.f64("k", 0, h), x.f64("v", 0, h), w.softmax_scale, False,
                                        allowed=expand_block_mask(bm, w.N, rows=rows), rows=rows)
        check(errors(o[0, h, rows], o_ref, l[0, h, rows], l_ref), "bf16", f"sparse long head {h}")


def test_alibi_full_wide_fp8_sampled():
    """B=2, H=8, N=16384, d=256 on FP8 inputs with ALiBi, non-causal: sampled
    rows of one head per batch (the full launch shape of the d = 256 variant)."""
    w = by_name("wide_fp8_b2h8n16384d256")
    _print_case("alibi-wide-fp8", w.name)
    x = make_inputs(w)
    slopes = alibi_slopes(w.H)
    o, l = run_alibi(x, slopes)
    rows = _sample_rows(w.N, 3)
    for b, h in ((0, 0), (1, 7)):
        o_ref, l_ref = attention_biased(x.f64("q", b, h), x.f64("k", b, h), x.f64("v", b, h), w.softmax_scale,
                                        w.causal, bias=alibi_bias(w.N, float(slopes[h]), rows), rows=rows)
        check(errors(o[b, h, rows], o_ref, l[b, h, rows], l_ref), "fp8", f"alibi wide fp8 b{b} h{h}")


def test_blocksparse_full_wide_bf16_sampled():
    """B=2, H=8, N=16384, d=256, bf16, causal, a local + global block pattern:
    sampled rows."""
    w = by_name("wide_bf16_b2h8n16384d256").with_(causal=True)
    _print_case("sparse-wide-bf16")
    x = make_inputs(w)
    nb = w.N // 128
    bm = np.zeros((nb, nb), dtype=np.uint8)
    for i in range(nb):
        bm[i, max(0, i - 2):i + 1] = 1
        bm[i, 0] = 1
    o, l = run_sparse(x, bm)
    rows = _sample_rows(w.N, 4)
    for b, h in ((0, 3), (1, 5)):
        o_ref, l_ref = attention_biased(x.f64("q", b, h), x.f64("k", b, h), x.f64("v", b, h), w.softmax_scale, True,
                                        allowed=expand_block_mask(bm, w.N, rows=rows), rows=rows)
        check(errors(o[b, h, rows], o_ref, l[b, h, rows], l_ref), "bf16", f"sparse wide b{b} h{h}")
