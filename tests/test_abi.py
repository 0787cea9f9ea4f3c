"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments with the documented status before any
HIP call.  No compute entry point is called with valid arguments here."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


@pytest.fixture(scope="module")
def lib():
    from exact_io_aware_48_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from exact_io_aware_48_amd.build import build
        build()
    return _lib.load()


def declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names.update(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fa_bwd", "fa_bwd_workspace_size", "fa_fwd", "fa_fwd_alibi",
                                    "fa_fwd_alibi_fp8", "fa_fwd_blocksparse", "fa_fwd_blocksparse_fp8", "fa_fwd_fp8", "fa_fwd_gqa", "fa_fwd_gqa_fp8", "fa_fwd_split",
                                    "fa_fwd_split_fp8", "fa_fwd_split_noalloc", "fa_fwd_split_plan", "fa_lse_merge", "fa_plan",
                                    "fa_split_scratch_bytes", "fa_status_string", "fa_timeline_read", "fa_version"]


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(lib._name)
    for name in declared_functions():
        assert hasattr(raw, name), name


PROBE = os.path.join(ROOT, "exact_io_aware_48_amd", "libfa_probe.so")


@pytest.mark.skipif(not os.path.exists(PROBE), reason="probe library not built")
def test_probe_library_host_side():
    """The probe library's table and argument checks (no launch: a NULL output
    buffer or a zero iteration count is refused before any HIP call)."""
    from exact_io_aware_48_amd import _lib
    lib = _lib.load_probe()
    n = lib.fa_probe_mixed_count()
    assert n == 12
    names = [lib.fa_probe_mixed_name(i).decode() for i in range(n)]
    assert len(set(names)) == n and lib.fa_probe_mixed_name(n) == b""
    w = (ctypes.c_int * 5)()
    for i in range(n):
        assert lib.fa_probe_mixed_work(i, w) == 0
        wps, mf, fma, ex, lds = list(w)
        assert wps in (1, 2) and names[i].startswith(f"{wps} wave")
        assert (f"{mf} MFMA" in names[i]) == (mf > 0) and (f"{fma} FMA" in names[i]) == (fma > 0)
        assert (f"{ex} exp" in names[i]) == (ex > 0) and (f"{lds} ds_read" in names[i]) == (lds > 0)
    assert lib.fa_probe_mixed_work(n, w) == 2 and lib.fa_probe_mixed_work(-1, w) == 2
    ms = ctypes.c_float()
    assert lib.fa_probe_mixed(0, None, 1 << 20, 10, 1, ctypes.byref(ms)) == 2
    assert lib.fa_probe_roles(1, None, 1 << 20, 10, 1, ctypes.byref(ms)) == 2
    assert lib.fa_probe_mixed(0, FAKE, 1 << 20, 0, 1, ctypes.byref(ms)) == 2


def test_timeline_read_is_unsupported_in_the_product_build(lib):
    import numpy as np
    buf = np.zeros(12, dtype=np.uint64)
    assert lib.fa_timeline_read(buf.ctypes.data, buf.nbytes) == 3        # FA_ERR_UNSUPPORTED
    assert not buf.any()


def test_status_strings_and_version(lib):
    for code in range(8):
        s = lib.fa_status_string(code).decode()
        assert s.startswith("FA_")
    assert lib.fa_status_string(99).decode() == "unknown fa_status"
    assert lib.fa_version() >= 100


FAKE = 0x10000      # aligned, never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,expected", [
    # q, k, v, o, lse, B, H, N, d, scale, causal, dtype
    ((0, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 0.1, 0, 1), 1),
    ((FAKE, FAKE, FAKE, FAKE, 0, 1, 1, 64, 64, 0.1, 0, 1), 1),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 64, 64, 0.1, 0, 1), 2),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 0, 64, 0.1, 0, 1), 2),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, -3, 64, 64, 0.1, 0, 1), 2),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 2**40, 64, 0.1, 0, 1), 2),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 2**31, 2**31, 64, 64, 0.1, 0, 1), 2),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 96, 0.1, 0, 1), 3),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 0.1, 0, 7), 3),
    ((FAKE + 2, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 0.1, 0, 1), 4),
    ((FAKE, FAKE, FAKE, FAKE, FAKE + 4, 1, 1, 64, 64, 0.1, 0, 1), 4),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, float("inf"), 0, 1), 5),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, float("nan"), 1, 0), 5),
])
def test_fa_fwd_validation(lib, args, expected):
    assert lib.fa_fwd(*args, None) == expected


@pytest.mark.parametrize("descales,expected", [((1.0, 0.0, 1.0), 5), ((-1.0, 1.0, 1.0), 5),
                                                ((1.0, 1.0, float("nan")), 5), ((1.0, float("inf"), 1.0), 5)])
def test_fa_fwd_fp8_descale_validation(lib, descales, expected):
    assert lib.fa_fwd_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 0.1, *descales, 0, None) == expected


@pytest.mark.parametrize("H,H_kv,expected", [(8, 0, 2), (8, -2, 2), (8, 3, 2), (6, 4, 2), (4, 8, 2)])
def test_fa_fwd_gqa_group_validation(lib, H, H_kv, expected):
    assert lib.fa_fwd_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, H, H_kv, 64, 64, 0.1, 0, 1, None) == expected
    assert lib.fa_fwd_gqa_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 1, H, H_kv, 64, 64, 0.1, 1.0, 1.0, 1.0, 0,
                              None) == expected


def test_fa_fwd_gqa_checks_the_rest_like_fa_fwd(lib):
    # a valid grouping still gets every other check of fa_fwd, before any launch
    assert lib.fa_fwd_gqa(0, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, 64, 0.1, 0, 1, None) == 1
    assert lib.fa_fwd_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, 96, 0.1, 0, 1, None) == 3
    assert lib.fa_fwd_gqa(FAKE, FAKE + 8, FAKE, FAKE, FAKE, 1, 8, 2, 64, 64, 0.1, 0, 1, None) == 4
    assert lib.fa_fwd_gqa_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, 64, 0.1, 1.0, 0.0, 1.0, 0, None) == 5


def test_fp8_scale_overflow_rejected(lib):
    assert lib.fa_fwd_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 1e30, 1e10, 1e10, 1.0, 0, None) == 5


def test_plan_counts():
    from exact_io_aware_48_amd import fa_plan, FA_BF16, FA_FP8_E4M3
    p = fa_plan(1, 32, 8192, 128, causal=True, dtype=FA_BF16)
    br, bc = p["block_rows"], p["block_cols"]
    assert p["workgroups"] == 32 * 8192 // br
    # causal: row block i streams ceil((i+1)*br/bc) tiles -- the blocks fully above the diagonal are skipped
    per_head = sum(min(8192 // bc, ((i + 1) * br - 1) // bc + 1) for i in range(8192 // br))
    assert p["kv_tiles"] == 32 * per_head
    assert per_head < (8192 // br) * (8192 // bc) * 0.52
    q = fa_plan(2, 8, 16384, 256, causal=False, dtype=FA_FP8_E4M3)
    assert q["kv_tiles"] == 16 * (16384 // q["block_rows"]) * (16384 // q["block_cols"])
    assert q["lds_bytes"] <= 160 * 1024
    r = fa_plan(1, 1, 1, 64)
    assert r["workgroups"] == 1 and r["kv_tiles"] == 1


def test_binding_fails_loudly_without_library(monkeypatch):
    from exact_io_aware_48_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libfa_fwd.so")
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def test_fa_bwd_workspace_size(lib):
    n = ctypes.c_int64()
    assert lib.fa_bwd_workspace_size(2, 3, 3, 100, 64, ctypes.byref(n)) == 0 and n.value == 2 * 3 * 2 * 128 * 4
    assert lib.fa_bwd_workspace_size(1, 1, 1, 64, 128, ctypes.byref(n)) == 0 and n.value == 512
    assert lib.fa_bwd_workspace_size(1, 1, 1, 65, 64, ctypes.byref(n)) == 0 and n.value == 1024
    # grouped heads: statistics plus room for dK and dV partials of every query head
    assert lib.fa_bwd_workspace_size(1, 8, 2, 64, 128, ctypes.byref(n)) == 0 and n.value == 8 * 512 + 2 * 8 * 64 * 128 * 4
    assert lib.fa_bwd_workspace_size(1, 1, 1, 64, 64, None) == 1
    assert lib.fa_bwd_workspace_size(0, 1, 1, 64, 64, ctypes.byref(n)) == 2
    assert lib.fa_bwd_workspace_size(1, 1, 1, 0, 64, ctypes.byref(n)) == 2
    assert lib.fa_bwd_workspace_size(1, 8, 3, 64, 64, ctypes.byref(n)) == 2
    assert lib.fa_bwd_workspace_size(1, 1, 1, 64, 96, ctypes.byref(n)) == 3
    # d = 256: the same statistics; partials scale with d
    assert lib.fa_bwd_workspace_size(1, 8, 2, 64, 256, ctypes.byref(n)) == 0 and n.value == 8 * 512 + 2 * 8 * 64 * 256 * 4


def _bwd_args(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, ws=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             B=1, H=2, H_kv=2, N=64, d=64, scale=0.1, causal=0, dtype=1)
    a.update(kw)
    return [a[n] for n in ("q", "k", "v", "o", "do", "lse", "ws", "dq", "dk", "dv", "B", "H", "H_kv", "N", "d",
                           "scale", "causal", "dtype")] + [None]


@pytest.mark.parametrize("kw,expected", [
    ({"q": 0}, 1), ({"do": 0}, 1), ({"lse": 0}, 1), ({"ws": 0}, 1), ({"dv": 0}, 1),
    ({"B": 0}, 2), ({"N": 0}, 2), ({"H_kv": 0}, 2), ({"H_kv": 3}, 2), ({"H": 2, "H_kv": 4}, 2),
    ({"N": 2**40}, 2), ({"B": 2**31, "H": 2**31}, 2),
    ({"d": 512}, 3), ({"d": 96}, 3), ({"dtype": 0}, 3), ({"dtype": 2}, 3),
    ({"o": FAKE + 8}, 4), ({"ws": FAKE + 4}, 4), ({"dk": FAKE + 2}, 4),
    ({"scale": float("inf")}, 5), ({"scale": float("nan")}, 5), ({"scale": 3e38}, 5),
])
def test_fa_bwd_validation(lib, kw, expected):
    assert lib.fa_bwd(*_bwd_args(**kw)) == expected


def _plan(lib, B, H, H_kv, N_q, N_k, d, splits, dtype=1):
    sp, nb = ctypes.c_int(), ctypes.c_int64()
    st = lib.fa_fwd_split_plan(B, H, H_kv, N_q, N_k, d, splits, dtype, ctypes.byref(sp), ctypes.byref(nb))
    return st, sp.value, nb.value


def test_fa_fwd_split_plan(lib):
    # asked-for splits: 8192 keys in 32-key tiles (d = 128) -> 8 splits of 1024 keys
    st, sp, nb = _plan(lib, 2, 32, 8, 1, 8192, 128, 8)
    assert st == 0 and sp == 8 and nb == 8 * 2 * 32 * 1 * 129 * 4
    # more splits than tiles: one per tile
    st, sp, _ = _plan(lib, 1, 4, 4, 1, 100, 64, 50)
    assert st == 0 and sp == 2
    # 10 tiles over 3 requested splits: chunks of 4 tiles -> 3 splits
    st, sp, _ = _plan(lib, 1, 1, 1, 1, 640, 64, 3)
    assert st == 0 and sp == 3
    # automatic: at least one, never more than a quarter of the tiles
    st, sp, _ = _plan(lib, 1, 8, 8, 1, 100, 64, 0)
    assert st == 0 and sp == 1
    st, sp, _ = _plan(lib, 1, 8, 1, 1, 65536, 128, 0)
    assert st == 0 and 1 <= sp <= 2048 // 4
    # d = 256 streams 32-key tiles too: 4096 keys asked in 4 splits -> 1024 keys each
    st, sp, nb = _plan(lib, 1, 8, 2, 1, 4096, 256, 4)
    assert st == 0 and sp == 4 and nb == 4 * 8 * 257 * 4


def test_fa_fwd_split_plan_fp8_takes_64_key_tiles(lib):
    # 100 keys at d = 128: four 32-key bf16 tiles, two 64-key fp8 tiles
    assert _plan(lib, 1, 4, 4, 1, 100, 128, 50)[:2] == (0, 4)
    assert _plan(lib, 1, 4, 4, 1, 100, 128, 50, dtype=2)[:2] == (0, 2)
    # 8192 keys asked in 8 splits: 1024 keys each either way, and the same fp32 partials
    assert _plan(lib, 2, 32, 8, 1, 8192, 128, 8, dtype=2) == _plan(lib, 2, 32, 8, 1, 8192, 128, 8)
    # 640 keys at d = 64 over 3 splits: ten 64-key tiles in chunks of 4 for both dtypes
    assert _plan(lib, 1, 1, 1, 1, 640, 64, 3, dtype=2)[:2] == (0, 3)
    assert _plan(lib, 1, 4, 4, 1, 100, 256, 0, dtype=2)[:2] == (0, 1)


@pytest.mark.parametrize("args,expected", [
    ((1, 8, 3, 1, 64, 64, 0), 2), ((1, 8, 8, 0, 64, 64, 0), 2), ((1, 8, 8, 65, 64, 64, 0), 2),
    ((1, 8, 8, 1, 64, 64, -1), 2), ((1, 8, 8, 1, 64, 512, 0), 3), ((1, 8, 8, 1, 64, 64, 0, 0), 3),
    ((1, 8, 8, 1, 64, 64, 0, 3), 3), ((1, 8, 8, 1, 64, 96, 0, 2), 3), ((1, 8, 3, 1, 64, 64, 0, 2), 2),
])
def test_fa_fwd_split_plan_validation(lib, args, expected):
    assert _plan(lib, *args)[0] == expected


@pytest.mark.parametrize("kw,expected", [
    ({"q": 0}, 1), ({"ws": 0}, 1), ({"N_q": 5, "N_k": 4}, 2), ({"H_kv": 3}, 2), ({"d": 512}, 3), ({"dtype": 0}, 3),
    ({"dtype": 2}, 3), ({"o": FAKE + 2}, 4), ({"ws": FAKE + 8}, 4), ({"scale": float("nan")}, 5),
])
def test_fa_fwd_split_validation(lib, kw, expected):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=FAKE, B=1, H=4, H_kv=2, N_q=1, N_k=64, d=64, scale=0.1,
             causal=0, splits=0, dtype=1)
    a.update(kw)
    args = [a[n] for n in ("q", "k", "v", "o", "lse", "ws", "B", "H", "H_kv", "N_q", "N_k", "d", "scale", "causal",
                           "splits", "dtype")] + [None]
    assert lib.fa_fwd_split(*args) == expected


@pytest.mark.parametrize("kw,expected", [
    ({"q": 0}, 1), ({"v": 0}, 1), ({"ws": 0}, 1), ({"N_q": 5, "N_k": 4}, 2), ({"H_kv": 3}, 2), ({"B": 0}, 2),
    ({"d": 512}, 3), ({"d": 96}, 3), ({"k": FAKE + 1}, 4), ({"ws": FAKE + 8}, 4), ({"scale": float("nan")}, 5),
    ({"dq": 0.0}, 5), ({"dk": -1.0}, 5), ({"dv": float("inf")}, 5), ({"dq": float("nan")}, 5),
    ({"scale": 3e38, "dq": 1e3}, 5),
])
def test_fa_fwd_split_fp8_validation(lib, kw, expected):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=FAKE, B=1, H=4, H_kv=2, N_q=1, N_k=64, d=64, scale=0.1,
             dq=1.0, dk=1.0, dv=1.0, causal=0, splits=0)
    a.update(kw)
    args = [a[n] for n in ("q", "k", "v", "o", "lse", "ws", "B", "H", "H_kv", "N_q", "N_k", "d", "scale", "dq", "dk",
                           "dv", "causal", "splits")] + [None]
    assert lib.fa_fwd_split_fp8(*args) == expected


@pytest.mark.parametrize("args,expected", [
    ((0, FAKE, 2, 4, 64, FAKE, FAKE, 1), 1), ((FAKE, FAKE, 0, 4, 64, FAKE, FAKE, 1), 2),
    ((FAKE, FAKE, 2, 0, 64, FAKE, FAKE, 1), 2), ((FAKE, FAKE, 2, 4, 5000, FAKE, FAKE, 1), 2),
    ((FAKE, FAKE, 2, 4, 64, FAKE, FAKE, 2), 3), ((FAKE, FAKE + 4, 2, 4, 64, FAKE, FAKE, 1), 4),
])
def test_fa_lse_merge_validation(lib, args, expected):
    assert lib.fa_lse_merge(*args, None) == expected


@pytest.mark.parametrize("kw,expected", [
    ({"slopes": 0}, 1), ({"q": 0}, 1), ({"dtype": 3}, 3), ({"dtype": -1}, 3), ({"d": 96}, 3), ({"N": 0}, 2),
    ({"dtype": 0, "d": 256}, 3),
    ({"slopes": FAKE + 2}, 4), ({"scale": float("inf")}, 5),
])
def test_fa_fwd_alibi_validation(lib, kw, expected):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, slopes=FAKE, B=1, H=2, N=64, d=64, scale=0.1, causal=0, dtype=1)
    a.update(kw)
    args = [a[n] for n in ("q", "k", "v", "o", "lse", "slopes", "B", "H", "N", "d", "scale", "causal", "dtype")]
    assert lib.fa_fwd_alibi(*args, None) == expected


@pytest.mark.parametrize("kw,expected", [
    ({"mask": 0}, 1), ({"o": 0}, 1), ({"sb": -1}, 2), ({"sh": -5}, 2), ({"dtype": 3}, 3), ({"d": 32}, 3),
    ({"dtype": 0, "d": 256}, 3),
    ({"q": FAKE + 8}, 4), ({"scale": float("nan")}, 5),
])
def test_fa_fwd_blocksparse_validation(lib, kw, expected):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, mask=FAKE + 1, sb=0, sh=0, B=1, H=2, N=64, d=64, scale=0.1,
             causal=0, dtype=1)
    a.update(kw)
    args = [a[n] for n in ("q", "k", "v", "o", "lse", "mask", "sb", "sh", "B", "H", "N", "d", "scale", "causal",
                           "dtype")]
    assert lib.fa_fwd_blocksparse(*args, None) == expected


@pytest.mark.parametrize("kw,expected", [
    ({"slopes": 0}, 1), ({"v": 0}, 1), ({"d": 96}, 3), ({"H": 0}, 2), ({"slopes": FAKE + 1}, 4),
    ({"dq": 0.0}, 5), ({"dk": -1.0}, 5), ({"dv": float("inf")}, 5), ({"scale": float("nan")}, 5),
])
def test_fa_fwd_alibi_fp8_validation(lib, kw, expected):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, slopes=FAKE, B=1, H=2, N=64, d=256, scale=0.1, dq=1.0,
             dk=1.0, dv=1.0, causal=1)
    a.update(kw)
    args = [a[n] for n in ("q", "k", "v", "o", "lse", "slopes", "B", "H", "N", "d", "scale", "dq", "dk", "dv",
                           "causal")]
    assert lib.fa_fwd_alibi_fp8(*args, None) == expected


@pytest.mark.parametrize("kw,expected", [
    ({"mask": 0}, 1), ({"lse": 0}, 1), ({"sb": -1}, 2), ({"N": -4}, 2), ({"d": 512}, 3), ({"o": FAKE + 2}, 4),
    ({"dq": -0.5}, 5), ({"dv": float("nan")}, 5),
])
def test_fa_fwd_blocksparse_fp8_validation(lib, kw, expected):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, mask=FAKE + 1, sb=0, sh=0, B=1, H=2, N=64, d=128, scale=0.1,
             dq=1.0, dk=1.0, dv=1.0, causal=0)
    a.update(kw)
    args = [a[n] for n in ("q", "k", "v", "o", "lse", "mask", "sb", "sh", "B", "H", "N", "d", "scale", "dq", "dk",
                           "dv", "causal")]
    assert lib.fa_fwd_blocksparse_fp8(*args, None) == expected


def test_split_noalloc_rejects_oversized_requests_before_any_launch(lib):
    cap = lib.fa_split_scratch_bytes()
    assert cap == 32 << 20
    # 64 splits of B*H*N_q = 8192 rows at d = 128 need 64 * 8192 * 129 * 4 bytes > 32 MiB
    need = ctypes.c_int64()
    st = lib.fa_fwd_split_plan(8, 1024, 1024, 1, 65536, 128, 64, 1, None, ctypes.byref(need))
    assert st == 0 and need.value > cap
    st = lib.fa_fwd_split_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 1024, 1024, 1, 65536, 128, 0.1, 1, 64, 1, None)
    assert st == 7
    assert lib.fa_status_string(7).decode().startswith("FA_ERR_SCRATCH")
    # argument errors keep fa_fwd_split's codes
    assert lib.fa_fwd_split_noalloc(0, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 64, 128, 0.1, 1, 0, 1, None) == 1
    assert lib.fa_fwd_split_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 2, 1, 128, 0.1, 1, 0, 1, None) == 2
    assert lib.fa_fwd_split_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 64, 96, 0.1, 1, 0, 1, None) == 3
    assert lib.fa_fwd_split_noalloc(FAKE + 8, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 64, 128, 0.1, 1, 0, 1, None) == 4
    # bf16 only, as fa_fwd_split
    assert lib.fa_fwd_split_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 64, 128, 0.1, 1, 0, 2, None) == 3
    # fa_fwd_split still requires its workspace
    assert lib.fa_fwd_split(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 1, 1, 1, 64, 128, 0.1, 1, 0, 1, None) == 1
