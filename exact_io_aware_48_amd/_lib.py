"""ctypes view of libfa_fwd.so: the C ABI declared in include/fa_fwd.h, fa_bwd.h and fa_split.h, nothing else."""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_fwd.so")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_SCALE, FA_ERR_HIP, FA_ERR_SCRATCH = range(8)
FA_F32, FA_BF16, FA_FP8_E4M3 = 0, 1, 2

_lib = None


def load():
    """Load the in-tree library; raise loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_48_amd.build`")
    _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def load_timeline():
    """The diagnostic timeline build (a separate library, loaded beside the
    product one); raise if it has not been built."""
    path = os.path.join(os.path.dirname(LIB_PATH), "libfa_fwd_timeline.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_io_aware_48_amd.build --timeline`")
    return _declare(ctypes.CDLL(path))


def load_probe():
    """The issue-rate microbenchmarks (libfa_probe.so, a diagnostic library of
    their own, csrc/fa_issue_probe.hip); raise if they have not been built."""
    path = os.path.join(os.path.dirname(LIB_PATH), "libfa_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_io_aware_48_amd.build --probes`")
    lib = ctypes.CDLL(path)
    i32, i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    pf = ctypes.POINTER(ctypes.c_float)
    lib.fa_probe_mixed_count.argtypes = []
    lib.fa_probe_mixed_count.restype = i32
    lib.fa_probe_mixed_name.argtypes = [i32]
    lib.fa_probe_mixed_name.restype = ctypes.c_char_p
    lib.fa_probe_mixed_work.argtypes = [i32, ctypes.POINTER(i32)]
    lib.fa_probe_mixed_work.restype = i32
    lib.fa_probe_mixed.argtypes = [i32, vp, i64, i32, i32, pf]
    lib.fa_probe_mixed.restype = i32
    lib.fa_probe_roles.argtypes = [i32, vp, i64, i32, i32, pf]
    lib.fa_probe_roles.restype = i32
    return lib


def _declare(lib):
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i32, vp]
    lib.fa_fwd.restype = i32
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, f32, f32, f32, i32, vp]
    lib.fa_fwd_fp8.restype = i32
    lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, i32, vp]
    lib.fa_fwd_gqa.restype = i32
    lib.fa_fwd_gqa_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, f32, f32, f32, i32, vp]
    lib.fa_fwd_gqa_fp8.restype = i32
    pi, pl = ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int64)
    lib.fa_plan.argtypes = [i64, i64, i64, i64, i32, i32, pi, pi, pl, pi, pi, pl]
    lib.fa_plan.restype = i32
    lib.fa_status_string.argtypes = [i32]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_fwd_alibi.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i32, vp]
    lib.fa_fwd_alibi.restype = i32
    lib.fa_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, i32, i32, vp]
    lib.fa_fwd_blocksparse.restype = i32
    lib.fa_fwd_alibi_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, f32, f32, f32, i32, vp]
    lib.fa_fwd_alibi_fp8.restype = i32
    lib.fa_fwd_blocksparse_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, f32, f32, f32,
                                           i32, vp]
    lib.fa_fwd_blocksparse_fp8.restype = i32
    lib.fa_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, pl]
    lib.fa_bwd_workspace_size.restype = i32
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, i32, vp]
    lib.fa_bwd.restype = i32
    lib.fa_fwd_split_plan.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32, pi, pl]
    lib.fa_fwd_split_plan.restype = i32
    lib.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, i32, i32, i32, vp]
    lib.fa_fwd_split.restype = i32
    lib.fa_fwd_split_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, f32, f32, f32, i32, i32,
                                     vp]
    lib.fa_fwd_split_fp8.restype = i32
    lib.fa_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, i32, i32, i32, vp]
    lib.fa_fwd_split_noalloc.restype = i32
    lib.fa_split_scratch_bytes.argtypes = []
    lib.fa_split_scratch_bytes.restype = i64
    lib.fa_lse_merge.argtypes = [vp, vp, i64, i64, i64, vp, vp, i32, vp]
    lib.fa_lse_merge.restype = i32
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i32
    lib.fa_timeline_read.argtypes = [vp, i64]
    lib.fa_timeline_read.restype = i32
    return lib
