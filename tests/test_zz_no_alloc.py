"""fa_fwd_split_noalloc (partials in the library's fixed per-GPU array) against
fa_fwd_split (partials in a caller workspace), through the C ABI.

Same split count, same kernels: the outputs must be bitwise equal.  Two calls
in a row, the second on a smaller problem, check that the array keeps no
state a call depends on (the split kernel writes every partial the merge
reads).  Each call is also held to the bf16 tolerances against the float64
oracle on every element.
"""

import ctypes

import numpy as np
import pytest
import torch

from oracle import attention_decode_gqa, errors
from workloads import DECODE_WORKLOADS

from gpu_util import check, to_device

pytestmark = pytest.mark.gpu


def _abi():
    from exact_io_aware_48_amd import _lib
    return _lib.load(), _lib


def _run_both(x, num_splits, causal=True):
    lib, L = _abi()
    w = x.workload
    q, k, v = to_device(x)
    B, H, N_q, d = q.shape
    H_kv, N_k = k.shape[1], k.shape[2]
    stream = torch.cuda.current_stream().cuda_stream
    # fa_fwd_split with a workspace
    splits, nbytes = ctypes.c_int(), ctypes.c_int64()
    assert lib.fa_fwd_split_plan(B, H, H_kv, N_q, N_k, d, num_splits, L.FA_BF16, ctypes.byref(splits),
                                 ctypes.byref(nbytes)) == L.FA_OK
    assert nbytes.value <= lib.fa_split_scratch_bytes()
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device="cuda")
    o_ref = torch.empty_like(q)
    l_ref = torch.empty((B, H, N_q), dtype=torch.float32, device="cuda")
    st = lib.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ref.data_ptr(), l_ref.data_ptr(),
                          ws.data_ptr(), B, H, H_kv, N_q, N_k, d, w.softmax_scale, int(causal), num_splits,
                          L.FA_BF16, stream)
    assert st == L.FA_OK
    # the same call without a workspace
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N_q), dtype=torch.float32, device="cuda")
    st = lib.fa_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, H, H_kv, N_q, N_k, d, w.softmax_scale, int(causal), num_splits,
                                  L.FA_BF16, stream)
    assert st == L.FA_OK
    torch.cuda.synchronize()
    return o, lse, o_ref, l_ref, splits.value


def test_noalloc_matches_workspace_call_twice_second_smaller():
    big = DECODE_WORKLOADS[0].with_(B=4, H=16, H_kv=4, N_q=4, N=8192, seed=41)
    small = big.with_(B=2, H=8, H_kv=2, N_q=1, N=3000, seed=42)
    from workloads import make_inputs
    for w, splits in ((big, 8), (small, 3)):
        print("CASE noalloc", w.B, w.H, w.kv_heads, w.q_rows, w.N, "splits", splits, flush=True)
        x = make_inputs(w)
        o, lse, o_ref, l_ref, used = _run_both(x, splits)
        assert used == splits
        assert torch.equal(o, o_ref), "O differs from fa_fwd_split's"
        assert torch.equal(lse, l_ref), "lse differs from fa_fwd_split's"
        # and both hold the bf16 tolerances against the oracle, every element
        ro, rl = attention_decode_gqa(x.f64("q"), x.f64("k"), x.f64("v"), w.softmax_scale, True)
        got_o = o.float().cpu().numpy().astype(np.float64)
        got_l = lse.cpu().numpy().astype(np.float64)
        check(errors(got_o, ro, got_l, rl), "bf16", f"noalloc B={w.B} H={w.H}/{w.kv_heads} N_q={w.q_rows} N_k={w.N}")


def test_noalloc_automatic_split_count_and_binding():
    import exact_io_aware_48_amd as fa
    from workloads import make_inputs
    w = DECODE_WORKLOADS[0].with_(B=2, H=8, H_kv=8, N_q=1, N=5000, seed=43)
    x = make_inputs(w)
    q, k, v = to_device(x)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, 1), dtype=torch.float32, device="cuda")
    fa.fa_fwd_split_noalloc(q, k, v, o, lse, scale=w.softmax_scale, causal=True)
    o_ref, l_ref = fa.fa_fwd_split(q, k, v, scale=w.softmax_scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
