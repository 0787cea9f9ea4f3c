"""The diagnostic timeline build (-DFA_TIMELINE): its forward computes
exactly what the product build computes, and every workgroup of a launch
leaves one record with ordered stamps and its own (head, row block).
Skipped when libfa_fwd_timeline.so has not been built."""

import os

import numpy as np
import pytest
import torch

import exact_io_aware_48_amd as fa
from exact_io_aware_48_amd import _lib
from gpu_util import to_device
from workloads import by_name, make_inputs

pytestmark = pytest.mark.gpu

TIMELINE = os.path.join(os.path.dirname(_lib.LIB_PATH), "libfa_fwd_timeline.so")


@pytest.mark.skipif(not os.path.exists(TIMELINE), reason="timeline build not present")
@pytest.mark.parametrize("name,B,H,N", [("gpt2s_causal_bf16_b8h12n1024d64", 2, 3, 1000),
                                         ("long_causal_bf16_b1h32n8192d128", 1, 4, 2000),
                                         ("wide_bf16_b2h8n16384d256", 1, 2, 1500)])
def test_timeline_records_every_workgroup_and_changes_no_result(name, B, H, N):
    import ctypes
    print("CASE timeline", name, B, H, N, flush=True)
    w = by_name(name).with_(B=B, H=H, N=N)
    x = make_inputs(w)
    q, k, v = to_device(x)
    o_ref, l_ref = fa.fa_fwd(q, k, v, scale=w.softmax_scale, causal=w.causal)
    tl = _lib.load_timeline()
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert tl.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, w.d,
                     w.softmax_scale, int(w.causal), 1, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    grid = ctypes.c_int64()
    i32 = ctypes.c_int
    assert tl.fa_plan(B, H, N, w.d, int(w.causal), 1, ctypes.byref(i32()), ctypes.byref(i32()), ctypes.byref(grid),
                      ctypes.byref(i32()), ctypes.byref(i32()), ctypes.byref(ctypes.c_int64())) == 0
    buf = np.zeros(grid.value * 6, dtype=np.uint64)
    assert tl.fa_timeline_read(buf.ctypes.data, buf.nbytes) == 0
    t = buf.reshape(-1, 6).astype(np.int64)
    assert np.all(t[:, 0] > 0)
    assert np.all(np.diff(t[:, :4], axis=1) >= 0), "stamps out of order"
    heads_rows = sorted(zip((t[:, 5] & 0xFFFFFFFF).tolist(), (t[:, 5] >> 32).tolist()))
    nrb = grid.value // (B * H)
    assert heads_rows == [(bh, rb) for bh in range(B * H) for rb in range(nrb)]
