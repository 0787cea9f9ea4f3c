"""The forward captured in a HIP graph: every replay equals an eager launch.

A serving loop (and bench.py --graph) issues the forward as HIP graph replays,
so a replay must compute exactly what an eager launch computes.  Each replay here runs on fresh
input contents written in place between replays (with other eager work in
between, as a serving loop would have), and is compared bitwise with an eager
launch on the same inputs: the kernel is deterministic, so any difference is a
capture or replay fault.
"""

import pytest
import torch

import exact_io_aware_48_amd as fa
from workloads import by_name, make_inputs
from gpu_util import to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,B,H,N", [("gpt2s_causal_bf16_b8h12n1024d64", 2, 3, 333),
                                         ("wide_fp8_b2h8n16384d256", 1, 2, 200)])
def test_graph_replays_match_eager(name, B, H, N):
    w = by_name(name).with_(B=B, H=H, N=N)
    print("CASE graph", name, B, H, N, flush=True)
    x = make_inputs(w)
    q, k, v = to_device(x)
    o = torch.empty((B, H, N, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def launch(oo, ll):
        if w.dtype == "fp8":
            return fa.fa_fwd_fp8(q, k, v, *x.descale, o=oo, lse=ll, scale=w.softmax_scale, causal=w.causal)
        return fa.fa_fwd(q, k, v, o=oo, lse=ll, scale=w.softmax_scale, causal=w.causal)

    launch(o, lse)                      # warm: the library caches its device queries
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(o, lse)
    gen = torch.Generator(device="cuda").manual_seed(7)
    for r in range(4):
        # new input contents in place (permuted rows of the originals, so dtypes and ranges stay valid)
        perm = torch.randperm(N, device="cuda", generator=gen)
        for t in (q, k, v):
            raw = t.view(torch.uint8 if w.dtype == "fp8" else torch.int16)   # bit-exact row shuffle
            raw.copy_(raw[:, :, perm].clone())
        scratch = torch.randn(1 << 20, device="cuda").sum()    # unrelated eager work between replays
        o_e = torch.empty_like(o)
        lse_e = torch.empty_like(lse)
        launch(o_e, lse_e)
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert torch.equal(o, o_e), f"replay {r}: O differs from the eager launch"
        assert torch.equal(lse, lse_e), f"replay {r}: L differs from the eager launch"
