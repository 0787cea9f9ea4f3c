"""The issue-rate microbenchmarks of the probe library (libfa_probe.so,
csrc/fa_issue_probe.hip, run by ``bench.py --issue-probes``): every
configuration launches, finishes and reports a positive time, and a longer
run takes longer.  Skipped when the probe library has not been built."""

import ctypes
import os

import pytest
import torch

from exact_io_aware_48_amd import _lib

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(_lib.LIB_PATH), "libfa_probe.so")
ROLES = (1, 2, 3, 6, 7)


def _out():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return torch.empty(cus * 512, dtype=torch.float32, device="cuda")


@pytest.mark.skipif(not os.path.exists(PROBE), reason="probe library not built")
def test_every_probe_runs():
    lib = _lib.load_probe()
    out, ms = _out(), ctypes.c_float()
    for i in range(lib.fa_probe_mixed_count()):
        print("CASE probe mixed", i, flush=True)
        assert lib.fa_probe_mixed(i, out.data_ptr(), out.numel(), 20, 2, ctypes.byref(ms)) == 0
        assert ms.value > 0
    for r in ROLES:
        print("CASE probe roles", r, flush=True)
        assert lib.fa_probe_roles(r, out.data_ptr(), out.numel(), 20, 2, ctypes.byref(ms)) == 0
        assert ms.value > 0
    assert torch.isfinite(out).all()


@pytest.mark.skipif(not os.path.exists(PROBE), reason="probe library not built")
def test_probe_time_grows_with_iterations():
    lib = _lib.load_probe()
    out, ms = _out(), ctypes.c_float()
    print("CASE probe scaling", flush=True)
    assert lib.fa_probe_mixed(0, out.data_ptr(), out.numel(), 100, 3, ctypes.byref(ms)) == 0
    short = ms.value
    assert lib.fa_probe_mixed(0, out.data_ptr(), out.numel(), 2000, 3, ctypes.byref(ms)) == 0
    assert ms.value > 5 * short
