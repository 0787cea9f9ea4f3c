"""Build step: compile the HIP sources into the in-tree shared library.

    python -m exact_io_aware_48_amd.build

produces ``exact_io_aware_48_amd/libfa_fwd.so`` for gfx950.  It always
recompiles (a build check must not trust a stale binary).
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa_fwd.so")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, f) for f in ("fa_api.hip", "fa_bwd_api.hip", "fa_split_api.hip")]
HEADERS = [os.path.join(CSRC, h) for h in ("fa_common.hpp", "fa_tile.hpp", "fa_fwd_kernel.hpp", "fa_pipe_kernel.hpp",
                                           "fa_bwd_kernel.hpp",
                                           "fa_split_kernel.hpp", "fa_host.hpp")] + \
    [os.path.join(INCLUDE, h) for h in ("fa_fwd.h", "fa_bwd.h", "fa_split.h")]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_cmd(out=LIB, extra=()):
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep the compiler from forming packed-fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}", "-o", out, *SOURCES, *extra,
    ]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = compile_cmd(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
