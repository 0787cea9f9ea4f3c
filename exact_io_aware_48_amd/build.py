"""Build step: compile the HIP sources into the in-tree shared libraries.

    python -m exact_io_aware_48_amd.build [--timeline | --probes | --all]

produces ``exact_io_aware_48_amd/libfa_fwd.so`` for gfx950 (``--timeline``:
the diagnostic build ``libfa_fwd_timeline.so``, whose forward kernels stamp
their phases, see fa_timeline_read; ``--probes``: ``libfa_probe.so``, the
issue-rate microbenchmarks of ``csrc/fa_issue_probe.hip`` that
``bench.py --issue-probes`` runs; ``--all``: the three).  It always
recompiles (a build check must not trust a stale binary).
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa_fwd.so")
# diagnostic build with per-workgroup timeline stamps (-DFA_TIMELINE)
LIB_TIMELINE = os.path.join(PKG, "libfa_fwd_timeline.so")
# diagnostic microbenchmarks (not part of the product library)
LIB_PROBE = os.path.join(PKG, "libfa_probe.so")
PROBE_SOURCE = os.path.join(CSRC, "fa_issue_probe.hip")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, f) for f in ("fa_api.hip", "fa_var_api.hip", "fa_bwd_api.hip", "fa_split_api.hip")]
HEADERS = [os.path.join(CSRC, h) for h in ("fa_common.hpp", "fa_tile.hpp", "fa_fwd_kernel.hpp", "fa_pipe_kernel.hpp",
                                           "fa_launch.hpp", "fa_bwd_kernel.hpp", "fa_split_kernel.hpp",
                                           "fa_host.hpp")] + \
    [os.path.join(INCLUDE, h) for h in ("fa_fwd.h", "fa_bwd.h", "fa_split.h")]
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         # keep the compiler from forming packed-fp32 VALU ops
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_cmd(src, obj, extra=()):
    """One translation unit to an object file."""
    return [hipcc(), *FLAGS, f"-I{INCLUDE}", "-c", "-o", obj, src, *extra]


def link_cmd(objs, out):
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out, *objs]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")


def build(verbose=False, jobs=None, timeline=False):
    """Compile every source (in parallel) and link the library (timeline=True:
    the diagnostic timeline build, a separate file)."""
    from concurrent.futures import ThreadPoolExecutor
    out = LIB_TIMELINE if timeline else LIB
    extra = ["-DFA_TIMELINE"] if timeline else []
    tmpdir = tempfile.mkdtemp(prefix="fa_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            list(pool.map(_run, [compile_cmd(src, obj, extra) for src, obj in zip(SOURCES, objs)]))
        tmp = out + ".tmp"
        _run(link_cmd(objs, tmp))
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    if verbose:
        print(f"built {out}")
    return out


def build_probes(verbose=False):
    """Compile the issue-rate microbenchmarks into their own library."""
    tmpdir = tempfile.mkdtemp(prefix="fa_build_")
    try:
        obj = os.path.join(tmpdir, "fa_issue_probe.o")
        _run(compile_cmd(PROBE_SOURCE, obj))
        tmp = LIB_PROBE + ".tmp"
        _run(link_cmd([obj], tmp))
        os.replace(tmp, LIB_PROBE)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    if verbose:
        print(f"built {LIB_PROBE}")
    return LIB_PROBE


def build_all(verbose=False):
    """The product library, its timeline build and the probe library."""
    return [build(verbose), build(verbose, timeline=True), build_probes(verbose)]


if __name__ == "__main__":
    args = sys.argv[1:]
    if "--all" in args:
        build_all(verbose=True)
    elif "--probes" in args:
        build_probes(verbose=True)
    else:
        build(verbose=True, timeline="--timeline" in args)
