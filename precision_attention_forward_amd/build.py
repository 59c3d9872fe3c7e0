"""Build the gfx950 shared library ``libattnfp4.so`` from ``csrc/*.hip``.

Run as ``python -m precision_attention_forward_amd.build`` or through
``__graft_entry__.build()``.  Objects go to ``_build/`` at the repository
root; the library is written next to this file so that it travels with the
source tree.

``python -m precision_attention_forward_amd.build --phase-trace`` builds the
diagnostic ``libattnfp4_trace.so`` instead: the same objects, except that the
forward attention kernel is compiled with ``-DATTN_FWD_PHASE_TRACE`` (per-wave
shader-clock stamps of its key-loop phases, read by ``bench.py
--phase-trace``).  The product library is never built that way.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattnfp4.so")
TRACE_LIB = os.path.join(PKG, "libattnfp4_trace.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed FP32 instructions (see DESIGN notes); hipcc's host pass warns, harmlessly
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every float rounding in the quantizers and the score path is explicit
    "-ffp-contract=off",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src, obj, extra=()):
    cmd = [_hipcc(), *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(lib, objs):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def _sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose=True, jobs=None):
    """Compile every HIP source for gfx950 and link libattnfp4.so.  Always
    recompiles (it is the build check)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2) // 2), 8)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s), os.path.join(BUILD, s + ".o")) for s in srcs]
        for f in futs:
            objs.append(f.result())
    _link(LIB, objs)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


def build_phase_trace(verbose=True):
    """Link libattnfp4_trace.so: the regular objects (built first) with the
    forward attention kernel recompiled under -DATTN_FWD_PHASE_TRACE."""
    build(verbose=False)
    traced = "fwd_lowp.hip"
    obj = _compile(os.path.join(CSRC, traced), os.path.join(BUILD, traced + ".trace.o"),
                   extra=("-DATTN_FWD_PHASE_TRACE",))
    objs = [obj if s == traced else os.path.join(BUILD, s + ".o") for s in _sources()]
    _link(TRACE_LIB, objs)
    if verbose:
        print(f"built {TRACE_LIB} (forward key-loop phase trace)")
    return TRACE_LIB


if __name__ == "__main__":
    if "--phase-trace" in sys.argv[1:]:
        build_phase_trace()
    else:
        build()
    sys.exit(0)
