"""Build libmoe_mi355x.so (the C-ABI library) from csrc/*.hip with hipcc for gfx950.

Run ``python -m routing_align_sort_amd.build`` (or ``__graft_entry__.build()``).
Objects go to ``_build/`` at the repository root; the library is written next
to this file, where the Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
# a separate copy kernel of known traffic, used to calibrate profiler byte counters
PROBE_SRC = os.path.join(PKG, "probe", "copy_probe.hip")
PROBE_LIB = os.path.join(PKG, "libmoe_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ops stay off: all fp32 vector math is scalar per lane
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, extra, build_dir) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip() and os.environ.get("MOE_BUILD_VERBOSE"):
        sys.stderr.write(r.stderr)
    return obj


def build(verbose: bool = False, extra=(), out: str = LIB, build_dir: str = BUILD_DIR) -> str:
    """Compile every kernel source and link the shared library; returns its path.

    ``extra`` adds hipcc flags (e.g. -D overrides of the kernels' tuning macros);
    ``out`` / ``build_dir`` redirect the library and the objects."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    extra = list(extra)
    if verbose:
        extra += ["-Rpass-analysis=kernel-resource-usage"]
        os.environ["MOE_BUILD_VERBOSE"] = "1"
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), srcs))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if out == LIB:
        build_probe()
    return out


def build_probe() -> str:
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-shared", "-o", tmp, PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
