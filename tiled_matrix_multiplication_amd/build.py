"""Build libtmm.so in-tree with hipcc for gfx950.

Each csrc/*.hip file is compiled to an object under _build/ (in parallel),
then linked into tiled_matrix_multiplication_amd/libtmm.so; the measurement
kernels under probes/ become libtmm_probes.so.  Run as
``python tiled_matrix_multiplication_amd/build.py`` (not through the package,
whose import loads the library this script replaces).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtmm.so")
PROBES = os.path.join(PKG, "probes")
PROBE_LIB = os.path.join(PKG, "libtmm_probes.so")
ARCH = "gfx950"

CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    hipcc = _hipcc()
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    if not srcs:
        raise RuntimeError("no HIP sources in " + CSRC)

    def compile_one(src: str) -> str:
        obj = os.path.join(OUT_DIR, src[:-4] + ".o")
        cmd = [hipcc, *CXXFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probes(hipcc, verbose)
    return LIB


def build_probes(hipcc: str, verbose: bool = False) -> str:
    """The measurement kernels (include/tmm_probes.h) as libtmm_probes.so."""
    srcs = sorted(os.path.join(PROBES, f) for f in os.listdir(PROBES) if f.endswith(".hip"))
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc, *CXXFLAGS, "-shared", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on the probes:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
