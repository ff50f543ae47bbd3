"""Builds libsfa.so (the HIP library behind include/sfa.h) for gfx950 with hipcc.

Every ``csrc/*.hip`` unit is compiled separately (in parallel) and linked into
``sparse_attention_13_amd/libsfa.so``; ``ubench/*.hip`` (the ceiling microbenchmarks) into
``libsfa_ubench.so``.  Run ``python -m sparse_attention_13_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsfa.so")
UBENCH = os.path.join(PKG, "ubench")
UBENCH_LIB = os.path.join(PKG, "libsfa_ubench.so")
ARCH = os.environ.get("SFA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs rather than AGPRs: no AGPR <-> VGPR copies around the
    # softmax rescale and the chunk loop, and fewer registers per wave
    "-mllvm", "--amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(os.path.dirname(src)) + "_" + os.path.basename(src) + ".o")
    cmd = [hipcc()] + FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
    return obj


def _link(objs, lib: str):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, lib)


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compiles all HIP units and links libsfa.so (the library) and libsfa_ubench.so (the
    ceiling microbenchmarks of bench.py --ceilings); always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    usrcs = sorted(glob.glob(os.path.join(UBENCH, "*.hip")))
    jobs = jobs or min(len(srcs) + len(usrcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs + usrcs))
    _link(objs[: len(srcs)], LIB)
    _link(objs[len(srcs):], UBENCH_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} units and {UBENCH_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
