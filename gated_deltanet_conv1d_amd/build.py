"""Build libgdn.so in-tree with hipcc for gfx950 (MI355X).

    python -m gated_deltanet_conv1d_amd.build        # or build() from Python

Every .hip/.cpp source under csrc/ is compiled to an object in _build/ (in
parallel), then linked into gated_deltanet_conv1d_amd/libgdn.so.  No JIT
cache: the built library travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "libgdn.so")
ARCH = "gfx950"

# -packed-fp32-ops off: hipcc -O3 would otherwise emit packed fp32 math by
# itself; the kernels are written for scalar fp32 VALU and MFMA.
# -disable-promote-alloca-to-lds: keep per-thread register arrays (prefetched
# rows, accumulator tiles) in registers; the kernels size their own LDS.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=fast",
             "-mllvm", "-disable-promote-alloca-to-lds"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _compile(src: str, obj: str) -> str:
    cmd = [_hipcc(), *HIP_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, csrc: str = CSRC, lib: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source under csrc and link them into lib (defaults: the
    package's sources and libgdn.so; the launch-shape tuner builds variants
    of a copied source tree elsewhere)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.cpp")))
    objs = [os.path.join(build_dir, os.path.basename(s) + ".o") for s in srcs]
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(_compile, srcs, objs))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources", file=sys.stderr)
    return lib


if __name__ == "__main__":
    build()
