"""Build libdash.so (HIP for gfx950) in-tree with hipcc.

    python -m long_context_sparse_stage0_amd.build

Every source is compiled for gfx950 only.  Packed-fp32 VALU forms are disabled for the
device code (-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import ctypes
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdash.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast", "-munsafe-fp-atomics",
    # never let the compiler move per-thread arrays into LDS behind our back: an array it
    # cannot keep in registers should show up as scratch in the resource report instead
    "-mllvm", "-disable-promote-alloca-to-lds",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(OBJ, os.path.basename(src) + ".o")
        cmd = [hipcc, *FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose:
            errs = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
            if errs:
                print("\n".join(errs))
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # resolve every symbol now: a kernel whose host-side launch stub the compiler dropped
    # links fine but cannot be loaded
    try:
        ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    except OSError as e:
        raise RuntimeError(f"the built library does not load: {e}") from None
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
