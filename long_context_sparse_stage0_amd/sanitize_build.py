"""Build the host-sanitizer check of the C ABI (CPU only).

    python -m long_context_sparse_stage0_amd.sanitize_build

Compiles the library's host-side argument validation (csrc/dash_api.cpp) together with
sanitize_driver.cpp with AddressSanitizer and UndefinedBehaviorSanitizer on the HOST pass
only (each sanitizer flag follows -Xarch_host; device code is built as usual), links the
other kernel sources unsanitised, and returns the path of the executable.  The driver only
makes calls that fail validation or query workspace sizes, so it runs without a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

from . import build as B

EXE = os.path.join(B.OBJ, "sanitize_check")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized() -> str:
    hipcc = B._hipcc()
    os.makedirs(B.OBJ, exist_ok=True)
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"]
    objs = []
    for src in B.sources():
        base = os.path.basename(src)
        if base == "dash_api.cpp":
            obj = os.path.join(B.OBJ, "dash_api.san.o")
            cmd = [hipcc, *flags, *HOST_SAN, "-c", src, "-o", obj]
        else:
            obj = os.path.join(B.OBJ, base + ".o")
            if os.path.exists(obj) and os.path.getmtime(obj) >= os.path.getmtime(src):
                objs.append(obj)
                continue
            cmd = [hipcc, *B.FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
        objs.append(obj)
    drv = os.path.join(B.PKG, "sanitize_driver.cpp")
    dobj = os.path.join(B.OBJ, "sanitize_driver.o")
    cmd = [hipcc, "-O1", "-g", "-std=c++17", *HOST_SAN, "-I", os.path.join(B.ROOT, "include"),
           "-c", drv, "-o", dobj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    cmd = [hipcc, f"--offload-arch={B.ARCH}", *HOST_SAN, "-o", EXE, dobj, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    return EXE


if __name__ == "__main__":
    exe = build_sanitized()
    print(exe)
    sys.exit(subprocess.run([exe]).returncode)
