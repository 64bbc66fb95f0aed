"""Build the HIP library in-tree: mla_paged_decode_02_amd/lib/libmla_decode.so.

    python -m mla_paged_decode_02_amd.build        # or: python mla_paged_decode_02_amd/build.py

Compiles for gfx950 only.  Packed fp32 VALU ops are disabled in device code
(``-packed-fp32-ops``); the host pass warns that it does not know the feature,
which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libmla_decode.so")
SOURCES = [os.path.join(CSRC, "mla_kernels.hip"), os.path.join(CSRC, "mla_host.cpp")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required)")


def compile_flags() -> list[str]:
    return [
        "--offload-arch=gfx950",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-I", CSRC,
        "-Wall",
        "-Wno-unused-function",
    ]


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc()] + compile_flags() + SOURCES + ["-o", tmp]
    t = time.time()
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "--hip-link" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{msgs}")
    os.replace(tmp, LIB)
    if verbose:
        if msgs.strip():
            print(msgs)
        print(f"built {LIB} in {time.time() - t:.1f}s")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
