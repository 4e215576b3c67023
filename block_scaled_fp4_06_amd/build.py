"""Build libnvfp4.so in-tree with hipcc for gfx950.

    python -m block_scaled_fp4_06_amd.build

Flags: -ffp-contract=off keeps a*b+c unfused so the kernels round exactly like a plain
IEEE evaluation; packed-FP32 instructions are disabled (``-packed-fp32-ops``).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnvfp4.so")
ARCH = os.environ.get("NVFP4_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra) + [
        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp] + sources()
    subprocess.check_call(cmd, cwd=ROOT)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(extra=sys.argv[1:]))
