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


def build(out: str = LIB, extra=(), timeline_out: str | None = None) -> str:
    """Compile every source to an object (in parallel, one hipcc per file), then link.

    timeline_out: also link a test-only variant of the library there, whose quantize
    kernels are compiled with NVFP4_TIMELINE (phase timestamps; nvfp4_timeline_attach)."""
    tmp = out + ".tmp%d" % os.getpid()
    objs, procs = [], []

    def compile_(src, obj, more=()):
        cmd = [hipcc()] + [f for f in HIPCC_FLAGS if f != "-shared"] + list(extra) + list(more) + [
            "-c", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", obj, src]
        procs.append((src, subprocess.Popen(cmd, cwd=ROOT)))

    for src in sources():
        obj = "%s.%d.%d.o" % (out, os.getpid(), len(objs))
        objs.append(obj)
        compile_(src, obj)
    tl_obj = None
    if timeline_out:
        tl_obj = "%s.%d.timeline.o" % (out, os.getpid())
        compile_(os.path.join(CSRC, "quantize.hip"), tl_obj, ["-DNVFP4_TIMELINE=1"])
    try:
        for src, pr in procs:
            if pr.wait() != 0:
                raise subprocess.CalledProcessError(pr.returncode, "hipcc " + src)
        subprocess.check_call([hipcc()] + HIPCC_FLAGS + list(extra) + ["-o", tmp] + objs,
                              cwd=ROOT)
        os.replace(tmp, out)
        if timeline_out:
            qobj = objs[sources().index(os.path.join(CSRC, "quantize.hip"))]
            tl_objs = [tl_obj if o == qobj else o for o in objs]
            tmp2 = timeline_out + ".tmp%d" % os.getpid()
            subprocess.check_call([hipcc()] + HIPCC_FLAGS + list(extra) + ["-o", tmp2] + tl_objs,
                                  cwd=ROOT)
            os.replace(tmp2, timeline_out)
    finally:
        for pr in procs:
            if pr[1].poll() is None:
                pr[1].kill()
        for o in objs + ([tl_obj] if tl_obj else []):
            if os.path.exists(o):
                os.remove(o)
    return out


if __name__ == "__main__":
    print(build(extra=sys.argv[1:]))
