"""UndefinedBehaviorSanitizer runs of the host code (no GPU needed).

* The C ABI's argument layer (csrc/api.hip) is compiled for the host only, with the kernel
  launchers replaced by stubs (tests/native/launch_stubs.hip) that launch nothing, and
  driven by tests/native/abi_ubsan_main.c with overflowing, wrapping and extreme sizes and
  strides, the largest accepted shapes and out-of-range status codes.
* The CPU oracle (oracle/nvfp4_oracle.c) is compiled with gcc and run by
  tests/native/oracle_ubsan_main.c over edge-value tensors with every option.

Both builds halt on the first sanitizer report, so a clean exit means none was made.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "block_scaled_fp4_06_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
ENV = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_layer_under_ubsan(tmp_path):
    d = str(tmp_path)
    # host-only compilation: each -fsanitize option applies to the host side alone
    host = [HIPCC, "--offload-host-only", "-O1", "-g", "-std=c++17",
            "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
            "-I", INCLUDE, "-I", CSRC, "-c"]
    _run(host + [os.path.join(CSRC, "api.hip"), "-o", "api.o"], d)
    _run(host + [os.path.join(NATIVE, "launch_stubs.hip"), "-o", "stubs.o"], d)
    _run([CLANG, "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
          "-fsanitize=undefined", "-fno-sanitize-recover=all", "-I", INCLUDE, "-c",
          os.path.join(NATIVE, "abi_ubsan_main.c"), "-o", "main.o"], d)
    _run([CLANG + "++", "-fsanitize=undefined", "main.o", "api.o", "stubs.o",
          "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", "abi_ubsan"], d)
    r = subprocess.run([os.path.join(d, "abi_ubsan")], capture_output=True, text=True,
                       timeout=120, env=ENV)
    assert r.returncode == 0 and "abi ubsan ok" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr, r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_ubsan(tmp_path):
    d = str(tmp_path)
    oracle_dir = os.path.join(ROOT, "oracle")
    _run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fsanitize=undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
          "-I", oracle_dir, os.path.join(oracle_dir, "nvfp4_oracle.c"),
          os.path.join(NATIVE, "oracle_ubsan_main.c"), "-lm", "-o", "oracle_ubsan"], d)
    r = subprocess.run([os.path.join(d, "oracle_ubsan")], capture_output=True, text=True,
                       timeout=300, env=ENV)
    assert r.returncode == 0 and "oracle ubsan ok" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr, r.stderr
