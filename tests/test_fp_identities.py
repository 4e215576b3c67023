"""Binary32 identities behind three arithmetic shortcuts of the HIP quantization kernels.

The kernels (1) divide a block amax by 6 with a product and one FMA correction instead
of a division, (2) take the tensor amax after the RHT without forming the last butterfly
stage, using max(|a+b|, |a-b|) = |a| + |b| under monotonic rounding, and (3) fold the
RHT's final 1/4 into the block multiplier; (4) encode stochastic rounding with the
hardware stochastic fp4 conversion after rounding |v| up to a multiple of 2^-23; and (5)
fold that conversion's 2^23 input scale into the block multiplier.  Each shortcut must give bit-identical
results to the plain form that the oracle evaluates (RHT and scale steps of the NVIDIA
developer blog "NVFP4 trains with precision of 16-bit ...", section on the pre-training
quantization recipe).  These are properties of IEEE binary32 arithmetic, checked here on
the CPU by tests/native/fp_identities.c: exhaustively for (1), on random pairs spanning
the whole exponent range for (2), (3) and (5), and for (4) on a sweep of [0, 6) and every
decision point (with the conversion modelled as recorded on the GPU; the GPU tests check
the instruction itself).
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("fpid") / "fp_identities")
    src = os.path.join(HERE, "native", "fp_identities.c")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", src,
                    "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    res = {}
    for line in out.strip().splitlines():
        name, n, bad = line.split()
        res[name] = (int(n), int(bad))
    return res


def test_div6_exhaustive(results):
    n, bad = results["div6"]
    assert n == 0x7F800000 - 0x01000000
    assert bad == 0


def test_absadd_max(results):
    n, bad = results["absadd"]
    assert n == 20_000_000 and bad == 0


def test_quarter_fold(results):
    n, bad = results["quarter"]
    assert n > 10_000_000 and bad == 0


def test_stochastic_code_formula(results):
    # the kernels' stochastic E2M1 encoder (input rounded up to the 2^-23 grid, draw
    # operand 0xFFFF7C00 - (k << 16), conversion as recorded) against the definition
    n, bad = results["srstep"]
    assert n > 200_000_000 and bad == 0


def test_fold23(results):
    n, bad = results["fold23"]
    assert n > 5_000_000 and bad == 0
