"""The division-free Q8_1 block rule of the kernels, checked on the CPU.

The kernels reach d = RN(amax / 127) and every RN(x / d) without a division
instruction, by Markstein's theorem (a correctly rounded reciprocal, one
product, one exact fma residual, one fma correction).  These tests run the same
formulas in plain C (IEEE fp32, correctly rounded fmaf) against the IEEE
division: exhaustively over binades for amax / 127 and over every significand
for the Newton-refined reciprocal, and over every x in [1, 4) for sampled
divisors.  Both identities are scale-invariant away from underflow, and the
kernels keep every operand normal (blocks with amax < 2^-60 are scaled by
2^64 first), so the binades checked stand for all of them.  The GPU parity
tests compare the kernels' Q8_1 bytes with the oracle, which divides.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "markstein_check.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler on this host")
    exe = str(tmp_path_factory.mktemp("markstein") / "markstein_check")
    # no contraction: every fma in the source is an explicit fmaf
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-fno-fast-math", SRC, "-o", exe, "-lm"],
                   check=True, capture_output=True)
    return exe


def _run(exe, *args):
    res = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=600)
    return tuple(map(int, res.stdout.split()))[1:]


def test_d_equals_division_denormals_and_binades(checker):
    # every denormal, and every float in [2^-3, 2^9) (covers amax of unit-scale
    # activations and the rounding of 1/127 at every significand)
    tested, bad = _run(checker, 1, -3, 9)
    assert tested == (1 << 23) * 13 and bad == 0


def test_newton_reciprocal_is_correctly_rounded(checker):
    """Every start within an ulp of 1/d lands on RN(1/d), save one: the lower
    neighbour (1/2) of 1/d for the all-ones significand d = 2 - 2^-23, where
    1/d lies just above the midpoint of 1/2 and its upper neighbour.  The
    kernels therefore rely on the hardware reciprocal not returning that
    neighbour; on the GPU the reciprocal plus the step equals RN(1/d) for every
    normal d below 2^126 (the kernels' d is at most 2^121)."""
    tested, bad, exception = _run(checker, 2)
    assert tested == 2 * (1 << 23) and bad == 0 and exception == 1


def test_quotients_equal_division(checker):
    tested, bad = _run(checker, 3, 24)
    assert tested == 24 * (1 << 24) and bad == 0
