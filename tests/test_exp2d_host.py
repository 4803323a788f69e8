"""The acceptance's float64 2^y (csrc/isd_exp2d.hpp), built for the host with
g++ and checked against long double exp2l: the sampling weights it produces
must be float64-accurate for the sampled token to match an exact evaluation.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "speculative_verify_isd_amd", "csrc")


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("exp2d") / "exp2d_host")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, os.path.join(HERE, "exp2d_host.cpp"),
                    "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return {k: float(v) for k, v in (line.split() for line in out.splitlines())}


def test_relative_error_below_one_ulp(results):
    assert results["worst_rel"] < 2.3e-16, results


def test_exact_points(results):
    assert results["at_0"] == 1.0
    assert results["at_1"] == 2.0
    assert results["at_m1"] == 0.5
    assert abs(results["at_half"] - 2 ** 0.5) <= 2.3e-16 * 2 ** 0.5


def test_underflow_and_special_values(results):
    assert results["at_m1074"] == 2.0 ** -1074   # smallest subnormal
    assert results["at_m1075"] == 0.0
    assert results["at_minf"] == 0.0
    assert results["at_nan"] == 0.0               # clamped, never NaN
    assert results["at_1024"] == float("inf")


def test_table_variant(results):
    # exp2t (table of 2^(j/64) and a degree-5 polynomial): a few ulp
    assert results["worst_rel_t"] < 4.5e-16, results
    assert results["t_at_0"] == 1.0 and results["t_at_m1"] == 0.5
    assert results["t_at_m1075"] == 0.0 and results["t_at_nan"] == 0.0


def test_scaled_table_variant_is_bit_identical(results):
    # exp2t64 takes 64 y and power-of-two-scaled coefficients: every step is
    # exp2t's step times a power of two, so the bits agree for y <= 0
    assert results["t64_count"] > 4e6
    assert results["t64_mismatch"] == 0, results
