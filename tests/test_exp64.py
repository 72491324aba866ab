"""Accuracy of the samplers' float64 exp (csrc/exp64.hpp), compiled for the host.

The proposal sampler sums exp(logit - max) in float64 with a table-driven
exp of its own; its draws agree with a float64 inverse CDF only if that exp
is accurate to a few units in the last place.  This sweep compares it with
the C library's exp over [-746, 0] (4 million points) and checks the special
cases: exp(0) = 1 exactly, -inf, NaN (the difference of two -inf logits) and arguments past the underflow threshold
give 0, results in the subnormal range are within two subnormal steps.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "introspective_strided_decoding_amd", "csrc")


@pytest.fixture(scope="module")
def sweep(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("exp64") / "exp64_check")
    subprocess.run([cxx, "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", CSRC, os.path.join(ROOT, "tests", "native", "exp64_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return {line.split()[0]: [float(v) for v in line.split()[1:]] for line in out.splitlines()}


def test_relative_error_a_few_ulp(sweep):
    assert sweep["worst_rel"][0] < 1e-15


def test_subnormal_results(sweep):
    assert sweep["worst_abs_subnormal"][0] <= 2 * 4.9406564584124654e-324


def test_special_cases(sweep):
    assert sweep["exp0"][0] == 1.0
    assert sweep["exp_minus_tiny"][0] == 1.0
    assert sweep["exp_minus_inf"][0] == 0.0
    assert sweep["exp_nan"][0] == 0.0
    assert sweep["exp_minus_800"][0] == 0.0
    assert sweep["exp_minus_745_3"][0] == 0.0        # below half the smallest subnormal
    a, b = sweep["exp_minus_1"]
    assert abs(a - b) <= 2.3e-16 * b
