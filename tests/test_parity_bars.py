"""The parity bar for results rounded once to bf16 (gpu_util.assert_bf16_output)
admits exactly-rounded outputs at any magnitude and rejects an error of two
bf16 ulps.  Runs on the CPU: the bar is host code."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_bf16_output


def _rounded(ref):
    return oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(oracle.bf16_round(ref)))


def test_exact_bf16_rounding_passes_at_every_magnitude():
    ref = np.random.default_rng(1).standard_normal(200000) * 3.0
    ref[:6] = [9.3, -12.7, 0.001, 1e-6, 15.99, -250.3]
    assert_bf16_output(_rounded(ref), ref, "exact rounding")


def test_two_ulp_error_fails():
    ref = np.random.default_rng(2).standard_normal(1000)
    ref[7] = 12.7                       # bf16 ulp 2^-4 in [8, 16)
    got = _rounded(ref)
    got[7] += 2 * 2.0 ** -4
    with pytest.raises(AssertionError):
        assert_bf16_output(got, ref, "planted")
