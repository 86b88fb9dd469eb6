"""Pins for the oracle's INT8-weight linear layer (comfyui-wiki news page,
单张 4090 配置, and the huaweicloud blog, section 3.5 table: DiT weights stored
INT8, linear layers computed in BF16)."""
import math
from fractions import Fraction

import numpy as np

import oracle
from oracle import brute
import synth


def _inputs(M, K, N, seed=61, scale=None):
    x = synth.random_bf16(seed, (M, K))
    g = np.random.default_rng(seed)
    codes = g.integers(-127, 128, size=(N, K), dtype=np.int8)
    s = (np.abs(g.standard_normal(N)) * 0.01 + 1e-3).astype(np.float32) if scale is None else scale
    return x, codes, s


def test_matches_brute_force():
    x, codes, s = _inputs(5, 48, 7)
    y = oracle.w8a16_linear(x, codes, s)
    xf = oracle.bf16_bits_to_f64(x).tolist()
    for n in range(7):
        w = [brute.round_bf16(brute.round_f32(Fraction(int(c)) * Fraction(float(s[n])))) for c in codes[n]]
        for m in range(5):
            ref = math.fsum(a * b for a, b in zip(xf[m], w))
            assert abs(y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_unit_scale_is_the_integer_code_matrix():
    """scale 1: every weight is its integer code, exactly representable."""
    x, codes, _ = _inputs(9, 64, 5, seed=62)
    y = oracle.w8a16_linear(x, codes, np.ones(5, np.float32))
    xf = oracle.bf16_bits_to_f64(x)
    ref = np.array([[math.fsum(xf[m, k] * int(codes[n, k]) for k in range(64)) for n in range(5)] for m in range(9)])
    np.testing.assert_allclose(y, ref, rtol=1e-15, atol=0)


def test_power_of_two_scales_scale_output_columns():
    """A power-of-two scale is exact in the dequantisation, so output column n
    is the code product times scale n: the scale belongs to the output
    channel, not to the input channel."""
    x, codes, _ = _inputs(6, 32, 4, seed=63)
    s = np.array([2.0 ** -7, 2.0 ** -3, 1.0, 2.0 ** -10], np.float32)
    y = oracle.w8a16_linear(x, codes, s)
    base = oracle.w8a16_linear(x, codes, np.ones(4, np.float32))
    np.testing.assert_array_equal(y, base * s.astype(np.float64)[None, :])


def test_rows_subset():
    x, codes, s = _inputs(20, 32, 6, seed=64)
    y = oracle.w8a16_linear(x, codes, s)
    np.testing.assert_array_equal(oracle.w8a16_linear(x, codes, s, rows=[3, 17]), y[[3, 17]])
