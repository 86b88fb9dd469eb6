"""Pins for the oracle's INT8 quantiser (cached K/V stored as INT8: comfyui-wiki
news page, 单张 4090 配置; huaweicloud blog, section 3.5 table).  Reading:
symmetric absmax/127, one fp32 scale per (token, head), rne with the exact
quotient, codes in [-127, 127]."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute
import synth


def _all_positive_bf16():
    bits = np.arange(0x0080, 0x7F80, dtype=np.uint16)      # normal, finite, > 0
    a = oracle.bf16_bits_to_f64(bits)
    return a[a >= 2.0 ** -100]     # keep a/127 a normal float32 (the workloads' range)


def test_scale_is_the_exactly_rounded_quotient_for_every_bf16():
    """fl32(a/127) taken through a float64 quotient equals the float32
    rounding of the exact rational a/127, for every positive bf16 a."""
    a = _all_positive_bf16()
    got = (a / 127.0).astype(np.float32)
    for av, gv in zip(a[::1], got[::1]):
        assert float(gv) == brute.round_f32(Fraction(av) / 127)


def test_matches_exact_rational_brute_force():
    inp = synth.tiny_inputs()
    rng = np.random.default_rng(3)
    rows = [oracle.bf16_bits_to_f64(inp["k"][j, h]) for j in range(0, 192, 5) for h in range(2)]
    # outlier-like rows and tiny-magnitude rows
    big = oracle.bf16_round(rng.standard_normal((6, 128)) * np.where(rng.random(128) < 0.02, 20.0, 1.0))
    small = oracle.bf16_round(rng.standard_normal((4, 128)) * 1e-3)
    rows += list(big) + list(small)
    X = np.stack(rows)
    q, s = oracle.quantise(X)
    for i, r in enumerate(X):
        qb, sb = brute.quantise_row([float(v) for v in r])
        assert float(s[i]) == sb
        assert list(q[i].astype(int)) == qb


def test_round_trip_is_bit_exact():
    rng = np.random.default_rng(4)
    X = oracle.bf16_round(rng.standard_normal((500, 128)) * rng.exponential(1.0, (500, 1)))
    q, s = oracle.quantise(X)
    q2, s2 = oracle.quantise(oracle.dequant(q, s))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_error_bound_and_full_range():
    rng = np.random.default_rng(5)
    X = oracle.bf16_round(rng.standard_normal((500, 128)))
    q, s = oracle.quantise(X)
    err = np.abs(X - oracle.dequant(q, s))
    assert np.all(err <= s[:, None].astype(np.float64) / 2 * (1 + 1e-12))
    assert np.all(np.abs(q).max(axis=1) == 127)
    assert q.min() >= -127


def test_zero_row():
    q, s = oracle.quantise(np.zeros((2, 128)))
    assert np.all(q == 0) and np.all(s == 0)


def test_ties_round_to_even():
    x = np.zeros(128)
    x[0] = 127.0                          # scale exactly 1.0
    x[1:9] = [2.5, 3.5, 0.5, 1.5, -2.5, -3.5, -0.5, 126.5]
    q, s = oracle.quantise(x[None])
    assert float(s[0]) == 1.0
    assert list(q[0, :9]) == [127, 2, 4, 0, 2, -2, -4, 0, 126]


def test_exact_when_values_are_multiples_of_the_scale():
    rng = np.random.default_rng(6)
    k = rng.integers(-127, 128, 128)
    k[17] = 127
    x = k / 8.0                             # scale 127/8/127 = 1/8
    q, s = oracle.quantise(x[None])
    assert float(s[0]) == 0.125
    assert np.array_equal(q[0].astype(int), k)


def test_dequant_bf16_operand():
    """bf16(fl32(q*s)): the fp32 product then one RNE rounding to bf16."""
    rng = np.random.default_rng(7)
    q = rng.integers(-127, 128, (50, 128)).astype(np.int8)
    s = (rng.random(50) * 0.05).astype(np.float32)
    got = oracle.dequant_bf16(q, s)
    for i in range(0, 50, 7):
        for c in range(0, 128, 11):
            p = brute.round_f32(Fraction(int(q[i, c])) * Fraction(float(s[i])))
            assert got[i, c] == brute.round_bf16(p)
