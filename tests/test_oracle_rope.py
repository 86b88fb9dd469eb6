"""Pins for the oracle's 3D RoPE (comfyui-wiki news page, 模型内部: 3D RoPE
[16, 56, 56], theta 256): closed forms, identity at position 0, relative
position property, and agreement with the pure-Python brute force."""
import math

import numpy as np
import pytest

import oracle
from oracle import brute
import synth


def test_t_axis_frequencies_are_powers_of_two():
    # 256^(-2i/16) = 2^-i exactly
    np.testing.assert_allclose(oracle.rope_omega(0), 2.0 ** -np.arange(8), rtol=2e-16, atol=0)


def test_hw_axis_frequencies_closed_form():
    for a in (1, 2):
        om = oracle.rope_omega(a)
        assert om.shape == (28,)
        assert om[0] == 1.0
        # 256^(-2i/56) = 2^(-2i/7): i = 7, 14, 21 give 1/4, 1/16, 1/64
        np.testing.assert_allclose(om[[7, 14, 21]], [0.25, 1 / 16, 1 / 64], rtol=2e-16)
        np.testing.assert_allclose(om, 2.0 ** (-2.0 * np.arange(28) / 7), rtol=4e-16)


@pytest.mark.parametrize("axis,i", [(0, 0), (0, 3), (0, 7), (1, 0), (1, 5), (1, 27), (2, 1), (2, 13), (2, 27)])
def test_unit_vector_rotates_by_p_omega(axis, i):
    """e_{2i} of chunk `axis` at position p goes to (cos p w_i, sin p w_i) in
    the pair's two channels, e_{2i+1} to (-sin, cos); nothing else moves."""
    seg = (0, 5, 1, 7, 9)            # a single video frame at t=5, 7x9 grid
    vid, t, h, w = oracle.token_positions([seg])
    tok = 4 * 9 + 6                  # h = 4, w = 6
    p = (t[tok], h[tok], w[tok])[axis]
    off = oracle.AXIS_OFFSETS[axis]
    ang = p * 256.0 ** (-2.0 * i / oracle.AXES[axis])
    for which, expect in ((0, (math.cos(ang), math.sin(ang))), (1, (-math.sin(ang), math.cos(ang)))):
        x = np.zeros((len(vid), 1, 128))
        x[tok, 0, off + 2 * i + which] = 1.0
        y = oracle.rope3d_pos(x, vid, t, h, w)[tok, 0]
        np.testing.assert_allclose(y[off + 2 * i: off + 2 * i + 2], expect, atol=1e-15)
        rest = np.delete(y, [off + 2 * i, off + 2 * i + 1])
        assert np.all(rest == 0)


def test_text_tokens_and_origin_are_identity():
    segs = [(5, 0, 1, 2, 3)]
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5 + 6, 2, 128))
    y = oracle.rope3d(x, segs)
    assert np.array_equal(y[:5], x[:5])          # text
    assert np.array_equal(y[5], x[5])            # video token at (0, 0, 0)
    assert not np.allclose(y[6], x[6])           # (0, 0, 1) moves


def test_pair_norms_preserved():
    rng = np.random.default_rng(1)
    segs = [(0, 3, 2, 4, 5)]
    x = rng.standard_normal((40, 3, 128))
    y = oracle.rope3d(x, segs)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-13)


def test_relative_position_property():
    """<R(p) q, R(p') k> depends on p - p' only (per axis)."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    one = np.ones(1, bool)

    def score(pq, pk):
        rq = oracle.rope3d_pos(q, one, *[np.array([v]) for v in pq])
        rk = oracle.rope3d_pos(k, one, *[np.array([v]) for v in pk])
        return float(np.sum(rq * rk))

    for _ in range(20):
        pq = rng.integers(0, 300, 3)
        pk = rng.integers(0, 300, 3)
        dlt = rng.integers(-200, 200, 3)
        dlt = np.maximum(dlt, -np.minimum(pq, pk))      # keep positions >= 0
        s0, s1 = score(pq, pk), score(pq + dlt, pk + dlt)
        assert abs(s0 - s1) <= 1e-12 * max(1.0, abs(s0)) * 100


def test_matches_brute_force_on_tiny():
    inp = synth.tiny_inputs()
    segs = [s.astuple() for s in inp["segs"]]
    x = oracle.bf16_bits_to_f64(inp["k"])
    y = oracle.rope3d(x, segs)
    pos = brute.positions(segs)
    for j in range(0, len(pos), 7):
        for h in range(2):
            yb = brute.rope_vec([float(v) for v in x[j, h]], pos[j])
            np.testing.assert_allclose(y[j, h], yb, rtol=0, atol=1e-14)
