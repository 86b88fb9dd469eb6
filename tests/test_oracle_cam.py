"""Pins for the oracle's camera path (comfyui-wiki news page, 相机控制作为一等输入:
c2w [N,4,4], normalised, grouped per 4 frames into 64-d tokens that video
tokens query by cross-attention; translation scale 1.0, rotation scale 2.5)."""
import math

import numpy as np

import oracle
from oracle import brute


def rotz(a):
    c, s = math.cos(a), math.sin(a)
    return np.array([[c, -s, 0], [s, c, 0], [0, 0, 1.0]])


def make_path(Rs, ts):
    N = len(Rs)
    m = np.zeros((N, 4, 4))
    for k in range(N):
        m[k, :3, :3], m[k, :3, 3], m[k, 3, 3] = Rs[k], ts[k], 1.0
    return m


def test_static_camera_gives_identity_tokens():
    R0 = rotz(0.7) @ np.array([[1, 0, 0], [0, 0, -1], [0, 1, 0.0]])
    tok = oracle.cam_tokens(make_path([R0] * 8, [np.array([1.0, 2, 3])] * 8))
    assert tok.shape == (2, 64)
    np.testing.assert_allclose(tok, np.tile(np.eye(4).reshape(16), 4)[None].repeat(2, 0), atol=1e-14)


def test_translation_relative_to_first_frame_and_scaled():
    R0 = rotz(0.3)
    v = np.array([0.5, -1.0, 2.0])
    path = make_path([R0] * 4, [np.array([3.0, 1, 0]) + k * v for k in range(4)])
    for scale in (1.0, 2.0):
        tok = oracle.cam_tokens(path, translation_scale=scale).reshape(4, 4, 4)
        for k in range(4):
            np.testing.assert_allclose(tok[k, :3, 3], scale * k * (R0.T @ v), atol=1e-14)
            np.testing.assert_allclose(tok[k, :3, :3], np.eye(3), atol=1e-14)


def test_rotation_angle_scaled_by_2_5():
    a = 0.05
    path = make_path([rotz(0.2 + k * a) for k in range(8)], [np.zeros(3)] * 8)
    tok = oracle.cam_tokens(path).reshape(8, 4, 4)
    for k in range(8):
        np.testing.assert_allclose(tok[k, :3, :3], rotz(2.5 * k * a), atol=1e-13)
    tok1 = oracle.cam_tokens(path, rotation_scale=1.0).reshape(8, 4, 4)
    np.testing.assert_allclose(tok1[3, :3, :3], rotz(3 * a), atol=1e-13)


def test_single_camera_token_returns_its_value():
    rng = np.random.default_rng(8)
    H = 2
    q = oracle.f64_to_bf16_bits(oracle.bf16_round(rng.standard_normal((10, H, 128))))
    wk = oracle.f64_to_bf16_bits(oracle.bf16_round(rng.standard_normal((64, H * 128)) / 8))
    wv = oracle.f64_to_bf16_bits(oracle.bf16_round(rng.standard_normal((64, H * 128)) / 8))
    cam = rng.standard_normal((1, 64)).astype(np.float32)
    out = oracle.cam_xattn(q, cam, wk, wv, 1 / math.sqrt(128))
    _, Vc = oracle.cam_kv(cam, wk, wv, H)
    np.testing.assert_allclose(out, np.broadcast_to(Vc[0][None], out.shape), atol=1e-15)


def test_matches_brute_force():
    rng = np.random.default_rng(9)
    H, Lq, Nc = 2, 6, 3
    q = oracle.f64_to_bf16_bits(oracle.bf16_round(rng.standard_normal((Lq, H, 128))))
    wk = oracle.f64_to_bf16_bits(oracle.bf16_round(rng.standard_normal((64, H * 128)) / 8))
    wv = oracle.f64_to_bf16_bits(oracle.bf16_round(rng.standard_normal((64, H * 128)) / 8))
    cam = rng.standard_normal((Nc, 64)).astype(np.float32)
    sm = 1 / math.sqrt(128)
    out = oracle.cam_xattn(q, cam, wk, wv, sm)
    qf = oracle.bf16_bits_to_f64(q).tolist()
    ob = brute.cam_xattn(qf, cam.astype(np.float64).tolist(), oracle.bf16_bits_to_f64(wk).tolist(),
                         oracle.bf16_bits_to_f64(wv).tolist(), H, sm)
    np.testing.assert_allclose(out, np.array(ob), atol=1e-12)
    # rows of the camera softmax sum to one: values that are the same for every
    # camera token (only weight row 0 is non-zero, cam[:, 0] = 1) come back unchanged
    wv1 = np.zeros((64, H * 128), np.uint16)
    wv1[0, :] = oracle.f64_to_bf16_bits(np.full(H * 128, 0.75))
    cam1 = cam.copy()
    cam1[:, 0] = 1.0
    out1 = oracle.cam_xattn(q, cam1, wk, wv1, sm)
    np.testing.assert_allclose(out1, 0.75, rtol=0, atol=1e-15)


def _skew(a):
    x, y, z = a
    return np.array([[0, -z, y], [z, 0, -x], [-y, x, 0.0]])


NEAR_PI_AXES = [np.array([0.3, -0.8, 0.5]), np.array([-0.6, 0.0, 0.8]), np.array([0.0, 0.0, -1.0]),
                np.array([0.2, 0.9, -0.1])]


def near_pi_cases():
    """(c2w path of 4 frames, expected relative rotation of frame 1 after the
    x2.5 angle scale) for rotations of pi - 1e-3, pi - 1e-7 and exactly pi.
    Expected values are matrix exponentials of the scaled skew matrix (scipy),
    not the oracle's own exp; at exactly pi the axis is the one whose largest
    component is positive (the sign convention for a half turn)."""
    import scipy.linalg as sl

    out = []
    R0 = rotz(0.4)
    for a in NEAR_PI_AXES:
        a = a / np.linalg.norm(a)
        for sgn in (1.0, -1.0):
            ax = sgn * a
            for eps in (1e-3, 1e-7, 0.0):
                if eps == 0.0:
                    Rrel = 2.0 * np.outer(ax, ax) - np.eye(3)          # exactly a half turn
                    conv = ax if ax[np.argmax(np.abs(ax))] > 0 else -ax
                    want = sl.expm(2.5 * math.pi * _skew(conv))
                else:
                    Rrel = sl.expm((math.pi - eps) * _skew(ax))
                    want = sl.expm(2.5 * (math.pi - eps) * _skew(ax))
                path = make_path([R0, R0 @ Rrel, R0, R0], [np.zeros(3)] * 4)
                out.append((path, want, (tuple(ax), eps)))
    return out


def test_rotation_near_pi_keeps_its_axis():
    """A relative rotation just short of a half turn keeps its axis sign, so
    the x2.5 scaled rotation is R(a, 2.5 theta) (comfyui-wiki news page,
    相机控制作为一等输入: rotation scale 2.5) all the way to pi; exactly at pi
    the axis with a positive largest component is used."""
    for path, want, case in near_pi_cases():
        tok = oracle.cam_tokens(path).reshape(4, 4, 4)
        np.testing.assert_allclose(tok[1, :3, :3], want, atol=1e-12, err_msg=str(case))
        np.testing.assert_allclose(tok[0, :3, :3], np.eye(3), atol=1e-14)


def test_rotation_scale_continuous_up_to_pi():
    """Tokens of rotations pi - eps about a fixed axis converge to the
    half-turn token R(a, 2.5 pi) as eps -> 0, down to eps = 1e-10 (no jump
    where sin(theta) gets small; the sign convention of a half turn applies
    only within 1e-12 of pi, where rounding decides the sign)."""
    a = np.array([0.3, -0.8, 0.5])
    a /= np.linalg.norm(a)
    import scipy.linalg as sl
    for eps in (1e-2, 1e-4, 1e-6, 1e-8, 1e-10):
        path = make_path([np.eye(3), sl.expm((math.pi - eps) * _skew(a))] + [np.eye(3)] * 2, [np.zeros(3)] * 4)
        tok = oracle.cam_tokens(path).reshape(4, 4, 4)[1, :3, :3]
        lim = sl.expm(2.5 * math.pi * _skew(a))
        assert np.abs(tok - lim).max() <= 2.5 * eps * 1.01 + 1e-12, eps
