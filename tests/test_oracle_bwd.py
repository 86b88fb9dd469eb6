"""Pins for the oracle's backward pass of packed segment-causal attention
(segment-forcing training on packed sequences: huaweicloud blog, section 2.3;
the block-causal mask of the comfyui-wiki news page, 一个世界，分段生成).

The gradient is pinned to things other than its own formula: central finite
differences of the oracle's forward (itself pinned to brute force), torch's
autograd through masked softmax attention, exact invariances of the mask,
identities of softmax attention that hold at any size, and closed forms of
degenerate cases."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

SM = float(np.float32(1 / math.sqrt(128)))


def _rng(seed):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))


def _empty_cache(H):
    z8 = np.zeros((H, 0, 128), np.int8)
    z = np.zeros((H, 0), np.float32)
    return z8, z8, z, z


def _loss(q, k, v, dO, segs, sm):
    """L = sum dO * O for the packed forward without rounding."""
    kc, vc, ks, vs = _empty_cache(q.shape[1])
    out, _ = oracle.seg_attn(q, k, v, segs, kc, vc, ks, vs, 0, sm, bf16_operands=False)
    return float(np.sum(dO * out))


# two segments with text and video tokens on all three RoPE axes
FD_SEGS = [(3, 0, 2, 2, 3), (2, 2, 1, 2, 3)]


def _fd_case(seed=5):
    g = _rng(seed)
    L = sum(s[0] + s[2] * s[3] * s[4] for s in FD_SEGS)
    shp = (L, 2, 128)
    return [g.standard_normal(shp) for _ in range(4)]


@pytest.mark.parametrize("which", [0, 1, 2])
def test_directional_derivatives_match_finite_differences(which):
    """<grad, u> equals (L(x + h u) - L(x - h u)) / 2h for random directions u
    of q, k or v: covers the mask, the softmax, both products and the
    transpose of the rotation."""
    q, k, v, dO = _fd_case()
    sm = 0.25
    grads = oracle.seg_attn_bwd(q, k, v, dO, FD_SEGS, sm, bf16_operands=False)
    x = [q, k, v]
    g = _rng(100 + which)
    h = 1e-5
    for _ in range(3):
        u = g.standard_normal(x[which].shape)
        xp = list(x)
        xm = list(x)
        xp[which] = x[which] + h * u
        xm[which] = x[which] - h * u
        fd = (_loss(*xp, dO, FD_SEGS, sm) - _loss(*xm, dO, FD_SEGS, sm)) / (2 * h)
        an = float(np.sum(grads[which] * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("tok,head,ch", [(0, 0, 5), (4, 1, 3), (9, 0, 40), (20, 1, 100), (13, 1, 127)])
def test_single_coordinates_match_finite_differences(tok, head, ch):
    """Coordinates in a text token and in each RoPE chunk (t: 3, h: 40,
    w: 100, 127) of video tokens of both segments, for q and k."""
    q, k, v, dO = _fd_case(7)
    sm = 0.25
    dq, dk, _ = oracle.seg_attn_bwd(q, k, v, dO, FD_SEGS, sm, bf16_operands=False)
    h = 1e-5
    for grad, idx in ((dq, 0), (dk, 1)):
        xs = [q.copy(), k.copy()]
        xs[idx][tok, head, ch] += h
        lp = _loss(xs[0], xs[1], v, dO, FD_SEGS, sm)
        xs[idx][tok, head, ch] -= 2 * h
        lm = _loss(xs[0], xs[1], v, dO, FD_SEGS, sm)
        fd = (lp - lm) / (2 * h)
        assert abs(fd - grad[tok, head, ch]) <= 1e-6 * max(1.0, abs(fd)), (idx, fd, grad[tok, head, ch])


def test_matches_torch_autograd_on_text_segments():
    """Text-only segments (no rotation): torch float64 autograd through
    softmax attention with the block-causal mask."""
    segs = [(7, 0, 0, 1, 1), (5, 0, 0, 1, 1), (9, 0, 0, 1, 1)]
    g = _rng(11)
    L, H = 21, 2
    q, k, v, dO = (g.standard_normal((L, H, 128)) for _ in range(4))
    dq, dk, dv = oracle.seg_attn_bwd(q, k, v, dO, segs, SM, bf16_operands=False)
    ends = np.cumsum([s[0] for s in segs])
    seg_of = np.searchsorted(ends, np.arange(L), side="right")
    allowed = torch.tensor(np.arange(L)[None, :] < ends[seg_of][:, None])
    tq, tk, tv = (torch.tensor(x.transpose(1, 0, 2).copy(), requires_grad=True) for x in (q, k, v))
    s = (tq @ tk.transpose(1, 2)) * SM
    s = s.masked_fill(~allowed, float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    (o * torch.tensor(dO.transpose(1, 0, 2).copy())).sum().backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)


def _tiny3():
    inp = synth.tiny_inputs()
    d_out = synth.random_bf16(77, inp["q"].shape)
    return [s.astuple() for s in inp["segs"]], inp["q"], inp["k"], inp["v"], d_out


def test_mask_invariances_are_exact():
    """dq of segments 0 and 1 ignores every input of segment 2; dk and dv of
    segments 1 and 2 ignore q and dO of segment 0 (no query of segment 0
    attends to them)."""
    segs, q, k, v, dO = _tiny3()
    dq, dk, dv = oracle.seg_attn_bwd(q, k, v, dO, segs, SM)
    g = _rng(3)
    late = slice(128, 192)
    q2, k2, v2, d2 = (x.copy() for x in (q, k, v, dO))
    for x in (q2, k2, v2, d2):
        x[late] = synth.to_bf16_bits(g.standard_normal(x[late].shape).astype(np.float32) * 4)
    dq2, _, _ = oracle.seg_attn_bwd(q2, k2, v2, d2, segs, SM)
    assert np.array_equal(dq2[:128], dq[:128])
    assert not np.array_equal(dq2[128:], dq[128:])
    q3, d3 = q.copy(), dO.copy()
    for x in (q3, d3):
        x[:64] = synth.to_bf16_bits(g.standard_normal(x[:64].shape).astype(np.float32) * 4)
    _, dk3, dv3 = oracle.seg_attn_bwd(q3, k, v, d3, segs, SM)
    assert np.array_equal(dk3[64:], dk[64:]) and np.array_equal(dv3[64:], dv[64:])
    assert not np.array_equal(dk3[:64], dk[:64])


@pytest.mark.parametrize("bf16_operands", [True, False])
def test_softmax_identities(bf16_operands):
    """Identities of softmax attention, true at any size:
    sum_k dv_k = sum_q dO_q (rows of P sum to one);
    sum_k dKr_k = 0 (rows of dS sum to zero);
    sum_q <Qr_q, dQr_q> = sum_k <Kr_k, dKr_k> (both are sum dS * S)."""
    segs, q, k, v, dO = _tiny3()
    dq, dk, dv = oracle.seg_attn_bwd(q, k, v, dO, segs, SM, bf16_operands=bf16_operands)
    f = oracle.bf16_bits_to_f64
    rnd = oracle.bf16_round if bf16_operands else (lambda a: a)
    np.testing.assert_allclose(dv.sum(axis=0), f(dO).sum(axis=0), rtol=0, atol=1e-11)
    dKr = oracle.rope3d(dk, segs)
    assert np.abs(dKr.sum(axis=0)).max() <= 1e-12 * np.abs(dKr).sum(axis=0).max()
    Qr = rnd(oracle.rope3d(f(q), segs))
    Kr = rnd(oracle.rope3d(f(k), segs))
    dQr = oracle.rope3d(dq, segs)
    lhs = np.einsum("lhc,lhc->h", Qr, dQr)
    rhs = np.einsum("lhc,lhc->h", Kr, dKr)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-11)


def test_transpose_rotation_inverts_rope():
    segs, q, _, _, _ = _tiny3()
    x = oracle.bf16_bits_to_f64(q)
    pos = oracle.token_positions(segs)
    back = oracle.rope3d_pos(oracle.rope3d_pos(x, *pos), *pos, inverse=True)
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-13)


def test_lone_token_and_uniform_values():
    """A token alone in segment 0 sees only itself: P = 1, O = v, dS = 0, so
    its dq is zero.  With every value row equal, dP = D and dS = 0: dq and
    dk vanish.  With every key zero, P is uniform over the allowed keys and
    dv_j = sum over segments a that see j of (sum of dO over a) / (keys of a)."""
    segs = [(1, 0, 0, 1, 1), (4, 0, 1, 2, 2), (3, 1, 1, 2, 2)]
    L, H = 1 + 8 + 7, 2
    g = _rng(21)
    q, k, v, dO = (g.standard_normal((L, H, 128)) for _ in range(4))
    dq, _, _ = oracle.seg_attn_bwd(q, k, v, dO, segs, SM, bf16_operands=False)
    assert np.abs(dq[0]).max() <= 1e-15
    vu = np.broadcast_to(g.standard_normal((1, H, 128)), (L, H, 128)).copy()
    dq, dk, _ = oracle.seg_attn_bwd(q, k, vu, dO, segs, SM, bf16_operands=False)
    assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13
    _, _, dv = oracle.seg_attn_bwd(q, np.zeros_like(k), v, dO, segs, SM, bf16_operands=False)
    ends = np.cumsum([s[0] + s[2] * s[3] * s[4] for s in segs])
    starts = np.concatenate([[0], ends[:-1]])
    want = np.zeros_like(dv)
    for a in range(len(segs)):
        want[:ends[a]] += dO[starts[a]:ends[a]].sum(axis=0) / ends[a]
    np.testing.assert_allclose(dv, want, rtol=0, atol=1e-13)


def test_rows_subset_matches_full():
    segs, q, k, v, dO = _tiny3()
    dq, _, _ = oracle.seg_attn_bwd(q, k, v, dO, segs, SM)
    rows = np.array([0, 17, 63, 64, 100, 191])
    dqs, dks, dvs = oracle.seg_attn_bwd(q, k, v, dO, segs, SM, rows=rows, want_kv=False)
    assert dks is None and dvs is None
    np.testing.assert_allclose(dqs, dq[rows], rtol=0, atol=1e-13)


def test_key_subset_matches_full():
    """The key-subset mode (dk, dv of chosen keys only, for sequences too long
    for the full gradient) equals the full gradients at those keys: keys of
    every segment, segment boundaries and a text-only segment."""
    segs = [(5, 0, 2, 3, 4), (0, 2, 1, 5, 3), (7, 0, 0, 1, 1), (2, 3, 1, 4, 4)]
    L = sum(s[0] + s[2] * s[3] * s[4] for s in segs)
    H = 2
    q, k, v, d = (synth.random_bf16(1300 + i, (L, H, 128)) for i in range(4))
    sm = 1 / math.sqrt(128)
    _, dk, dv = oracle.seg_attn_bwd(q, k, v, d, segs, sm)
    ends = np.cumsum([s[0] + s[2] * s[3] * s[4] for s in segs])
    for keys in ([0, 1, 28], [29, 43, 44, 50, 51, L - 1], [L - 1], list(range(L))):
        dq_s, dk_s, dv_s = oracle.seg_attn_bwd(q, k, v, d, segs, sm, keys=keys)
        assert dq_s is None and dk_s.shape == (len(keys), H, 128)
        np.testing.assert_allclose(dk_s, dk[keys], rtol=0, atol=1e-13 * np.abs(dk).max())
        np.testing.assert_allclose(dv_s, dv[keys], rtol=0, atol=1e-13 * np.abs(dv).max())
    assert ends[-1] == L
