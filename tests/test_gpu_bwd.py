"""GPU parity of nomas_seg_attn_bwd (gradients of packed segment-causal
attention, segment-forcing training: huaweicloud blog, section 2.3) against
the CPU oracle.  The forward outputs it consumes come from nomas_seg_attn on
the GPU; the expected gradients come from the oracle alone.

Parity bar for the fp32 gradients: relative L2 error <= 5e-3 per tensor and
max-abs error <= 2e-2 times the tensor's largest magnitude.  The kernels
round P and dS to bf16 (relative 2^-9 per term) before their products and
take D from the forward's bf16 output; sums are fp32.  Where a gradient is
exactly zero (a token alone in its segment has P = 1 and dS = 0), the
relative error has no meaning; its max-abs error is then bounded by 2e-2
times the largest magnitude among the case's three gradients."""
import numpy as np
import pytest
import torch

import oracle
import segment_causal_attention_amd as nomas
import synth
from gpu_util import SM, dev16, say

pytestmark = pytest.mark.gpu

GRAD_REL_L2 = 5e-3
GRAD_MAX_REL = 2e-2


def _grads_gpu(q, k, v, d_out, segs, H, sm=SM):
    Ln = q.shape[0]
    qd, kd, vd, dd = dev16(q), dev16(k), dev16(v), dev16(d_out)
    lse = torch.empty((H, Ln), dtype=torch.float32, device="cuda:0")
    out = nomas.seg_attn(qd, kd, vd, segs, cache_len=0, sm_scale=sm, lse=lse)
    dq, dk, dv = nomas.seg_attn_bwd(qd, kd, vd, out, lse, dd, segs, sm_scale=sm)
    torch.cuda.synchronize()
    return [t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]


def _close(got, ref, what, case_scale=0.0):
    assert np.all(np.isfinite(got)), "%s: non-finite gradient" % what
    d = got - ref
    scale = float(np.abs(ref).max())
    mx = float(np.abs(d).max())
    nref = float(np.linalg.norm(ref))
    rl2 = float(np.linalg.norm(d) / nref) if nref > 0 else 0.0
    say("%s: max-abs %.3e (of max %.3e) rel-L2 %.3e" % (what, mx, scale, rl2))
    assert rl2 <= GRAD_REL_L2 and mx <= GRAD_MAX_REL * max(scale, case_scale), (what, mx, scale, rl2)


def _close3(got, ref, name):
    case_scale = max(float(np.abs(r).max()) for r in ref)
    for g, r, w in zip(got, ref, ("dq", "dk", "dv")):
        _close(g, r, "%s %s" % (name, w), case_scale)


def _check(name, segs, H, seed, sm=SM):
    L = sum(s[0] + s[2] * s[3] * s[4] for s in segs)
    q, k, v, d_out = (synth.random_bf16(seed + i, (L, H, 128)) for i in range(4))
    say("seg_attn_bwd", name, "L", L, "H", H, "segs", segs[:4], "sm_scale", sm)
    got = _grads_gpu(q, k, v, d_out, segs, H, sm)
    ref = oracle.seg_attn_bwd(q, k, v, d_out, segs, sm)
    _close3(got, ref, name)


def test_bwd_tiny_three_segments():
    inp = synth.tiny_inputs()
    segs = [s.astuple() for s in inp["segs"]]
    d_out = synth.random_bf16(77, inp["q"].shape)
    say("seg_attn_bwd tiny (3 x 64 tokens, H 2)")
    got = _grads_gpu(inp["q"], inp["k"], inp["v"], d_out, segs, 2)
    ref = oracle.seg_attn_bwd(inp["q"], inp["k"], inp["v"], d_out, segs, SM)
    _close3(got, ref, "tiny")


CASES = [
    # ragged segments: partial tiles, a workgroup with idle waves, text-only and one-token segments
    ("ragged", [(5, 0, 3, 7, 9), (0, 3, 2, 5, 11), (37, 0, 0, 1, 1), (1, 0, 0, 1, 1)], 3),
    # an empty segment between two others, a single-segment sequence
    ("empty-middle", [(20, 0, 2, 6, 10), (0, 0, 0, 0, 0), (3, 2, 1, 9, 14)], 2),
    ("one-segment", [(0, 0, 5, 8, 9)], 2),
    ("one-token", [(1, 0, 0, 0, 0)], 1),
    # several workgroups per segment (1,472 tokens each) and late positions
    ("three-turns", [(64, 18 * i, 2, 22, 32) for i in range(3)], 2),
    ("late-t", [(3, 16000, 2, 7, 5), (0, 9, 1, 30, 33)], 2),
    # 16 heads; segment lengths that are whole tiles (64 and 128 tokens)
    ("heads16", [(10, 0, 1, 10, 20), (5, 1, 1, 10, 20)], 16),
    ("tile-aligned", [(64, 0, 0, 1, 1), (0, 0, 2, 8, 8), (0, 2, 1, 8, 8)], 2),
    # 40 small segments: long segment tables, one workgroup per segment
    ("forty-segments", [(1 + (i % 3), i, 1, 2 + (i % 2), 3) for i in range(40)], 2),
    # the 64-segment limit
    ("sixty-four-segments", [(i % 5, i, 1, 3, 2 + (i % 3)) for i in range(64)], 2),
]


@pytest.mark.parametrize("name,segs,H", CASES, ids=[c[0] for c in CASES])
def test_bwd_matches_oracle(name, segs, H):
    _check(name, segs, H, 500 + 7 * len(name))


@pytest.mark.parametrize("sm", [0.3, 0.02])
def test_bwd_softmax_scale(sm):
    """A sharp softmax (0.3: scores spread over tens of log units, P close to
    one-hot) and a flat one (0.02)."""
    _check("scale-%g" % sm, [(9, 0, 2, 6, 7), (4, 2, 1, 6, 7)], 2, 700, sm)


def test_bwd_mask_invariance_bitwise():
    """dq of segments 0-1 is bitwise unchanged when every input of segment 2
    changes (even to NaN keys and values); dk and dv of segments 1-2 are
    bitwise unchanged when q and dO of segment 0 change."""
    segs = [(10, 0, 2, 5, 7), (0, 2, 1, 9, 9), (4, 3, 2, 6, 6)]
    n = [s[0] + s[2] * s[3] * s[4] for s in segs]
    L, H = sum(n), 2
    q, k, v, d_out = (synth.random_bf16(900 + i, (L, H, 128)) for i in range(4))
    say("seg_attn_bwd invariance", segs)
    base = _grads_gpu(q, k, v, d_out, segs, H)
    e1 = n[0] + n[1]
    q2, k2, v2, d2 = (x.copy() for x in (q, k, v, d_out))
    q2[e1:] = synth.random_bf16(950, q2[e1:].shape, 3.0)
    d2[e1:] = synth.random_bf16(951, d2[e1:].shape, 3.0)
    k2[e1:] = 0x7FC0       # NaN
    v2[e1:] = 0x7FC0
    late = _grads_gpu(q2, k2, v2, d2, segs, H)
    assert np.array_equal(late[0][:e1], base[0][:e1])
    q3, d3 = q.copy(), d_out.copy()
    q3[:n[0]] = synth.random_bf16(960, q3[:n[0]].shape, 3.0)
    d3[:n[0]] = synth.random_bf16(961, d3[:n[0]].shape, 3.0)
    early = _grads_gpu(q3, k, v, d3, segs, H)
    assert np.array_equal(early[1][n[0]:], base[1][n[0]:])
    assert np.array_equal(early[2][n[0]:], base[2][n[0]:])


def test_bwd_training_sequence_full_size():
    """The packed training sequence at full size (22 turns of 16,096 tokens,
    354,112 tokens, one GPU's 2 heads of a head-sharded layer): dq on rows
    sampled in every segment against the oracle row by row, and identities
    of softmax attention that hold at any size for dk and dv:
    sum_k dv_k = sum_q dO_q and sum_k R dk_k = 0, and dk, dv element by
    element on sampled keys of the last segment."""
    segs = [s.astuple() for s in synth.train_segs()]
    H = 2
    inp = synth.train_inputs(synth.train_segs(), H)
    q, k, v, d_out = inp["q"], inp["k"], inp["v"], inp["d_out"]
    L = q.shape[0]
    say("seg_attn_bwd full training sequence L", L, "H", H)
    dq, dk, dv = _grads_gpu(q, k, v, d_out, segs, H)
    assert all(np.all(np.isfinite(g)) for g in (dq, dk, dv))
    ends = np.cumsum([s[0] + s[2] * s[3] * s[4] for s in segs])
    starts = np.concatenate([[0], ends[:-1]])
    rng = np.random.Generator(np.random.PCG64(5))
    rows = np.unique(np.concatenate([starts, ends - 1, starts + 255, starts + 256,
                                     rng.integers(0, L, 20)]))
    ref, _, _ = oracle.seg_attn_bwd(q, k, v, d_out, segs, SM, rows=rows, want_kv=False)
    _close(dq[rows], ref, "full dq (%d sampled rows)" % len(rows))
    # sum_k dv_k = sum_q dO_q (rows of P sum to one)
    dof = oracle.bf16_bits_to_f64(d_out)
    lhs, rhs = dv.sum(axis=0), dof.sum(axis=0)
    tol = 1e-6 * np.abs(dof).sum(axis=0)
    say("full sum dv: max |diff| %.3e, max tol %.3e" % (np.abs(lhs - rhs).max(), tol.max()))
    assert np.all(np.abs(lhs - rhs) <= tol)
    # sum_k dKr_k = 0 (rows of dS sum to zero), against the size of the terms
    dkr = oracle.rope3d(dk, segs)
    s, a = np.abs(dkr.sum(axis=0)), np.abs(dkr).sum(axis=0)
    say("full sum dKr: max |sum| / sum |.| = %.3e" % (s / a).max())
    assert np.all(s <= 1e-3 * a)
    # dk and dv element by element on keys of the last segment (the oracle
    # forms the whole softmax rows of the 16,096 queries that see them)
    keys = np.unique(np.concatenate([[starts[-1], starts[-1] + 63, starts[-1] + 64, starts[-1] + 255,
                                      starts[-1] + 256, ends[-1] - 1], rng.integers(starts[-1], L, 26)]))
    _key_grads("full", q, k, v, d_out, segs, H, keys, dk, dv)


def _key_grads(name, q, k, v, d_out, segs, H, keys, dk, dv):
    """dk, dv of the GPU at `keys` against the oracle's key-subset mode,
    head by head."""
    for h in range(H):
        say("%s: oracle dk, dv on %d keys, head %d" % (name, len(keys), h))
        _, rdk, rdv = oracle.seg_attn_bwd(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], d_out[:, h:h + 1], segs,
                                          SM, keys=keys)
        _close(dk[keys][:, h:h + 1], rdk, "%s dk head %d (%d keys)" % (name, h, len(keys)))
        _close(dv[keys][:, h:h + 1], rdv, "%s dv head %d (%d keys)" % (name, h, len(keys)))


def test_bwd_six_turns_first_segment_keys():
    """Six packed turns of 1 s (6 latent frames + 256 text tokens: 5,536
    tokens each, 33,216 in all, 2 heads): dk and dv of keys in the first
    segment, which every later query tile of the sequence sees (the longest
    walk of the dK/dV kernel), element by element."""
    tsegs = synth.train_segs(6, T=6)
    segs = [s.astuple() for s in tsegs]
    H = 2
    inp = synth.train_inputs(tsegs, H, inst=1)
    q, k, v, d_out = inp["q"], inp["k"], inp["v"], inp["d_out"]
    L = q.shape[0]
    say("seg_attn_bwd six turns L", L, "H", H)
    dq, dk, dv = _grads_gpu(q, k, v, d_out, segs, H)
    assert all(np.all(np.isfinite(g)) for g in (dq, dk, dv))
    n0 = segs[0][0] + segs[0][2] * segs[0][3] * segs[0][4]
    rng = np.random.Generator(np.random.PCG64(6))
    keys = np.unique(np.concatenate([[0, 1, 255, 256, segs[0][0], n0 - 64, n0 - 1], rng.integers(0, n0, 25)]))
    _key_grads("six turns", q, k, v, d_out, segs, H, keys, dk, dv)
