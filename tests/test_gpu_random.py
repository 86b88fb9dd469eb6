"""Seeded random sweeps of GPU parity against the oracle.

Besides the hand-picked edge cases of the other GPU tests, each entry point
runs on configurations drawn from a fixed generator: segment mixes with
empty, text-only and ragged video segments, cache lengths from none to a few
hundred tokens, forced key-range parts, history selections, 1 to 3 heads,
linear-layer shapes around the GEMM's tile sizes, and random lengths, head
counts, offsets and camera-token counts for the RoPE, quantise-and-append,
camera and grouped-head entry points.  The bars are those of
the hand-picked cases (the helpers are shared with them)."""
import math

import numpy as np
import pytest
import torch

import oracle
import segment_causal_attention_amd as nomas
import synth
from gpu_util import SM, assert_bf16_output, assert_close, bits, cache_tensors, dev, dev16, f64, say
from test_gpu_bwd import _close3, _grads_gpu
from test_gpu_kernels import _check_case

pytestmark = pytest.mark.gpu


def _random_segs(rng, max_segs):
    segs = []
    for _ in range(int(rng.integers(1, max_segs + 1))):
        u = rng.random()
        if u < 0.1:
            segs.append((0, 0, 0, 0, 0))                                   # empty
        elif u < 0.25:
            segs.append((int(rng.integers(1, 80)), 0, 0, 0, 0))            # text only
        else:
            segs.append((int(rng.integers(0, 20)), int(rng.integers(0, 40)), int(rng.integers(1, 5)),
                         int(rng.integers(1, 17)), int(rng.integers(1, 21))))
    if sum(s[0] + s[2] * s[3] * s[4] for s in segs) == 0:
        segs[0] = (1, 0, 0, 0, 0)
    return segs


def _random_sel(rng, n_segs, Lc):
    """Sorted, non-overlapping, non-empty cache-token ranges per segment."""
    sel = []
    for _ in range(n_segs):
        cuts = np.sort(rng.choice(np.arange(Lc + 1), size=2 * int(rng.integers(0, 4)), replace=False))
        sel.append([(int(a), int(b)) for a, b in zip(cuts[0::2], cuts[1::2]) if b > a])
    return sel


def _fwd_config(seed):
    rng = np.random.default_rng(9000 + seed)
    segs = _random_segs(rng, 5)
    H = int(rng.integers(1, 4))
    Lc = 0 if rng.random() < 0.25 else int(rng.integers(1, 400))
    n_split = int(rng.choice([0, 0, 1, 2, 3, 4]))
    sel = _random_sel(rng, len(segs), Lc) if Lc > 1 and rng.random() < 0.4 else None
    return segs, H, Lc, n_split, sel


@pytest.mark.parametrize("seed", range(24))
def test_seg_attn_random_configs(seed):
    segs, H, Lc, n_split, sel = _fwd_config(seed)
    Ln = sum(s[0] + s[2] * s[3] * s[4] for s in segs)
    q, k, v = (synth.random_bf16(9100 + 3 * seed + i, (Ln, H, 128)) for i in range(3))
    cache = None
    if Lc > 0:
        kh = synth.random_bf16(9200 + seed, (Lc, H, 128))
        vh = synth.random_bf16(9300 + seed, (Lc, H, 128))
        cache = oracle.build_cache(kh, vh, [(0, 0, 1, 1, Lc)], cap=Lc + 5)
    _check_case("random-%d %s" % (seed, segs), q, k, v, segs, cache, Lc, H, n_split=n_split, sel=sel)


@pytest.mark.parametrize("seed", range(12))
def test_seg_attn_bwd_random_configs(seed):
    rng = np.random.default_rng(9400 + seed)
    segs = _random_segs(rng, 4)
    H = int(rng.integers(1, 4))
    sm = float(np.float32(rng.choice([1.0 / math.sqrt(128), 0.3, 0.05])))
    L = sum(s[0] + s[2] * s[3] * s[4] for s in segs)
    q, k, v, d_out = (synth.random_bf16(9500 + 4 * seed + i, (L, H, 128)) for i in range(4))
    say("seg_attn_bwd random-%d L %d H %d sm %.4f segs %s" % (seed, L, H, sm, segs))
    got = _grads_gpu(q, k, v, d_out, segs, H, sm)
    ref = oracle.seg_attn_bwd(q, k, v, d_out, segs, sm)
    _close3(got, ref, "random-%d" % seed)


# small calls (128 x 128 tiles throughout) and larger ones (384 x 256 tiles,
# with 128 x 128 tiles for the rows of a short last round where one arises)
W8_SHAPES = [(int(M), int(K), int(N)) for M, K, N in zip(
    np.random.default_rng(9600).integers(0, 2500, 12),
    64 * np.random.default_rng(9601).integers(1, 17, 12),
    256 * np.random.default_rng(9602).integers(1, 5, 12))] + [(int(M), int(K), int(N)) for M, K, N in zip(
    np.random.default_rng(9603).integers(5000, 40000, 4),
    64 * np.random.default_rng(9604).integers(1, 9, 4),
    1024 * np.random.default_rng(9605).integers(1, 4, 4))] + [
    (25000, 256, 1024),     # 264 big tiles: rows from 24,576 on take 128 x 128 tiles
    (13000, 512, 2048)]     # 272 big tiles: rows from 12,288 on take 128 x 128 tiles


@pytest.mark.parametrize("M,K,N", W8_SHAPES, ids=["M%d-K%d-N%d" % s for s in W8_SHAPES])
def test_w8a16_random_shapes(M, K, N):
    say("w8a16 random", M, K, N)
    x = synth.random_bf16(9700 + M, (M, K))
    g = np.random.default_rng(9800 + K + N)
    codes = g.integers(-127, 128, size=(N, K), dtype=np.int8)
    s = (1.0 / (73.0 * math.sqrt(K)) * (0.5 + g.random(N))).astype(np.float32)
    xd = dev16(x) if M else torch.empty((0, K), dtype=torch.int16, device="cuda:0")
    y = nomas.w8a16_linear(xd, dev(codes), dev(s))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (M, N)
    if M:
        assert_bf16_output(f64(y), oracle.w8a16_linear(x, codes, s), "w8a16 M=%d K=%d N=%d" % (M, K, N))


@pytest.mark.parametrize("seed", range(8))
def test_rope3d_random_configs(seed):
    """Bit-level, as the hand-picked rope3d cases: at most one bf16 ulp from
    the oracle's float64 rotation rounded once, in under 1e-5 of the values."""
    rng = np.random.default_rng(9900 + seed)
    segs = _random_segs(rng, 5)
    H = int(rng.integers(1, 17))
    L = sum(s[0] + s[2] * s[3] * s[4] for s in segs)
    x = synth.random_bf16(9910 + seed, (L, H, 128), 3.0)
    say("rope3d random-%d L %d H %d segs %s" % (seed, L, H, segs))
    y = nomas.rope3d(dev16(x), segs)
    torch.cuda.synchronize()
    ref = oracle.f64_to_bf16_bits(oracle.bf16_round(oracle.rope3d(oracle.bf16_bits_to_f64(x), segs)))
    got = bits(y)
    diff = got != ref
    if diff.any():
        assert np.abs(got[diff].astype(np.int32) - ref[diff].astype(np.int32)).max() <= 1
    assert diff.mean() < 1e-5


@pytest.mark.parametrize("seed", range(8))
def test_kv_quant_append_random_configs(seed):
    """Bit-exact codes and scales, appended at a random offset of a cache
    with room to spare; entries outside the appended range untouched."""
    rng = np.random.default_rng(9920 + seed)
    L, H = int(rng.integers(1, 3000)), int(rng.integers(1, 17))
    start = int(rng.integers(0, 500))
    cap = start + L + int(rng.integers(0, 40))
    k = synth.random_bf16(9930 + seed, (L, H, 128), float(rng.choice([1e-3, 1.0, 30.0])))
    v = synth.random_bf16(9940 + seed, (L, H, 128))
    say("kv_quant_append random-%d L %d H %d start %d cap %d" % (seed, L, H, start, cap))
    kc, vc, ks, vs = cache_tensors(H, cap)
    kc.fill_(55)
    vs.fill_(-2.0)
    assert nomas.kv_quant_append(dev16(k), dev16(v), kc, vc, ks, vs, start) == start + L
    torch.cuda.synchronize()
    for src, codes, scales in ((k, kc, ks), (v, vc, vs)):
        qo, so = oracle.quantise(oracle.bf16_bits_to_f64(src))
        assert np.array_equal(codes.cpu().numpy()[:, start:start + L].transpose(1, 0, 2), qo)
        assert np.array_equal(scales.cpu().numpy()[:, start:start + L].T.view(np.uint32), so.view(np.uint32))
    assert torch.all(kc[:, :start] == 55) and torch.all(kc[:, start + L:] == 55)
    assert torch.all(vs[:, :start] == -2.0) and torch.all(vs[:, start + L:] == -2.0)


@pytest.mark.parametrize("seed", range(8))
def test_cam_xattn_random_configs(seed):
    rng = np.random.default_rng(9950 + seed)
    Lq, H, Nc = int(rng.integers(1, 5000)), int(rng.integers(1, 5)), int(rng.integers(1, 129))
    q = synth.random_bf16(9960 + seed, (Lq, H, 128))
    wk = synth.random_bf16(9970 + seed, (64, H * 128), 1 / 8)
    wv = synth.random_bf16(9980 + seed, (64, H * 128), 1 / 8)
    cam = oracle.cam_tokens(synth.camera_path(seed, 7, 4 * Nc)).astype(np.float32)
    say("cam_xattn random-%d Lq %d H %d Nc %d" % (seed, Lq, H, Nc))
    out = nomas.cam_xattn(dev16(q), dev(cam), dev16(wk), dev16(wv), sm_scale=SM)
    torch.cuda.synchronize()
    assert_close(f64(out), oracle.cam_xattn(q, cam, wk, wv, SM), "cam_xattn random-%d" % seed)


@pytest.mark.parametrize("seed", range(8))
def test_gqa_attn_random_configs(seed):
    rng = np.random.default_rng(9990 + seed)
    Hkv = int(rng.integers(1, 5))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
    L = int(rng.integers(1, 2500))
    q = synth.random_bf16(10000 + seed, (L, Hq, 128))
    k = synth.random_bf16(10010 + seed, (L, Hkv, 128))
    v = synth.random_bf16(10020 + seed, (L, Hkv, 128))
    say("gqa_attn random-%d L %d Hq %d Hkv %d" % (seed, L, Hq, Hkv))
    lse = torch.empty((Hq, L), dtype=torch.float32, device="cuda:0")
    out = nomas.gqa_attn(dev16(q), dev16(k), dev16(v), sm_scale=SM, lse=lse)
    torch.cuda.synchronize()
    ref, lref = oracle.gqa_attn(q, k, v, SM)
    assert_close(f64(out), ref, "gqa random-%d" % seed)
    np.testing.assert_allclose(lse.cpu().numpy(), lref, rtol=0, atol=2.0 ** -8)
