"""Seeded random sweeps of GPU parity against the oracle.

Besides the hand-picked edge cases of the other GPU tests, each entry point
runs on configurations drawn from a fixed generator: segment mixes with
empty, text-only and ragged video segments, cache lengths from none to a few
hundred tokens, forced key-range parts, history selections, 1 to 3 heads,
and linear-layer shapes around the GEMM's tile sizes.  The bars are those of
the hand-picked cases (the helpers are shared with them)."""
import math

import numpy as np
import pytest
import torch

import oracle
import segment_causal_attention_amd as nomas
import synth
from gpu_util import assert_bf16_output, dev, dev16, f64, say
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
