"""GPU parity of each libnomas entry point against the CPU oracle, on small and
edge-case shapes (ragged tails, several query tiles, packed segments, short
caches).  Calls go through the C ABI (ctypes binding)."""
import math

import numpy as np
import pytest
import torch

import oracle
import segment_causal_attention_amd as nomas
import synth
from gpu_util import SM, assert_bf16_output, assert_close, bits, cache_tensors, dev, dev16, f64, say

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------
# rope3d: float64 rotation rounded once, so it should equal the oracle's bits


ROPE_CASES = [
    ("tiny", [s.astuple() for s in synth.TINY_SEGS], 2),
    ("text+video", [(256, 18, 2, 22, 40)], 16),
    ("late-t", [(3, 16000, 2, 7, 5), (0, 9, 1, 30, 33)], 3),
]


@pytest.mark.parametrize("name,segs,H", ROPE_CASES, ids=[c[0] for c in ROPE_CASES])
def test_rope3d_matches_oracle(name, segs, H):
    L = sum(s[0] + s[2] * s[3] * s[4] for s in segs)
    x = synth.random_bf16(101, (L, H, 128), 3.0)
    say("rope3d", name, L, H)
    xd = dev16(x)
    y = nomas.rope3d(xd, segs)
    torch.cuda.synchronize()
    ref = oracle.f64_to_bf16_bits(oracle.bf16_round(oracle.rope3d(oracle.bf16_bits_to_f64(x), segs)))
    got = bits(y)
    diff = got != ref
    say("  mismatching bf16 values: %d of %d" % (diff.sum(), diff.size))
    if diff.any():   # at most one unit in the last place
        assert np.abs(got[diff].astype(np.int32) - ref[diff].astype(np.int32)).max() <= 1
    assert diff.mean() < 1e-5
    # in place gives the same bits
    nomas.rope3d(xd, segs, out=xd)
    torch.cuda.synchronize()
    assert np.array_equal(bits(xd), got)


# ----------------------------------------------------------------------------
# kv_quant_append: bit-exact codes and scales


def _quant_inputs():
    rng_rows = []
    a = synth.random_bf16(7, (300, 3, 128), 1.0)
    b = synth.random_bf16(8, (300, 3, 128), 1.0)
    # outlier channels x20, tiny magnitudes, an all-zero row and exact ties
    b32 = oracle.bf16_bits_to_f64(b)
    b32[:, :, 5] *= 20.0
    b32[10:20] *= 1e-4
    b32[20] = 0.0
    b32[21, 0, :] = 0.0
    b32[21, 0, 0] = 127.0
    b32[21, 0, 1:9] = [2.5, 3.5, 0.5, 1.5, -2.5, -3.5, -0.5, 126.5]
    b = oracle.f64_to_bf16_bits(oracle.bf16_round(b32))
    return a, b


def test_kv_quant_append_bit_exact_and_offsets():
    k, v = _quant_inputs()
    L, H = k.shape[0], k.shape[1]
    cap = 2 * L + 37
    kc, vc, ks, vs = cache_tensors(H, cap)
    kc.fill_(77)
    ks.fill_(-1.0)
    n = nomas.kv_quant_append(dev16(k[:123]), dev16(v[:123]), kc, vc, ks, vs, 0)
    assert n == 123
    n = nomas.kv_quant_append(dev16(k), dev16(v), kc, vc, ks, vs, n)
    assert n == 123 + L
    torch.cuda.synchronize()
    for src, codes, scales, start in ((k[:123], kc, ks, 0), (k, kc, ks, 123), (v[:123], vc, vs, 0), (v, vc, vs, 123)):
        qo, so = oracle.quantise(oracle.bf16_bits_to_f64(src))          # [L][H][128], [L][H]
        qg = codes.cpu().numpy()[:, start:start + len(src)].transpose(1, 0, 2)
        sg = scales.cpu().numpy()[:, start:start + len(src)].T
        assert np.array_equal(qg, qo)
        assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    # entries past the appended range are untouched
    assert torch.all(kc[:, 123 + L:] == 77) and torch.all(ks[:, 123 + L:] == -1.0)
    # a full cache refuses and leaves everything as it was
    with pytest.raises(nomas.NomasError) as ei:
        nomas.kv_quant_append(dev16(k), dev16(v), kc, vc, ks, vs, n)
    assert ei.value.code == nomas.ECAPACITY


# ----------------------------------------------------------------------------
# seg_attn


def _run_gpu(q, k, v, segs, cache, Lc, H, with_lse=True, n_split=0, sel=None):
    Ln = q.shape[0]
    lse = torch.empty((H, Ln), dtype=torch.float32, device="cuda:0") if with_lse else None
    if Lc > 0:
        kc, vc, ks, vs = (dev(a) for a in cache)
    else:
        kc = vc = ks = vs = None
    out = nomas.seg_attn(dev16(q), dev16(k), dev16(v), segs, kc, vc, ks, vs, cache_len=Lc, sm_scale=SM, lse=lse,
                         n_split=n_split, sel=sel)
    torch.cuda.synchronize()
    return f64(out), (lse.cpu().numpy() if with_lse else None), out


def _check_case(name, q, k, v, segs, cache, Lc, H, n_split=0, sel=None):
    say("seg_attn", name, "Ln", q.shape[0], "Lc", Lc, "H", H, "n_split", n_split, "sel", sel)
    got, lse, _ = _run_gpu(q, k, v, segs, cache, Lc, H, n_split=n_split, sel=sel)
    kc, vc, ks, vs = cache if Lc > 0 else (np.zeros((H, 0, 128), np.int8),) * 2 + (np.zeros((H, 0), np.float32),) * 2
    ref, lref = oracle.seg_attn(q, k, v, segs, kc, vc, ks, vs, Lc, SM, sel=sel)
    assert_close(got, ref, name)
    # the row sum is taken over the bf16-rounded probabilities that also feed
    # P.V (relative error <= 2^-9 per term), so |lse error| <= ~2^-9 + fp32 terms
    np.testing.assert_allclose(lse, lref, rtol=0, atol=2.0 ** -8)


@pytest.mark.parametrize("mode", ["cache", "packed", "three"])
def test_seg_attn_tiny(mode):
    inp = synth.tiny_inputs()
    segs = [s.astuple() for s in inp["segs"]]
    q, k, v = inp["q"], inp["k"], inp["v"]
    n = 64
    if mode == "packed":
        _check_case("tiny-packed", q[:2 * n], k[:2 * n], v[:2 * n], segs[:2], None, 0, 2)
        return
    cache = oracle.build_cache(k[:n], v[:n], segs[:1])
    hi = 2 * n if mode == "cache" else 3 * n
    _check_case("tiny-" + mode, q[n:hi], k[n:hi], v[n:hi], segs[1:hi // n], cache, n, 2)


EDGE = [
    ("one-token", [(1, 0, 0, 0, 0)], 0, 2),
    ("one-token-cache1", [(1, 0, 0, 0, 0)], 1, 2),
    ("text-only-300", [(300, 0, 0, 0, 0)], 5, 1),
    ("ragged-97-cache130", [(7, 3, 2, 5, 9)], 130, 2),
    ("packed-5", [(3, 0, 1, 2, 3), (0, 1, 2, 3, 5), (10, 3, 1, 1, 1), (1, 4, 3, 2, 2), (0, 7, 1, 8, 8)], 77, 2),
    ("two-seg-multi-tile", [(5, 0, 1, 3, 4), (40, 1, 3, 10, 9)], 0, 3),
    ("turn-shape-small", [(256, 18, 2, 22, 40)], 1760, 2),
    ("empty-segment-between", [(4, 0, 1, 2, 2), (0, 0, 0, 0, 0), (2, 1, 2, 3, 3)], 64, 2),
    ("max-segments", [(i % 4, i, 1, 2, 2 + i % 3) for i in range(64)], 50, 2),   # the 64-segment limit
]


def _edge_inputs(segs, Lc, H):
    Ln = sum(s[0] + s[2] * s[3] * s[4] for s in segs)
    q = synth.random_bf16(201, (Ln, H, 128))
    k = synth.random_bf16(202, (Ln, H, 128))
    v = synth.random_bf16(203, (Ln, H, 128))
    cache = None
    if Lc > 0:
        hist = [(0, 0, 1, 1, Lc)]                 # a one-row "frame" of Lc history tokens
        kh = synth.random_bf16(204, (Lc, H, 128))
        vh = synth.random_bf16(205, (Lc, H, 128))
        cache = oracle.build_cache(kh, vh, hist, cap=Lc + 11)
    return q, k, v, cache


SPLIT = [("one-token", 4), ("ragged-97-cache130", 2), ("ragged-97-cache130", 3), ("packed-5", 4),
         ("turn-shape-small", 2), ("turn-shape-small", 4), ("empty-segment-between", 3)]


@pytest.mark.parametrize("name,n_split", SPLIT, ids=["%s-split%d" % c for c in SPLIT])
def test_seg_attn_split_keys(name, n_split):
    """Keys split into parts (some empty when a tile range is short) and
    merged by the log-sum-exp identity: same bar against the oracle, and
    the unsplit result to rounding."""
    (segs, Lc, H), = [(c[1], c[2], c[3]) for c in EDGE if c[0] == name]
    q, k, v, cache = _edge_inputs(segs, Lc, H)
    _check_case(name, q, k, v, segs, cache, Lc, H, n_split=n_split)
    one, lse1, _ = _run_gpu(q, k, v, segs, cache, Lc, H, n_split=1)
    many, lsen, _ = _run_gpu(q, k, v, segs, cache, Lc, H, n_split=n_split)
    # each part rounds its probabilities to bf16 against its own running max,
    # so sums differ at the 2^-9 level, as against the oracle
    np.testing.assert_allclose(many, one, rtol=0, atol=2.0 ** -7)
    np.testing.assert_allclose(lsen, lse1, rtol=0, atol=2.0 ** -8)


def test_seg_attn_last_round_split():
    """One segment whose query tiles leave the last round of workgroups
    nearly empty on a 256-CU device: 17 tiles x 16 heads = 272 units, 16 in
    the last round.  The library then splits only those 16 (head 15, tiles
    1..16) into key-range parts; the workspace holds the partial buffers.
    Rows of whole and split tiles against the oracle, with the library's
    plan and with one part forced."""
    segs, Lc, H = [(4352, 0, 0, 0, 0)], 8192, 16
    q, k, v, cache = _edge_inputs(segs, Lc, H)
    plain = nomas.seg_attn_workspace(segs, Lc, H, n_split=1)
    auto = nomas.seg_attn_workspace(segs, Lc, H, n_split=0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say("last-round split: CUs", cus, "workspace", plain, "->", auto)
    if cus == 256:
        assert auto > plain
    rows = np.array([0, 1, 255, 256, 257, 2047, 2048, 4095, 4096, 4350, 4351])
    ref, lref = oracle.seg_attn(q, k, v, segs, *cache, Lc, SM, rows=rows)
    for n_split in (0, 1):
        got, lse, _ = _run_gpu(q, k, v, segs, cache, Lc, H, n_split=n_split)
        assert_close(got[rows], ref, "last-round split n_split=%d" % n_split)
        np.testing.assert_allclose(lse[:, rows], lref, rtol=0, atol=2.0 ** -8)


@pytest.mark.parametrize("name,segs,Lc,H", EDGE, ids=[c[0] for c in EDGE])
def test_seg_attn_edge_shapes(name, segs, Lc, H):
    Ln = sum(s[0] + s[2] * s[3] * s[4] for s in segs)
    q = synth.random_bf16(201, (Ln, H, 128))
    k = synth.random_bf16(202, (Ln, H, 128))
    v = synth.random_bf16(203, (Ln, H, 128))
    cache = None
    if Lc > 0:
        hist = [(0, 0, 1, 1, Lc)]                 # a one-row "frame" of Lc history tokens
        kh = synth.random_bf16(204, (Lc, H, 128))
        vh = synth.random_bf16(205, (Lc, H, 128))
        cache = oracle.build_cache(kh, vh, hist, cap=Lc + 11)
    _check_case(name, q, k, v, segs, cache, Lc, H)


def test_seg_attn_future_segments_never_leak():
    """Rows of earlier packed segments give bit-identical outputs when every
    later-segment key and value is NaN, and stay finite."""
    inp = synth.tiny_inputs()
    segs = [s.astuple() for s in inp["segs"]]
    q, k, v = (inp[x].copy() for x in ("q", "k", "v"))
    got0, lse0, _ = _run_gpu(q, k, v, segs, None, 0, 2)
    k[64:] = 0x7FC0
    v[64:] = 0x7FC0
    got1, lse1, _ = _run_gpu(q, k, v, segs, None, 0, 2)
    assert np.all(np.isfinite(got1[:64])) and np.all(np.isfinite(lse1[:, :64]))
    assert np.array_equal(got0[:64], got1[:64]) and np.array_equal(lse0[:, :64], lse1[:, :64])
    assert np.all(np.isnan(got1[128:]))


@pytest.mark.parametrize("poison", ["x100", "nan"])
def test_seg_attn_future_segments_never_leak_unaligned(poison):
    """Packed segments whose boundaries fall inside 64-key tiles, over a
    77-token cache: the last key tile a row may read also holds keys of later
    segments.  Scaling those keys and values by 100 (or making them NaN)
    leaves every earlier row's output and lse bit-identical."""
    (segs, Lc, H), = [(c[1], c[2], c[3]) for c in EDGE if c[0] == "packed-5"]
    q, k, v, cache = _edge_inputs(segs, Lc, H)
    ends = np.cumsum([s[0] + s[2] * s[3] * s[4] for s in segs])
    got0, lse0, _ = _run_gpu(q, k, v, segs, cache, Lc, H)
    for cut in (1, 2, 4):
        n = int(ends[cut - 1])              # rows and keys of segments [0, cut)
        k1, v1 = k.copy(), v.copy()
        if poison == "nan":
            k1[n:] = 0x7FC0
            v1[n:] = 0x7FC0
        else:
            k1[n:] = oracle.f64_to_bf16_bits(oracle.bf16_round(oracle.bf16_bits_to_f64(k[n:]) * 100.0))
            v1[n:] = oracle.f64_to_bf16_bits(oracle.bf16_round(oracle.bf16_bits_to_f64(v[n:]) * 100.0))
        say("seg_attn leak", poison, "cut", cut, "rows", n)
        got1, lse1, _ = _run_gpu(q, k1, v1, segs, cache, Lc, H)
        assert np.array_equal(got0[:n], got1[:n]) and np.array_equal(lse0[:, :n], lse1[:, :n])


def _shift_gaps(q, k, segs, cache, Lc):
    """Per head and 32-row group of a one-segment input: c |q| max|k| over the
    allowed keys minus the largest score of the first 64 keys, the quantity
    whose size (against 64) decides between a fixed softmax shift and the
    running maximum (float64, from the oracle's rotations and dequantised
    cache)."""
    c = SM / math.log(2.0)
    qr = oracle.rope3d(oracle.bf16_bits_to_f64(q), segs)
    kr = oracle.bf16_round(oracle.rope3d(oracle.bf16_bits_to_f64(k), segs))
    kc, vc, ks, vs = cache
    K = np.concatenate([oracle.dequant_bf16(kc[:, :Lc], ks[:, :Lc]).transpose(1, 0, 2), kr], axis=0)
    gaps = []
    for h in range(q.shape[1]):
        kmax = np.sqrt((K[:, h] ** 2).sum(-1).max())
        for g0 in range(0, q.shape[0], 32):
            qg = qr[g0:g0 + 32, h]
            bound = c * np.sqrt((qg ** 2).sum(-1)) * kmax
            m0 = c * (qg @ K[:64, h].T).max(-1)
            gaps.append((bound - m0).max())
    return np.array(gaps)


@pytest.mark.parametrize("n_split", [1, 2])
def test_seg_attn_fixed_and_running_shift(n_split):
    """Row groups whose Cauchy-Schwarz bound is close to their first tile's
    largest score take a fixed softmax shift; groups of queries scaled x40
    (scores of a few hundred, base 2) are far from it and keep the running
    maximum with its rescaling.  The inputs hold both kinds; all rows meet
    the parity bar against the oracle."""
    segs, Lc, H = [(512, 0, 0, 0, 0)], 300, 2
    q, k, v, cache = _edge_inputs(segs, Lc, H)
    qf = oracle.bf16_bits_to_f64(q)
    for g0 in range(32, 512, 64):           # every other 32-row group
        qf[g0:g0 + 32] *= 40.0
    q = oracle.f64_to_bf16_bits(oracle.bf16_round(qf))
    gaps = _shift_gaps(q, k, segs, cache, Lc)
    say("shift gaps: min %.1f max %.1f" % (gaps.min(), gaps.max()))
    assert (gaps < 48).sum() >= 8 and (gaps > 96).sum() >= 8
    _check_case("fixed-and-running-shift", q, k, v, segs, cache, Lc, H, n_split=n_split)


# ----------------------------------------------------------------------------
# history selection (nomas_seg_attn_sel): each segment sees chosen cache tokens

SEL = [
    ("one-seg-3-ranges", [(7, 3, 2, 5, 9)], 300, 2, [[(0, 37), (100, 163), (250, 300)]], 0),
    ("one-seg-3-ranges-split3", [(7, 3, 2, 5, 9)], 300, 2, [[(0, 37), (100, 163), (250, 300)]], 3),
    ("packed-5-own-lists", [(3, 0, 1, 2, 3), (0, 1, 2, 3, 5), (10, 3, 1, 1, 1), (1, 4, 3, 2, 2), (0, 7, 1, 8, 8)], 77, 2,
     [[(0, 10)], [], [(5, 77)], [(0, 77)], [(30, 31), (40, 77)]], 0),
    ("two-seg-shared-list", [(5, 0, 1, 3, 4), (40, 1, 3, 10, 9)], 130, 3, [[(3, 90)], [(3, 90)]], 0),
    ("empty-selection", [(7, 3, 2, 5, 9)], 130, 2, [[]], 0),
    # the limits: 64 ranges in one list, and 64 segments (each with a list of its own: 64 key regions)
    ("max-ranges", [(7, 3, 2, 5, 9)], 2000, 2, [[(30 * i, 30 * i + 11) for i in range(64)]], 0),
    ("max-segments-own-lists", [(1 + i % 3, i, 1, 2, 3) for i in range(64)], 700, 2,
     [[(10 * i, 10 * i + 7 + i % 5)] for i in range(64)], 0),
]


@pytest.mark.parametrize("name,segs,Lc,H,sel,n_split", SEL, ids=[c[0] for c in SEL])
def test_seg_attn_selection_matches_oracle(name, segs, Lc, H, sel, n_split):
    q, k, v, cache = _edge_inputs(segs, Lc, H)
    _check_case(name, q, k, v, segs, cache, Lc, H, n_split=n_split, sel=sel)


def test_seg_attn_selection_of_the_whole_cache_is_bit_identical():
    """Selecting every cache token (in one range or two) packs the same keys
    as no selection: outputs and lse agree bit for bit."""
    segs, Lc, H = [(7, 3, 2, 5, 9)], 300, 2
    q, k, v, cache = _edge_inputs(segs, Lc, H)
    got0, lse0, _ = _run_gpu(q, k, v, segs, cache, Lc, H)
    for sel in ([[(0, Lc)]], [[(0, 64), (64, Lc)]]):
        got1, lse1, _ = _run_gpu(q, k, v, segs, cache, Lc, H, sel=sel)
        assert np.array_equal(got0, got1) and np.array_equal(lse0, lse1), sel


def test_seg_attn_selection_ignores_unselected_rows():
    """Rewriting every unselected cache row (codes and scales) leaves outputs
    and lse bit-identical."""
    (segs, Lc, H, sel, _), = [c[1:] for c in SEL if c[0] == "packed-5-own-lists"]
    q, k, v, cache = _edge_inputs(segs, Lc, H)
    got0, lse0, _ = _run_gpu(q, k, v, segs, cache, Lc, H, sel=sel)
    keep = np.zeros(Lc, bool)
    for ranges in sel:
        for lo, hi in ranges:
            keep[lo:hi] = True
    say("unselected cache rows:", int((~keep).sum()))
    kc, vc, ks, vs = (a.copy() for a in cache)
    rng = np.random.default_rng(7)
    for a in (kc, vc):
        a[:, :Lc][:, ~keep] = rng.integers(-127, 128, size=a[:, :Lc][:, ~keep].shape, dtype=np.int8)
    for a in (ks, vs):
        a[:, :Lc][:, ~keep] = np.float32(7.5)
    got1, lse1, _ = _run_gpu(q, k, v, segs, (kc, vc, ks, vs), Lc, H, sel=sel)
    assert np.array_equal(got0, got1) and np.array_equal(lse0, lse1)


def test_seg_attn_deterministic_and_cache_copy():
    inp = synth.tiny_inputs()
    segs = [s.astuple() for s in inp["segs"]]
    n = 64
    cache = oracle.build_cache(inp["k"][:n], inp["v"][:n], segs[:1])
    args = (inp["q"][n:], inp["k"][n:], inp["v"][n:], segs[1:], cache, n, 2)
    _, _, o1 = _run_gpu(*args)
    _, _, o2 = _run_gpu(*args)
    assert torch.equal(o1, o2)
    # a resumed cache (codes, scales and length copied elsewhere) gives the same bits
    kc, vc, ks, vs = (dev(a) for a in cache)
    kc2, vc2, ks2, vs2 = (t.clone() for t in (kc, vc, ks, vs))
    o3 = nomas.seg_attn(dev16(args[0]), dev16(args[1]), dev16(args[2]), segs[1:], kc2, vc2, ks2, vs2,
                        cache_len=n, sm_scale=SM)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3)


def test_seg_attn_on_a_side_stream_without_workspace():
    """A call queued on a stream other than the current one, with the
    workspace and output allocated by the binding, gives the same bits as on
    the current stream; the next allocations on the current stream run while
    the side stream may still be busy."""
    segs, Lc, H = [(256, 18, 2, 22, 40)], 1760, 2
    q, k, v, cache = _edge_inputs(segs, Lc, H)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    kc, vc, ks, vs = (dev(a) for a in cache)
    ref = nomas.seg_attn(qd, kd, vd, segs, kc, vc, ks, vs, cache_len=Lc, sm_scale=SM)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for i in range(3):
        outs.append(nomas.seg_attn(qd, kd, vd, segs, kc, vc, ks, vs, cache_len=Lc, sm_scale=SM, stream=side))
        junk = torch.empty(nomas.seg_attn_workspace(segs, Lc, H), dtype=torch.uint8, device="cuda:0")
        junk.fill_(0xFF)                      # would corrupt a workspace reused across streams
        del junk
    raw = nomas.seg_attn(qd, kd, vd, segs, kc, vc, ks, vs, cache_len=Lc, sm_scale=SM, stream=side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for o in outs + [raw]:
        assert torch.equal(o, ref)


def test_calls_after_shutdown_are_bit_identical():
    """After nomas_shutdown the next call uploads the RoPE tables again and
    looks up the static scratch again; results are bit-identical."""
    segs, Lc, H = [(16, 3, 2, 5, 7)], 90, 2
    q, k, v, cache = _edge_inputs(segs, Lc, H)
    a, la, _ = _run_gpu(q, k, v, segs, cache, Lc, H)
    r1 = nomas.rope3d(dev16(k), segs)
    x = dev16(synth.random_bf16(31, (100, 512)))
    codes = dev(np.random.default_rng(32).integers(-127, 128, size=(256, 512), dtype=np.int8))
    scale = dev(np.full(256, 0.01, np.float32))
    y1 = nomas.w8a16_linear_noalloc(x, codes, scale, torch.empty((100, 256), dtype=torch.int16, device="cuda:0"))
    torch.cuda.synchronize()
    nomas.shutdown()
    b, lb, _ = _run_gpu(q, k, v, segs, cache, Lc, H)
    r2 = nomas.rope3d(dev16(k), segs)
    y2 = nomas.w8a16_linear_noalloc(x, codes, scale, torch.empty((100, 256), dtype=torch.int16, device="cuda:0"))
    torch.cuda.synchronize()
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    assert torch.equal(r1, r2) and torch.equal(y1, y2)


# ----------------------------------------------------------------------------
# decoder window attention with grouped KV heads (nomas_gqa_attn)

GQA = [(100, 4, 2), (700, 8, 2), (3000, 32, 8), (257, 2, 1), (64, 3, 3), (1, 4, 4)]


@pytest.mark.parametrize("L,Hq,Hkv", GQA, ids=["L%d-%dq-%dkv" % c for c in GQA])
def test_gqa_attn_matches_oracle(L, Hq, Hkv):
    say("gqa_attn", L, Hq, Hkv)
    q = synth.random_bf16(401, (L, Hq, 128))
    k = synth.random_bf16(402, (L, Hkv, 128))
    v = synth.random_bf16(403, (L, Hkv, 128))
    lse = torch.empty((Hq, L), dtype=torch.float32, device="cuda:0")
    out = nomas.gqa_attn(dev16(q), dev16(k), dev16(v), sm_scale=SM, lse=lse)
    torch.cuda.synchronize()
    ref, lref = oracle.gqa_attn(q, k, v, SM)
    assert_close(f64(out), ref, "gqa L=%d Hq=%d Hkv=%d" % (L, Hq, Hkv))
    np.testing.assert_allclose(lse.cpu().numpy(), lref, rtol=0, atol=2.0 ** -8)


# ----------------------------------------------------------------------------
# INT8-weight linear layer (nomas_w8a16_linear)


def _w8_inputs(M, K, N, seed):
    """x ~ N(0, 1) bf16; codes uniform in [-127, 127]; scales around
    1 / (73 sqrt K) so that outputs are O(1) (the codes' std is ~73)."""
    x = synth.random_bf16(seed, (M, K))
    g = np.random.default_rng(seed)
    codes = g.integers(-127, 128, size=(N, K), dtype=np.int8)
    s = (1.0 / (73.0 * math.sqrt(K)) * (0.5 + g.random(N))).astype(np.float32)
    return x, codes, s


W8 = [(300, 128, 256), (1000, 2048, 512), (513, 2048, 6144), (64, 8192, 2048), (1, 64, 256), (0, 128, 256)]


@pytest.mark.parametrize("M,K,N", W8, ids=["M%d-K%d-N%d" % c for c in W8])
def test_w8a16_linear_matches_oracle(M, K, N):
    say("w8a16", M, K, N)
    x, codes, s = _w8_inputs(M, K, N, 701 + M)
    y = nomas.w8a16_linear(dev16(x) if M else torch.empty((0, K), dtype=torch.int16, device="cuda:0"),
                           dev(codes), dev(s))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (M, N)
    if M == 0:
        return
    ref = oracle.w8a16_linear(x, codes, s)
    assert_bf16_output(f64(y), ref, "w8a16 M=%d K=%d N=%d" % (M, K, N))


@pytest.mark.parametrize("K,N", [(2048, 8192), (2048, 2048)], ids=["ffn-up", "out-proj"])
def test_w8a16_linear_model_shape_sampled(K, N):
    """Linear layers of one 12 s segment, 63,360 tokens: the FFN up projection
    (2048 -> 8192, big tiles throughout) and the output projection (2048 ->
    2048: its last round of big tiles would be 40 of 256 tiles, so rows from
    61,440 on take the small tiles).  Sampled rows on both sides of that
    boundary and the ragged last tile against the oracle."""
    M = 63360
    x, codes, s = _w8_inputs(M, K, N, 777 + N)
    y = nomas.w8a16_linear(dev16(x), dev(codes), dev(s))
    torch.cuda.synchronize()
    rows = np.array(sorted(set(range(0, M, 997)) | set(range(61430, 61450)) | set(range(M - 40, M))))
    ref = oracle.w8a16_linear(x, codes, s, rows=rows)
    assert_bf16_output(f64(y)[rows], ref, "w8a16 model shape K=%d N=%d" % (K, N))


# ----------------------------------------------------------------------------
# cam_xattn


@pytest.mark.parametrize("Lq,H,Nc", [(100, 2, 1), (3000, 2, 72), (64, 3, 5), (2100, 1, 32), (700, 2, 33), (257, 2, 128)])
def test_cam_xattn_matches_oracle(Lq, H, Nc):
    say("cam_xattn", Lq, H, Nc)
    q = synth.random_bf16(301, (Lq, H, 128))
    wk = synth.random_bf16(302, (64, H * 128), 1 / 8)
    wv = synth.random_bf16(303, (64, H * 128), 1 / 8)
    c2w = synth.camera_path(5, 7, 4 * Nc)
    cam = oracle.cam_tokens(c2w).astype(np.float32)
    out = nomas.cam_xattn(dev16(q), dev(cam), dev16(wk), dev16(wv), sm_scale=SM)
    torch.cuda.synchronize()
    got = f64(out)
    ref = oracle.cam_xattn(q, cam, wk, wv, SM)
    assert_close(got, ref, "cam_xattn Lq=%d H=%d Nc=%d" % (Lq, H, Nc))
    if Nc == 1:   # one camera token: every query returns its value vector
        _, Vc = oracle.cam_kv(cam, wk, wv, H)
        np.testing.assert_allclose(got, np.broadcast_to(Vc[0][None], got.shape), rtol=0, atol=1e-2)


def test_cam_xattn_workspace_serves_consecutive_calls():
    """One workspace sized for 128 camera tokens serves calls with 128, then
    5, then 72 tokens: each call rebuilds the images it reads, so nothing of
    an earlier call's larger image leaks into a later one."""
    H, Lq = 2, 600
    q = synth.random_bf16(311, (Lq, H, 128))
    wk = synth.random_bf16(312, (64, H * 128), 1 / 8)
    wv = synth.random_bf16(313, (64, H * 128), 1 / 8)
    ws = torch.empty(nomas.cam_xattn_workspace(H, 128), dtype=torch.uint8, device="cuda:0")
    qd, wkd, wvd = dev16(q), dev16(wk), dev16(wv)
    for Nc in (128, 5, 72):
        cam = oracle.cam_tokens(synth.camera_path(5, 8 + Nc, 4 * Nc)).astype(np.float32)
        say("cam_xattn workspace reuse Nc", Nc)
        out = nomas.cam_xattn(qd, dev(cam), wkd, wvd, sm_scale=SM, workspace=ws)
        torch.cuda.synchronize()
        assert_close(f64(out), oracle.cam_xattn(q, cam, wk, wv, SM), "cam_xattn reused workspace Nc=%d" % Nc)
