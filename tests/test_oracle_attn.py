"""Pins for the oracle's segment-causal attention (comfyui-wiki news page,
一个世界，分段生成: each segment attends to the K/V cache of every earlier
segment, causal between segments; huaweicloud blog, section 2.1: text and
video K/V of each segment are cached and passed on)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import synth

SM = float(np.float32(1 / math.sqrt(128)))


def tiny_case(mode):
    """Inputs of the Tiny workload in one of its three modes."""
    inp = synth.tiny_inputs()
    segs = [s.astuple() for s in inp["segs"]]
    q, k, v = inp["q"], inp["k"], inp["v"]
    n = 64
    if mode == "cache":
        kc, vc, ks, vs = oracle.build_cache(k[:n], v[:n], segs[:1])
        return dict(q=q[n:2 * n], k=k[n:2 * n], v=v[n:2 * n], segs=segs[1:2], kc=kc, vc=vc, ks=ks, vs=vs, Lc=n)
    if mode == "packed":
        z8 = np.zeros((2, 0, 128), np.int8)
        z = np.zeros((2, 0), np.float32)
        return dict(q=q[:2 * n], k=k[:2 * n], v=v[:2 * n], segs=segs[:2], kc=z8, vc=z8, ks=z, vs=z, Lc=0)
    if mode == "three":
        kc, vc, ks, vs = oracle.build_cache(k[:n], v[:n], segs[:1])
        return dict(q=q[n:], k=k[n:], v=v[n:], segs=segs[1:], kc=kc, vc=vc, ks=ks, vs=vs, Lc=n)
    raise ValueError(mode)


def run(c, **kw):
    return oracle.seg_attn(c["q"], c["k"], c["v"], c["segs"], c["kc"], c["vc"], c["ks"], c["vs"], c["Lc"], SM, **kw)


@pytest.mark.parametrize("mode", ["cache", "packed", "three"])
def test_matches_brute_force(mode):
    c = tiny_case(mode)
    out, lse = run(c)
    f = lambda b: oracle.bf16_bits_to_f64(b).tolist()
    H = 2
    cache_k = [[(c["kc"][h, j].astype(int).tolist(), float(c["ks"][h, j])) for j in range(c["Lc"])] for h in range(H)]
    cache_v = [[(c["vc"][h, j].astype(int).tolist(), float(c["vs"][h, j])) for j in range(c["Lc"])] for h in range(H)]
    ob, lb, pb = brute.seg_attn(f(c["q"]), f(c["k"]), f(c["v"]), c["segs"], cache_k, cache_v, SM)
    np.testing.assert_allclose(out, np.array(ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), rtol=0, atol=1e-12)
    # the brute force's probabilities sum to one on every row
    for h in range(H):
        for row in pb[h]:
            assert abs(math.fsum(row) - 1.0) <= 1e-12


def test_rows_are_normalised():
    """Values equal for every key come back unchanged (sum of p is 1)."""
    c = tiny_case("three")
    c["v"] = np.full_like(c["v"], oracle.f64_to_bf16_bits(np.array([0.375]))[0])
    c["vc"] = np.full_like(c["vc"], 3)
    c["vs"] = np.full_like(c["vs"], np.float32(0.125))
    out, _ = run(c)
    np.testing.assert_allclose(out, 0.375, rtol=0, atol=1e-14)


@pytest.mark.parametrize("poison", ["finite", "nan"])
def test_earlier_segments_ignore_later_segments(poison):
    """Outputs of segment-0 rows are bit-identical when segment-1 keys and
    values change (packed mode), and stay finite when they hold NaN."""
    c = tiny_case("packed")
    out0, lse0 = run(c)
    rng = np.random.default_rng(10)
    c2 = dict(c)
    k2, v2 = c["k"].copy(), c["v"].copy()
    if poison == "finite":
        k2[64:] = oracle.f64_to_bf16_bits(oracle.bf16_round(rng.standard_normal(k2[64:].shape) * 30))
        v2[64:] = oracle.f64_to_bf16_bits(oracle.bf16_round(rng.standard_normal(v2[64:].shape) * 30))
    else:
        k2[64:] = 0x7FC0
        v2[64:] = 0x7FC0
    c2["k"], c2["v"] = k2, v2
    out1, lse1 = run(c2)
    assert np.array_equal(out0[:64], out1[:64]) and np.array_equal(lse0[:, :64], lse1[:, :64])
    assert np.all(np.isfinite(out1[:64]))
    if poison == "finite":
        assert not np.allclose(out0[64:], out1[64:])


def _text_only(rng, L, H):
    x = oracle.bf16_round(rng.standard_normal((L, H, 128)))
    return oracle.f64_to_bf16_bits(x)


def test_single_segment_is_textbook_sdpa():
    """Text-only segment (no rotation), no cache: softmax(QK^T s)V, checked
    against torch's scaled_dot_product_attention in float64 on the CPU."""
    rng = np.random.default_rng(11)
    L, H = 50, 3
    q, k, v = (_text_only(rng, L, H) for _ in range(3))
    z8, z = np.zeros((H, 0, 128), np.int8), np.zeros((H, 0), np.float32)
    out, _ = oracle.seg_attn(q, k, v, [(L, 0, 0, 1, 1)], z8, z8, z, z, 0, SM)
    t = lambda b: torch.from_numpy(oracle.bf16_bits_to_f64(b)).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=SM)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-13)


def test_packed_segments_are_block_causal_sdpa():
    rng = np.random.default_rng(12)
    lens, H = [7, 20, 13], 2
    L = sum(lens)
    q, k, v = (_text_only(rng, L, H) for _ in range(3))
    z8, z = np.zeros((H, 0, 128), np.int8), np.zeros((H, 0), np.float32)
    out, _ = oracle.seg_attn(q, k, v, [(n, 0, 0, 1, 1) for n in lens], z8, z8, z, z, 0, SM)
    seg = np.repeat(np.arange(3), lens)
    mask = torch.from_numpy(seg[None, :] <= seg[:, None])
    t = lambda b: torch.from_numpy(oracle.bf16_bits_to_f64(b)).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask, scale=SM)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-13)


def test_equal_keys_average_the_allowed_values():
    rng = np.random.default_rng(13)
    lens, H = [9, 15], 2
    L = sum(lens)
    q, v = _text_only(rng, L, H), _text_only(rng, L, H)
    k = np.broadcast_to(_text_only(rng, 1, H), (L, H, 128)).copy()
    Lc = 11
    kc = np.broadcast_to(np.arange(-64, 64, dtype=np.int8), (H, Lc, 128)).copy()
    ks = np.zeros((H, Lc), np.float32)      # zero scale: cached keys are 0 vectors
    vc = rng.integers(-127, 128, (H, Lc, 128)).astype(np.int8)
    vs = (rng.random((H, Lc)) * 0.02).astype(np.float32)
    # all new keys equal AND orthogonal... use a zero query so every score is 0
    q0 = np.zeros_like(q)
    out, lse = oracle.seg_attn(q0, k, v, [(n, 0, 0, 1, 1) for n in lens], kc, vc, ks, vs, Lc, SM)
    Vc = oracle.dequant_bf16(vc, vs)
    vf = oracle.bf16_bits_to_f64(v)
    for h in range(H):
        m0 = np.concatenate([Vc[h], vf[:9, h]]).mean(0)
        m1 = np.concatenate([Vc[h], vf[:, h]]).mean(0)
        np.testing.assert_allclose(out[:9, h], np.broadcast_to(m0, (9, 128)), atol=1e-14)
        np.testing.assert_allclose(out[9:, h], np.broadcast_to(m1, (15, 128)), atol=1e-14)
        np.testing.assert_allclose(lse[h, :9], math.log(Lc + 9), atol=1e-14)
        np.testing.assert_allclose(lse[h, 9:], math.log(Lc + 24), atol=1e-14)


def test_lse_merge_of_cache_and_new_parts():
    """Attention over cache + own segment equals the LSE-weighted merge of
    attention over the cache alone and over the segment alone."""
    c = tiny_case("cache")
    out, lse = run(c)
    H = 2
    z8, z = np.zeros((H, 0, 128), np.int8), np.zeros((H, 0), np.float32)
    out_n, lse_n = oracle.seg_attn(c["q"], c["k"], c["v"], c["segs"], z8, z8, z, z, 0, SM)
    qr = oracle.bf16_round(oracle.rope3d(oracle.bf16_bits_to_f64(c["q"]), c["segs"]))
    for h in range(H):
        Kc = oracle.dequant_bf16(c["kc"][h], c["ks"][h])
        Vc = oracle.dequant_bf16(c["vc"][h], c["vs"][h])
        o_c, l_c = oracle.attend(qr[:, h], Kc, Vc, SM)
        m = np.maximum(l_c, lse_n[h])
        wc, wn = np.exp(l_c - m), np.exp(lse_n[h] - m)
        merged = (wc[:, None] * o_c + wn[:, None] * out_n[:, h]) / (wc + wn)[:, None]
        np.testing.assert_allclose(out[:, h], merged, atol=1e-13)
        np.testing.assert_allclose(lse[h], m + np.log(wc + wn), atol=1e-13)


def test_cache_stands_in_for_the_earlier_segment():
    """Cache mode (segment 0 held as INT8) is close to packed mode's segment-1
    rows (segment 0 held exactly), and far from ignoring segment 0."""
    cc, cp = tiny_case("cache"), tiny_case("packed")
    out_c, _ = run(cc)
    out_p, _ = run(cp)
    H = 2
    z8, z = np.zeros((H, 0, 128), np.int8), np.zeros((H, 0), np.float32)
    out_n, _ = oracle.seg_attn(cc["q"], cc["k"], cc["v"], cc["segs"], z8, z8, z, z, 0, SM)
    d_cache = np.abs(out_c - out_p[64:]).max()
    d_none = np.abs(out_n - out_p[64:]).max()
    assert d_cache < 0.05 and d_none > 5 * d_cache


def test_rows_and_heads_subsets_agree_with_full_run():
    c = tiny_case("three")
    out, lse = run(c)
    rows = np.array([0, 5, 63, 64, 100, 127])
    o2, l2 = run(c, rows=rows, heads=[1])
    np.testing.assert_array_equal(o2[:, 0], out[rows, 1])
    np.testing.assert_array_equal(l2[0], lse[1, rows])


# ----------------------------------------------------------------------------
# history selection (huaweicloud blog, section 2.2 and the section 3.5 table;
# comfyui-wiki, 单张 4090 配置: a segment attends to a chosen subset of the
# earlier frames)

SEL_THREE = [[(0, 10), (30, 64)], [(5, 20)]]      # "three" mode: new segments 1 and 2


def test_selection_matches_brute_force():
    """Different selections per segment (three-segment mode) against the
    pure-Python brute force that gathers the selected cache rows itself."""
    c = tiny_case("three")
    out, lse = run(c, sel=SEL_THREE)
    f = lambda b: oracle.bf16_bits_to_f64(b).tolist()
    H = 2
    cache_k = [[(c["kc"][h, j].astype(int).tolist(), float(c["ks"][h, j])) for j in range(c["Lc"])] for h in range(H)]
    cache_v = [[(c["vc"][h, j].astype(int).tolist(), float(c["vs"][h, j])) for j in range(c["Lc"])] for h in range(H)]
    ob, lb, pb = brute.seg_attn(f(c["q"]), f(c["k"]), f(c["v"]), c["segs"], cache_k, cache_v, SM, sel=SEL_THREE)
    np.testing.assert_allclose(out, np.array(ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), rtol=0, atol=1e-12)
    # segment 1 rows see 10 + 34 cache keys and 64 new ones; segment 2 rows 15 + 128
    assert len(pb[0][0]) == 44 + 64 and len(pb[0][64]) == 15 + 128


def test_whole_cache_selection_is_no_selection():
    c = tiny_case("three")
    out0, lse0 = run(c)
    out1, lse1 = run(c, sel=[[(0, 64)], [(0, 30), (30, 64)]])
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_window_selection_is_the_sliced_cache():
    """A contiguous window of the cache gives exactly the result of a cache
    holding only that window."""
    c = tiny_case("cache")
    out1, lse1 = run(c, sel=[[(20, 52)]])
    c2 = dict(c, kc=np.ascontiguousarray(c["kc"][:, 20:52]), vc=np.ascontiguousarray(c["vc"][:, 20:52]),
              ks=np.ascontiguousarray(c["ks"][:, 20:52]), vs=np.ascontiguousarray(c["vs"][:, 20:52]), Lc=32)
    out2, lse2 = run(c2)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_empty_selection_is_no_cache():
    c = tiny_case("cache")
    out1, lse1 = run(c, sel=[[]])
    out2, lse2 = run(dict(c, Lc=0))
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_unselected_cache_rows_do_not_matter():
    """Changing every cache row outside the selection leaves outputs and lse
    bit-identical."""
    c = tiny_case("three")
    out0, lse0 = run(c, sel=SEL_THREE)
    keep = np.zeros(64, bool)
    for rng_list in SEL_THREE:
        for lo, hi in rng_list:
            keep[lo:hi] = True
    rng = np.random.default_rng(3)
    c2 = dict(c)
    for name in ("kc", "vc"):
        a = c[name].copy()
        a[:, ~keep] = rng.integers(-127, 128, size=a[:, ~keep].shape, dtype=np.int8)
        c2[name] = a
    for name in ("ks", "vs"):
        a = c[name].copy()
        a[:, ~keep] = np.float32(5.0)
        c2[name] = a
    out1, lse1 = run(c2, sel=SEL_THREE)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


# ----------------------------------------------------------------------------
# decoder window attention with grouped KV heads (comfyui-wiki, 模型内部)


def _gqa_inputs(L, Hq, Hkv, seed=21):
    q = synth.random_bf16(seed, (L, Hq, 128))
    k = synth.random_bf16(seed + 1, (L, Hkv, 128))
    v = synth.random_bf16(seed + 2, (L, Hkv, 128))
    return q, k, v


def test_gqa_matches_brute_force():
    q, k, v = _gqa_inputs(12, 4, 2)
    out, lse = oracle.gqa_attn(q, k, v, SM)
    f = lambda b: oracle.bf16_bits_to_f64(b).tolist()
    qf, kf, vf = f(q), f(k), f(v)
    for h in range(4):
        for i in range(12):
            o, l, p = brute.softmax_attend(qf[i][h], [kf[j][h // 2] for j in range(12)],
                                           [vf[j][h // 2] for j in range(12)], SM)
            np.testing.assert_allclose(out[i, h], o, rtol=0, atol=1e-12)
            assert abs(lse[h, i] - l) <= 1e-12


def test_gqa_is_sdpa_with_repeated_kv_heads():
    """Grouped heads equal torch's scaled_dot_product_attention (float64, CPU)
    with each KV head repeated for its query heads."""
    q, k, v = _gqa_inputs(50, 8, 2, seed=33)
    out, _ = oracle.gqa_attn(q, k, v, SM)
    t = lambda b, rep: torch.from_numpy(oracle.bf16_bits_to_f64(b)).repeat_interleave(rep, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q, 1), t(k, 4), t(v, 4), scale=SM).permute(1, 0, 2)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)


def test_gqa_with_equal_heads_is_segment_attention_of_one_text_segment():
    """Hq = Hkv: one all-text segment (no rotation) with no cache gives the
    same numbers through seg_attn."""
    q, k, v = _gqa_inputs(40, 2, 2, seed=44)
    out, lse = oracle.gqa_attn(q, k, v, SM)
    z8 = np.zeros((2, 0, 128), np.int8)
    z = np.zeros((2, 0), np.float32)
    o2, l2 = oracle.seg_attn(q, k, v, [(40, 0, 0, 0, 0)], z8, z8, z, z, 0, SM)
    np.testing.assert_allclose(out, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-13)
