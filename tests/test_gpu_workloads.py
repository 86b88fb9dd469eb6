"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses.  Every output tensor is computed in full on the GPU; the
oracle recomputes a seeded sample of rows (and of heads where a head's whole
cache must be rebuilt on the CPU), which it can do row by row because rows
are independent.

  3 s turn     16,096 queries x 31,936 keys, every 16th row + the last 64, all heads
  4 s segment  21,376 x 37,216, outlier channels x20, layers 0 and 53
  full cache   63,360 x 316,800, cache built on the GPU (rope3d + quantise)
  five turns   cache grown turn by turn to 253,440 tokens, camera cross-attention
  decoder      one 10-latent-frame window: 35,200 tokens, 32 query / 8 KV heads
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import threadpoolctl
import torch

import oracle
import segment_causal_attention_amd as nomas
import synth
from gpu_util import SM, assert_close, bits, cache_tensors, dev, dev16, f64, say

pytestmark = pytest.mark.gpu


def sample_rows(Lq, stride, tail=64, extra=()):
    rows = set(range(0, Lq, stride)) | set(range(max(0, Lq - tail), Lq)) | set(extra)
    return np.array(sorted(r for r in rows if 0 <= r < Lq))


def run_attn(q, k, v, segs, cache, Lc, H):
    kc, vc, ks, vs = cache
    lse = torch.empty((H, q.shape[0]), dtype=torch.float32, device="cuda:0")
    out = nomas.seg_attn(q, k, v, segs, kc, vc, ks, vs, cache_len=Lc, sm_scale=SM, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def check_rows(name, out, lse, inp_q, inp_k, inp_v, segs, ocache, Lc, rows, heads=None, gpu_heads=None):
    """Oracle rows vs GPU rows; `heads` index the oracle's inputs, `gpu_heads`
    the GPU output (the same heads unless the oracle got a head subset)."""
    kc, vc, ks, vs = ocache
    gpu_heads = heads if gpu_heads is None else gpu_heads
    say("%s: oracle on %d rows x %s heads" % (name, len(rows), "all" if heads is None else len(heads)))
    ref, lref = oracle.seg_attn(inp_q, inp_k, inp_v, segs, kc, vc, ks, vs, Lc, SM, rows=rows, heads=heads)
    got = f64(out)[rows]
    gl = lse.cpu().numpy()[:, rows]
    if gpu_heads is not None:
        got = got[:, gpu_heads]
        gl = gl[gpu_heads]
    assert_close(got, ref, name)
    np.testing.assert_allclose(gl, lref, rtol=0, atol=2.0 ** -8)


@pytest.mark.parametrize("name,layer", [("turn3s", 0), ("seg4s", 0), ("seg4s", 53)],
                         ids=["turn3s", "seg4s-layer0", "seg4s-layer53"])
def test_attention_with_oracle_cache(name, layer):
    """3 s turn and 4 s segment (with outliers): the INT8 history comes from
    the oracle's quantiser, byte for byte."""
    inp = synth.layer_inputs(name, layer)
    cfg = inp["cfg"]
    if cfg.outliers:
        assert len(inp["outlier_cols"]) == 20
    say("config", cfg.name, "layer", layer, "Lq", cfg.Lq, "Lc", cfg.Lc)
    ocache = oracle.build_cache(inp["k_hist"], inp["v_hist"], cfg.hist_segs)
    gcache = tuple(dev(a) for a in ocache)
    out, lse = run_attn(dev16(inp["q"]), dev16(inp["k_new"]), dev16(inp["v_new"]), cfg.new_segs, gcache, cfg.Lc, cfg.H)
    rows = sample_rows(cfg.Lq, 16 if name == "turn3s" else 64, extra=range(250, 262))
    check_rows("%s layer %d" % (cfg.name, layer), out, lse, inp["q"], inp["k_new"], inp["v_new"], cfg.new_segs,
               ocache, cfg.Lc, rows)


def gpu_append(k_new_d, v_new_d, segs, cache, length):
    """The path's per-segment cache update: rotate the keys, quantise, append."""
    k_rot = nomas.rope3d(k_new_d, segs)
    n = nomas.kv_quant_append(k_rot, v_new_d, *cache, length)
    torch.cuda.synchronize()
    return k_rot, n


def oracle_head_rows(k_bits, v_bits, segs, h):
    """The oracle's rotated bf16 keys and INT8 rows of one head."""
    kr = oracle.bf16_round(oracle.rope3d(oracle.bf16_bits_to_f64(k_bits[:, h:h + 1]), segs))[:, 0]
    kq, kscale = oracle.quantise(kr)
    vq, vscale = oracle.quantise(oracle.bf16_bits_to_f64(v_bits[:, h]))
    return kr, kq, kscale, vq, vscale


def check_cache_rows(name, cache, start, k_rot_d, k_bits, v_bits, segs, heads):
    """GPU-rotated keys equal the oracle's bf16 bits; GPU codes and scales
    equal the oracle's quantisation bit for bit."""
    kc, vc, ks, vs = cache
    L = k_bits.shape[0]
    for h in heads:
        kr, kq, kscale, vq, vscale = oracle_head_rows(k_bits, v_bits, segs, h)
        got_rot = bits(k_rot_d[:, h].contiguous())
        mism = int(np.sum(got_rot != oracle.f64_to_bf16_bits(kr)))
        say("%s head %d: rotated-key mismatches %d of %d" % (name, h, mism, got_rot.size))
        assert mism == 0
        assert np.array_equal(kc[h, start:start + L].cpu().numpy(), kq)
        assert np.array_equal(vc[h, start:start + L].cpu().numpy(), vq)
        assert np.array_equal(ks[h, start:start + L].cpu().numpy().view(np.uint32), kscale.view(np.uint32))
        assert np.array_equal(vs[h, start:start + L].cpu().numpy().view(np.uint32), vscale.view(np.uint32))


def rows_per_tile(Lq, per_tile, seed, tile=256, extra=()):
    """`per_tile` seeded rows from every `tile`-row query tile (all rows of a
    shorter last tile), plus `extra`."""
    rng = np.random.default_rng(seed)
    rows = set(int(r) for r in extra if 0 <= r < Lq)
    for t0 in range(0, Lq, tile):
        n = min(tile, Lq - t0)
        rows.update(int(t0 + r) for r in rng.choice(n, size=min(per_tile, n), replace=False))
    return np.array(sorted(rows))


def split_plan_rows(segs, Lc, H, Lq, cus):
    """Query rows of the last head whose tiles the library splits into key-range
    parts at this shape (one segment, the last-round units of the grid), and
    the part count, read back from the workspace sizes: the split adds
    parts x 516 bytes per (query, head) of the split tiles."""
    ntq = (Lq + 255) // 256
    units = ntq * H
    r = units % cus
    extra = nomas.seg_attn_workspace(segs, Lc, H, 0) - nomas.seg_attn_workspace(segs, Lc, H, 1)
    f0 = (units - r) // ntq * Lq + (units - r) % ntq * 256
    pairs = Lq * H - f0
    assert r > 0 and extra % (516 * pairs) == 0, (r, extra, pairs)
    return extra // (516 * pairs), f0


def test_full_cache_workload():
    """12 s segment over 288 cached latent frames (~317K keys), cache built on
    the GPU exactly as the benchmark builds it.  All 16 heads are compared on
    a seeded subset of 16 rows from every 256-row query tile (4,000 rows),
    which includes every query tile whose keys the launch plan splits into
    parts merged by the log-sum-exp identity."""
    inp = synth.layer_inputs("fullcache")
    cfg = inp["cfg"]
    H, Lq, Lc = cfg.H, cfg.Lq, cfg.Lc
    say("config", cfg.name, "Lq", Lq, "Lc", Lc)
    # the launch plan at this shape: with 256 CUs, 3,968 query-tile units leave
    # 128 for a last round; those (head 15, query tiles 120..247) run in 2 key parts
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    parts, f0 = split_plan_rows(cfg.new_segs, Lc, H, Lq, cus)
    say("launch plan: %d CUs, last-round tiles in %d key parts from (head, row) %d" % (cus, parts, f0))
    if cus == 256:
        assert parts == 2 and f0 == 15 * Lq + 120 * 256
    cache = cache_tensors(H, Lc + Lq)
    k_rot, n = gpu_append(dev16(inp["k_hist"]), dev16(inp["v_hist"]), cfg.hist_segs, cache, 0)
    assert n == Lc
    check_cache_rows("full-cache history", cache, 0, k_rot, inp["k_hist"], inp["v_hist"], cfg.hist_segs, [0, 9, 15])
    del k_rot
    out, lse = run_attn(dev16(inp["q"]), dev16(inp["k_new"]), dev16(inp["v_new"]), cfg.new_segs, cache, Lc, H)
    # the oracle's own cache for every head, bit-identical to the GPU's
    say("full cache: oracle quantises the history of all %d heads" % H)
    ocache = oracle.build_cache(inp["k_hist"], inp["v_hist"], cfg.hist_segs)
    for g, o, what in zip(cache, ocache, ("k codes", "v codes", "k scales", "v scales")):
        got = g[:, :Lc].cpu().numpy()
        assert np.array_equal(got.view(np.uint8 if got.itemsize == 1 else np.uint32),
                              o.view(np.uint8 if o.itemsize == 1 else np.uint32)), what
    rows = rows_per_tile(Lq, 16, 20261025, extra=list(range(880, 890)) + list(range(Lq - 16, Lq)))
    split_rows = rows[rows >= f0 - (H - 1) * Lq] if parts > 1 else rows[:0]
    say("full cache: %d rows x %d heads (%d rows in head %d's split tiles)" % (len(rows), H, len(split_rows), H - 1))
    assert parts == 1 or len(split_rows) >= 16 * ((Lq - (f0 - (H - 1) * Lq)) // 256)
    got = f64(out[torch.from_numpy(rows).to(out.device)])
    gl = lse.cpu().numpy()[:, rows]
    one = lambda h: oracle.seg_attn(inp["q"][:, h:h + 1], inp["k_new"][:, h:h + 1], inp["v_new"][:, h:h + 1],
                                    cfg.new_segs, *(a[h:h + 1] for a in ocache), Lc, SM, rows=rows)
    # heads are independent and numpy's exp is single-threaded: 4 heads at a
    # time, each with a quarter of the host's BLAS threads (more would oversubscribe)
    blas = max(1, int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 4) // 4)
    with threadpoolctl.threadpool_limits(blas, user_api="blas"), ThreadPoolExecutor(4) as ex:
        for h, (ref, lref) in enumerate(ex.map(one, range(H))):
            assert_close(got[:, h], ref[:, 0], "full cache head %d (%d rows)" % (h, len(rows)))
            np.testing.assert_allclose(gl[h], lref[0], rtol=0, atol=2.0 ** -8)
    heads = [0, 9]
    sub = lambda a: np.ascontiguousarray(a[:, heads])
    ocache = tuple(np.ascontiguousarray(a[heads]) for a in ocache)
    # history selection at this shape: 18 of the 288 cached latent frames (the
    # last of every 16), as the benchmark's selection workload runs it
    (hseg,) = cfg.hist_segs
    frame = hseg.Hg * hseg.Wg
    sel = [[(f * frame, (f + 1) * frame) for f in range(15, hseg.T, 16)]]
    lse2 = torch.empty((H, Lq), dtype=torch.float32, device="cuda:0")
    out2 = nomas.seg_attn(dev16(inp["q"]), dev16(inp["k_new"]), dev16(inp["v_new"]), cfg.new_segs, *cache,
                          cache_len=Lc, sm_scale=SM, lse=lse2, sel=sel)
    torch.cuda.synchronize()
    say("full cache, 18 selected frames")
    kc, vc, ks, vs = ocache
    ref, lref = oracle.seg_attn(sub(inp["q"]), sub(inp["k_new"]), sub(inp["v_new"]), cfg.new_segs, kc, vc, ks, vs,
                                Lc, SM, rows=rows, sel=sel)
    assert_close(f64(out2)[rows][:, heads], ref, "full cache, 18 selected frames")
    np.testing.assert_allclose(lse2.cpu().numpy()[heads][:, rows], lref, rtol=0, atol=2.0 ** -8)


def test_five_turns_growing_cache():
    """Five 12 s turns: each turn attends over the cache of all earlier turns,
    runs camera cross-attention, then rotates and appends its keys/values.
    Quantisation is checked every turn, attention and camera on turns 0 and 4
    (heads 3, 12 and 15, with a row in each of head 15's split query tiles)."""
    cfg = synth.WORKLOADS["fiveturns"]
    H = cfg.H
    cap = 5 * synth.turn_seg(0).ntok
    cache = cache_tensors(H, cap)
    heads = [3, 12, 15]     # head 15 holds the query tiles the launch plan splits into key parts
    length = 0
    okc = {h: [] for h in heads}
    for k in range(5):
        check = k in (0, 4)
        inp = synth.turn_inputs(k, with_cam=check)
        seg = inp["seg"]
        say("turn", k, "cache", length)
        kd, vd = dev16(inp["k_new"]), dev16(inp["v_new"])
        if check:
            out, lse = run_attn(dev16(inp["q"]), kd, vd, [seg], cache, length, H)
            # oracle cache of earlier turns for the sampled heads, from its own quantiser
            kcs = np.zeros((H, max(1, length), 128), np.int8)
            vcs = np.zeros_like(kcs)
            kss = np.zeros((H, max(1, length)), np.float32)
            vss = np.zeros_like(kss)
            for h in heads:
                if length:
                    kcs[h, :length] = np.concatenate([r[0] for r in okc[h]])
                    vcs[h, :length] = np.concatenate([r[2] for r in okc[h]])
                    kss[h, :length] = np.concatenate([r[1] for r in okc[h]])
                    vss[h, :length] = np.concatenate([r[3] for r in okc[h]])
            # one seeded row in each query tile from 120 on (head 15's split tiles at 256 CUs)
            split_tiles = rows_per_tile(seg.ntok, 1, 20261030 + k)
            rows = sample_rows(seg.ntok, 2048, tail=16, extra=split_tiles[split_tiles >= 120 * 256])
            check_rows("turn %d" % k, out, lse, inp["q"], inp["k_new"], inp["v_new"], [seg],
                       (kcs, vcs, kss, vss), length, rows, heads=heads)
            # camera cross-attention of the turn's video queries
            cam = nomas.cam_tokens(inp["c2w"])
            cam_o = oracle.cam_tokens(inp["c2w"]).astype(np.float32)
            np.testing.assert_allclose(cam, cam_o, rtol=0, atol=2e-6)
            oc = nomas.cam_xattn(dev16(inp["q_cam"]), dev(cam_o), dev16(inp["w_k"]), dev16(inp["w_v"]), sm_scale=SM)
            torch.cuda.synchronize()
            crow = sample_rows(seg.ntok, 997, tail=8)
            cref = oracle.cam_xattn(inp["q_cam"], cam_o, inp["w_k"], inp["w_v"], SM, rows=crow)
            assert_close(f64(oc)[crow], cref, "turn %d camera" % k)
        k_rot, n = gpu_append(kd, vd, [seg], cache, length)
        check_cache_rows("turn %d append" % k, cache, length, k_rot, inp["k_new"], inp["v_new"], [seg], heads)
        for h in heads:
            _, kq, kscale, vq, vscale = oracle_head_rows(inp["k_new"], inp["v_new"], [seg], h)
            okc[h].append((kq, kscale, vq, vscale))
        length = n
        del k_rot, kd, vd
    assert length == cap


def test_workspace_beyond_4gib():
    """One head over an 8M-token INT8 cache (8,388,608 cached + 64 new
    tokens): the tile images take 4.7 GB of workspace, so image addresses pass
    2^32 bytes, and the call's single query tile runs as key-range parts.
    All 64 rows against the oracle."""
    Lc, H = 1 << 23, 1
    segs = [(16, 5, 1, 4, 12)]                      # 64 new tokens: 16 text + 4 x 12 video
    say("workspace beyond 4 GiB: cache", Lc, "heads", H)
    kc, ks = synth.random_int8_cache(401, H, Lc)
    vc, vs = synth.random_int8_cache(402, H, Lc)
    q = synth.random_bf16(403, (64, H, 128))
    k = synth.random_bf16(404, (64, H, 128))
    v = synth.random_bf16(405, (64, H, 128))
    need = nomas.seg_attn_workspace(segs, Lc, H)
    say("workspace bytes", need)
    assert need > (1 << 32)
    lse = torch.empty((H, 64), dtype=torch.float32, device="cuda:0")
    out = nomas.seg_attn(dev16(q), dev16(k), dev16(v), segs, dev(kc), dev(vc), dev(ks), dev(vs), cache_len=Lc,
                         sm_scale=SM, lse=lse)
    torch.cuda.synchronize()
    say("oracle over", Lc + 64, "keys")
    ref, lref = oracle.seg_attn(q, k, v, segs, kc, vc, ks, vs, Lc, SM)
    assert_close(f64(out), ref, "8M-token cache, 4.7 GB workspace")
    np.testing.assert_allclose(lse.cpu().numpy(), lref, rtol=0, atol=2.0 ** -8)


def test_decoder_window():
    """One decoder window at 1280x704: 10 latent frames of 4x16x16 tubelets
    (10 x 44 x 80 = 35,200 tokens), 32 query heads over 8 KV heads."""
    L, Hq, Hkv = 10 * 44 * 80, 32, 8
    q = synth.random_bf16(501, (L, Hq, 128))
    k = synth.random_bf16(502, (L, Hkv, 128))
    v = synth.random_bf16(503, (L, Hkv, 128))
    say("decoder window", L, Hq, Hkv)
    lse = torch.empty((Hq, L), dtype=torch.float32, device="cuda:0")
    out = nomas.gqa_attn(dev16(q), dev16(k), dev16(v), sm_scale=SM, lse=lse)
    torch.cuda.synchronize()
    rows = sample_rows(L, 512, tail=16)
    heads = [0, 3, 4, 13, 31]
    ref, lref = oracle.gqa_attn(q, k, v, SM, rows=rows, heads=heads)
    assert_close(f64(out)[rows][:, heads], ref, "decoder window")
    np.testing.assert_allclose(lse.cpu().numpy()[heads][:, rows], lref, rtol=0, atol=2.0 ** -8)
