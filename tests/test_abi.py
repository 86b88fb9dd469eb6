"""The C-ABI library without a GPU: it loads, exports every function that
include/nomas.h declares, rejects bad arguments on the host before touching
the device, and its host-side pieces (RoPE table, camera tokens) agree with
the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import segment_causal_attention_amd as nomas
import synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "nomas.h")
FAKE = 0x10000          # an aligned, never-dereferenced address for host-side checks


def declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(nomas_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = nomas.lib()
    names = declared()
    assert set(names) >= {"nomas_rope3d", "nomas_kv_quant_append", "nomas_seg_attn", "nomas_cam_xattn"}
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(nomas.SYMBOLS)
    assert "gfx950" in nomas.version()


def test_strerror_covers_codes():
    for c in (nomas.OK, nomas.EINVAL, nomas.ECAPACITY, nomas.EHIP, nomas.EUNSUPPORTED):
        assert nomas.strerror(c) and nomas.strerror(c) != "unknown error code"
    assert nomas.strerror(12345) == "unknown error code"


def segs(*t):
    return nomas.seg_array(t)


def test_shutdown_drops_host_state():
    """nomas_shutdown needs no GPU, always succeeds and may be repeated; the
    host-only entry points work after it."""
    L = nomas.lib()
    assert L.nomas_shutdown() == nomas.OK
    assert L.nomas_shutdown() == nomas.OK
    nomas.shutdown()
    c, s = nomas.rope_table(0, 4)
    assert c.shape == (4, 8) and abs(float(c[0, 0]) - 1.0) == 0.0


def test_seg_attn_host_checks():
    L = nomas.lib()
    sa, n = segs((16, 0, 2, 4, 6))
    P = ctypes.c_void_p
    need = L.nomas_seg_attn_workspace(sa, n, 0, 2, 1)
    assert need == 2 * 35840 + 256                     # 16 + 2*4*6 = 64 new keys: one tile per head, + key norms
    good = dict(q=FAKE, k=FAKE, v=FAKE, segs=sa, n=n, kc=None, vc=None, ks=None, vs=None, cap=0, clen=0,
                H=2, sm=0.088, out=FAKE, lse=None, split=1, ws=FAKE, wsb=need)

    def call(**kw):
        a = dict(good, **kw)
        return L.nomas_seg_attn(P(a["q"]), P(a["k"]), P(a["v"]), a["segs"], a["n"], P(a["kc"]), P(a["vc"]),
                                P(a["ks"]), P(a["vs"]), a["cap"], a["clen"], a["H"], a["sm"], P(a["out"]),
                                P(a["lse"]), a["split"], P(a["ws"]), a["wsb"], None)

    assert call(q=None) == nomas.EINVAL
    assert call(out=None) == nomas.EINVAL
    assert call(q=FAKE + 2) == nomas.EINVAL            # misaligned
    assert call(H=0) == nomas.EINVAL
    assert call(sm=0.0) == nomas.EINVAL
    assert call(sm=float("nan")) == nomas.EINVAL
    assert call(n=0) == nomas.EINVAL
    assert call(clen=5, cap=4) == nomas.EINVAL        # cache_len > cap
    assert call(clen=4, cap=4) == nomas.EINVAL        # cache pointers missing
    bad, nb = segs((16, 0, 2, 0, 6))                  # video frames with a zero-height grid
    assert call(segs=bad, n=nb) == nomas.EINVAL
    neg, nn = segs((-1, 0, 2, 4, 6))
    assert call(segs=neg, n=nn) == nomas.EINVAL
    far, nf = segs((0, 16380, 8, 4, 6))               # t beyond the RoPE table
    assert call(segs=far, n=nf) == nomas.EUNSUPPORTED
    many, nm = nomas.seg_array([(1, 0, 0, 0, 0)] * (nomas.MAX_SEGS + 1))
    assert call(segs=many, n=nm) == nomas.EUNSUPPORTED
    empty, ne = segs((0, 0, 0, 0, 0))                 # no tokens: nothing to do
    assert call(segs=empty, n=ne) == nomas.OK
    assert call(ws=None) == nomas.EINVAL               # workspace missing, too small or misaligned
    assert call(wsb=need - 1) == nomas.EINVAL
    assert call(ws=FAKE + 8) == nomas.EINVAL
    # workspace size: H * ceil((cache + new tokens) / 64) tiles of 35840 bytes, then one float per tile
    # (the tile's largest squared key norm) padded to 256 bytes
    assert L.nomas_seg_attn_workspace(sa, n, 1000, 3, 1) == 3 * ((1000 + 64 + 63) // 64) * 35840 + 256
    assert L.nomas_seg_attn_workspace(sa, n, 4000, 4, 1) == 4 * 64 * 35840 + 1024
    # split keys: fp32 partial outputs and log-sum-exps of every part on top
    assert L.nomas_seg_attn_workspace(sa, n, 1000, 3, 2) == 3 * 17 * 35840 + 256 + 2 * 64 * 3 * 129 * 4
    # 560 bytes per (token, head): the full-cache shape (253,440 cached + 63,360 new tokens, 16 heads)
    full, nf = segs((0, 288, 72, 22, 40))
    ws_full = L.nomas_seg_attn_workspace(full, nf, 253440, 16, 1)
    assert ws_full == 16 * 4950 * 35840 + (16 * 4950 * 4 + 255) // 256 * 256
    assert 35840 // 64 == 560 and abs(ws_full / (16 * 316800) - 560) < 0.1 and 2.83e9 < ws_full < 2.85e9
    assert L.nomas_seg_attn_workspace(sa, n, -1, 3, 1) == nomas.EINVAL
    assert L.nomas_seg_attn_workspace(sa, n, 0, 0, 1) == nomas.EINVAL
    assert L.nomas_seg_attn_workspace(sa, n, 0, 2, -1) == nomas.EINVAL
    assert L.nomas_seg_attn_workspace(sa, n, 0, 2, nomas.MAX_SPLIT + 1) == nomas.EUNSUPPORTED
    assert call(split=-1) == nomas.EINVAL
    assert call(split=nomas.MAX_SPLIT + 1) == nomas.EUNSUPPORTED


def test_kv_quant_append_host_checks():
    L = nomas.lib()
    P = ctypes.c_void_p
    ln = ctypes.c_int64(10)

    def call(L_=4, H=2, cap=16, k=FAKE, sc=FAKE, length=ln):
        return L.nomas_kv_quant_append(P(k), P(FAKE), L_, H, P(FAKE), P(FAKE), P(sc), P(FAKE), cap,
                                       ctypes.byref(length) if length is not None else None, None)

    assert call(L_=7) == nomas.ECAPACITY and ln.value == 10      # 10 + 7 > 16: nothing written
    assert call(L_=-1) == nomas.EINVAL
    assert call(H=0) == nomas.EINVAL
    assert call(k=None) == nomas.EINVAL
    assert call(k=FAKE + 8) == nomas.EINVAL
    assert call(sc=FAKE + 2) == nomas.EINVAL
    assert call(length=None) == nomas.EINVAL
    assert call(L_=0) == nomas.OK and ln.value == 10               # empty append is a no-op
    big = ctypes.c_int64(17)
    assert call(length=big) == nomas.EINVAL                         # len > cap


def test_rope3d_and_cam_xattn_host_checks():
    L = nomas.lib()
    P = ctypes.c_void_p
    sa, n = segs((16, 0, 2, 4, 6))
    assert L.nomas_rope3d(P(None), P(FAKE), sa, n, 2, None) == nomas.EINVAL
    assert L.nomas_rope3d(P(FAKE), P(FAKE), sa, n, 0, None) == nomas.EINVAL
    W = 1 << 30

    def cam(Lq=10, H=2, c=FAKE, Nc=5, ws=FAKE, wsb=W):
        return L.nomas_cam_xattn(P(FAKE), Lq, H, P(c), Nc, P(FAKE), P(FAKE), 0.1, P(FAKE), P(ws), wsb, None)

    assert cam(Nc=0) == nomas.EINVAL
    assert cam(Nc=nomas.MAX_CAM + 1) == nomas.EUNSUPPORTED
    assert cam(c=None) == nomas.EINVAL
    assert cam(Lq=0, ws=None, wsb=0) == nomas.OK                  # nothing to do, no workspace needed
    assert cam(ws=None) == nomas.EINVAL
    assert cam(ws=FAKE + 8) == nomas.EINVAL
    need = L.nomas_cam_xattn_workspace(2, 5)
    assert cam(wsb=need - 1) == nomas.EINVAL
    # per head: Kc rows (32 per started block of 32 camera tokens, 136 bf16 each), then the 128 Vc^T
    # rows of 32 bf16 per key block + 8
    for H, Nc in ((2, 5), (16, 72), (3, 128), (1, 33)):
        nkb = (Nc + 31) // 32
        assert L.nomas_cam_xattn_workspace(H, Nc) == H * (32 * nkb * 136 + 128 * (32 * nkb + 8)) * 2
    assert L.nomas_cam_xattn_workspace(0, 5) == nomas.EINVAL
    assert L.nomas_cam_xattn_workspace(2, 0) == nomas.EINVAL
    assert L.nomas_cam_xattn_workspace(2, nomas.MAX_CAM + 1) == nomas.EUNSUPPORTED


@pytest.mark.parametrize("axis,npos", [(0, 400), (1, 22), (2, 40), (1, 1024)])
def test_rope_table_bit_identical_to_oracle(axis, npos):
    c, s = nomas.rope_table(axis, npos)
    co, so = oracle.rope_table_f32(axis, npos)
    assert np.array_equal(c.view(np.uint32), co.view(np.uint32))
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32))


def test_cam_tokens_match_oracle():
    c2w = synth.camera_path(5, 0, 288)
    got = nomas.cam_tokens(c2w)
    ref = oracle.cam_tokens(c2w)
    assert got.shape == (72, 64)
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-6)
    # same float32 values as rounding the oracle's float64 tokens, but for rare last-bit cases
    assert np.mean(got == ref.astype(np.float32)) > 0.99
    got2 = nomas.cam_tokens(c2w, translation_scale=2.0, rotation_scale=1.0)
    np.testing.assert_allclose(got2, oracle.cam_tokens(c2w, 2.0, 1.0), rtol=0, atol=2e-6)
    with pytest.raises(nomas.NomasError):
        nomas.cam_tokens(c2w[:6])


def test_cam_tokens_near_pi():
    """The library's host normalisation keeps the axis of rotations just short
    of a half turn and uses the positive-largest-component axis at exactly pi,
    as the oracle does (comfyui-wiki news page, 相机控制作为一等输入:
    rotation scale 2.5); expected values are scipy matrix exponentials."""
    from test_oracle_cam import near_pi_cases
    for path, want, case in near_pi_cases():
        got = nomas.cam_tokens(path).reshape(4, 4, 4)
        np.testing.assert_allclose(got[1, :3, :3], want, rtol=0, atol=2e-6, err_msg=str(case))
        np.testing.assert_allclose(got, oracle.cam_tokens(path).reshape(4, 4, 4), rtol=0, atol=2e-6)


def test_seg_attn_sel_host_checks():
    """History selection: workspace sizes of shared and per-segment key
    regions, and the errors of an invalid selection (host only)."""
    L = nomas.lib()
    P = ctypes.c_void_p
    one, n1 = segs((16, 0, 2, 4, 6))                      # 64 new tokens
    two, n2 = segs((16, 0, 2, 4, 6), (0, 2, 1, 4, 5))     # 64 + 20 new tokens

    def ws(arr, n, clen, sel, H=3, split=1):
        if sel is None:
            return L.nomas_seg_attn_sel_workspace(arr, n, clen, None, None, H, split)
        off, rng = nomas.sel_arrays(sel, n)
        return L.nomas_seg_attn_sel_workspace(arr, n, clen, off.ctypes.data, rng.ctypes.data, H, split)

    tiles = lambda t, H=3: H * t * 35840 + (H * t * 4 + 255) // 256 * 256
    assert ws(one, n1, 1000, None) == L.nomas_seg_attn_workspace(one, n1, 1000, 3, 1) == tiles(17)
    # one segment: its 2 ranges (100 + 31 cache tokens) then the 64 new tokens
    assert ws(one, n1, 1000, [[(0, 100), (500, 531)]]) == tiles((131 + 64 + 63) // 64)
    # two segments with the same list share one region holding all 84 new tokens
    assert ws(two, n2, 1000, [[(10, 20)], [(10, 20)]]) == tiles((10 + 84 + 63) // 64)
    # different lists: a region each, new tokens up to the segment's end
    assert ws(two, n2, 1000, [[(10, 20)], [(0, 600)]]) == tiles((10 + 64 + 63) // 64 + (600 + 84 + 63) // 64)
    assert ws(two, n2, 1000, [[], [(0, 1000)]]) == tiles(1 + (1000 + 84 + 63) // 64)
    # invalid selections
    for bad in ([[(5, 5)]], [[(-1, 3)]], [[(0, 1001)]], [[(10, 20), (15, 30)]], [[(20, 30), (0, 10)]]):
        assert ws(one, n1, 1000, bad) == nomas.EINVAL, bad
    off = np.array([1, 1], np.int32)                      # must start at 0
    rng = np.array([0, 5], np.int64)
    assert L.nomas_seg_attn_sel_workspace(one, n1, 1000, off.ctypes.data, rng.ctypes.data, 3, 1) == nomas.EINVAL
    off = np.array([0, 2, 1], np.int32)                   # decreasing
    rng = np.array([0, 5, 6, 9], np.int64)
    assert L.nomas_seg_attn_sel_workspace(two, n2, 1000, off.ctypes.data, rng.ctypes.data, 3, 1) == nomas.EINVAL
    many = [[(2 * i, 2 * i + 1) for i in range(nomas.MAX_SEL_RANGES + 1)]]
    assert ws(one, n1, 1000, many) == nomas.EUNSUPPORTED
    assert ws(one, n1, 1000, [[(2 * i, 2 * i + 1) for i in range(nomas.MAX_SEL_RANGES)]]) > 0
    # the call itself refuses an invalid selection before touching anything
    off, rng = nomas.sel_arrays([[(10, 20), (15, 30)]], n1)
    rc = L.nomas_seg_attn_sel(P(FAKE), P(FAKE), P(FAKE), one, n1, P(FAKE), P(FAKE), P(FAKE), P(FAKE), 2000, 1000,
                              off.ctypes.data, rng.ctypes.data, 2, 0.088, P(FAKE), None, 1, P(FAKE), 1 << 40, None)
    assert rc == nomas.EINVAL


def test_gqa_attn_host_checks():
    L = nomas.lib()
    P = ctypes.c_void_p
    # tiles are per KV head: ceil(100 / 64) = 2 tiles x 2 KV heads, norms padded to 256 bytes
    assert L.nomas_gqa_attn_workspace(100, 4, 2) == 2 * 2 * 35840 + 256
    assert L.nomas_gqa_attn_workspace(100, 4, 3) == nomas.EINVAL      # not a multiple
    assert L.nomas_gqa_attn_workspace(100, 0, 1) == nomas.EINVAL
    assert L.nomas_gqa_attn_workspace(-1, 4, 2) == nomas.EINVAL
    assert L.nomas_gqa_attn_workspace(1 << 22, 32, 8) == nomas.EUNSUPPORTED   # L * Hq beyond the limit
    args = lambda **kw: [P(kw.get("q", FAKE)), P(FAKE), P(FAKE), kw.get("L", 100), kw.get("Hq", 4), kw.get("Hkv", 2),
                         kw.get("sm", 0.088), P(FAKE), None, P(kw.get("ws", FAKE)), kw.get("wsb", 1 << 30), None]
    assert L.nomas_gqa_attn(*args(q=None)) == nomas.EINVAL
    assert L.nomas_gqa_attn(*args(q=FAKE + 4)) == nomas.EINVAL
    assert L.nomas_gqa_attn(*args(Hkv=3)) == nomas.EINVAL
    assert L.nomas_gqa_attn(*args(sm=-1.0)) == nomas.EINVAL
    assert L.nomas_gqa_attn(*args(wsb=100)) == nomas.EINVAL
    assert L.nomas_gqa_attn(*args(L=0)) == nomas.OK


def test_w8a16_host_checks():
    L = nomas.lib()
    P = ctypes.c_void_p
    assert L.nomas_w8a16_linear_workspace(2048, 8192) == 8192 * 2048 * 2
    assert L.nomas_w8a16_linear_workspace(2000, 8192) == nomas.EUNSUPPORTED   # K not a multiple of 64
    assert L.nomas_w8a16_linear_workspace(2048, 1000) == nomas.EUNSUPPORTED   # N not a multiple of 256
    assert L.nomas_w8a16_linear_workspace(0, 256) == nomas.EINVAL
    good = dict(x=FAKE, M=100, K=128, w=FAKE, s=FAKE, N=256, y=FAKE, ws=FAKE, wsb=256 * 128 * 2)

    def call(**kw):
        a = dict(good, **kw)
        return L.nomas_w8a16_linear(P(a["x"]), a["M"], a["K"], P(a["w"]), P(a["s"]), a["N"], P(a["y"]), P(a["ws"]),
                                    a["wsb"], None)

    assert call(M=-1) == nomas.EINVAL
    assert call(x=None) == nomas.EINVAL
    assert call(w=None) == nomas.EINVAL
    assert call(x=FAKE + 2) == nomas.EINVAL
    assert call(s=FAKE + 2) == nomas.EINVAL
    assert call(wsb=256 * 128 * 2 - 1) == nomas.EINVAL
    assert call(K=96) == nomas.EUNSUPPORTED
    assert call(N=300) == nomas.EUNSUPPORTED
    assert call(M=1 << 20, K=2048) == nomas.EUNSUPPORTED     # x beyond 2 GiB


def test_w8a16_noalloc_host_checks():
    """The allocation-free W8A16 entry point: the same argument checks, and
    weights whose dequantised copy exceeds the static scratch (32 MiB) are
    refused before anything touches the device."""
    L = nomas.lib()
    P = ctypes.c_void_p

    def call(x=FAKE, M=100, K=128, w=FAKE, s=FAKE, N=256, y=FAKE):
        return L.nomas_w8a16_linear_noalloc(P(x), M, K, P(w), P(s), N, P(y), None)

    assert nomas.W8A16_NOALLOC_MAX_BYTES == 32 << 20
    assert call(K=2048, N=8192 + 256) == nomas.EUNSUPPORTED      # 2048 x 8448 x 2 > 32 MiB
    assert call(K=8192 + 64, N=2048) == nomas.EUNSUPPORTED
    assert call(K=4096, N=4352) == nomas.EUNSUPPORTED
    assert call(M=-1) == nomas.EINVAL
    assert call(x=None) == nomas.EINVAL
    assert call(y=None) == nomas.EINVAL
    assert call(w=None) == nomas.EINVAL
    assert call(s=None) == nomas.EINVAL
    assert call(x=FAKE + 2) == nomas.EINVAL
    assert call(s=FAKE + 2) == nomas.EINVAL
    assert call(K=96) == nomas.EUNSUPPORTED
    assert call(N=300) == nomas.EUNSUPPORTED


def test_seg_attn_bwd_host_checks():
    """Backward pass: workspace = H x (tiles) x 70,656 bytes, every segment
    starting a new 64-token tile; bad arguments are rejected on the host."""
    L = nomas.lib()
    P = ctypes.c_void_p
    sa, n = segs((16, 0, 2, 4, 6), (3, 2, 1, 2, 2), (0, 0, 0, 0, 0), (70, 0, 0, 1, 1))
    assert L.nomas_seg_attn_bwd_workspace(sa, n, 2) == 2 * (1 + 1 + 0 + 2) * 70656
    assert L.nomas_seg_attn_bwd_workspace(sa, n, 0) == nomas.EINVAL
    assert L.nomas_seg_attn_bwd_workspace(sa, 0, 2) == nomas.EINVAL
    assert L.nomas_seg_attn_bwd_workspace(sa, n, 300) == nomas.EUNSUPPORTED
    big, nb = segs((1 << 20, 0, 0, 1, 1))
    assert L.nomas_seg_attn_bwd_workspace(big, nb, 16) == nomas.EUNSUPPORTED   # L * H beyond the limit
    need = L.nomas_seg_attn_bwd_workspace(sa, n, 2)
    good = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, segs=sa, n=n, H=2, sm=0.088,
                dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE, wsb=need)

    def call(**kw):
        a = dict(good, **kw)
        return L.nomas_seg_attn_bwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["o"]), P(a["lse"]), P(a["do"]), a["segs"],
                                    a["n"], a["H"], a["sm"], P(a["dq"]), P(a["dk"]), P(a["dv"]), P(a["ws"]), a["wsb"],
                                    None)

    for name in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "ws"):
        assert call(**{name: None}) == nomas.EINVAL, name
    for name in ("q", "k", "v", "o", "do", "dq", "dk", "dv", "ws"):
        assert call(**{name: FAKE + 4}) == nomas.EINVAL, name
    assert call(lse=FAKE + 2) == nomas.EINVAL
    assert call(sm=0.0) == nomas.EINVAL and call(sm=float("nan")) == nomas.EINVAL
    assert call(H=0) == nomas.EINVAL
    assert call(wsb=need - 1) == nomas.EINVAL
    assert call(n=nomas.MAX_SEGS + 1) == nomas.EUNSUPPORTED
    empty, ne = segs((0, 0, 0, 0, 0))
    assert call(segs=empty, n=ne, ws=None, wsb=0) == nomas.OK      # no tokens: nothing to do


def test_binding_allocates_on_the_call_stream(monkeypatch):
    """Workspace and outputs the binding allocates for a call queued on a
    given stream come from that stream's pool (torch.cuda.stream context), so
    the caching allocator cannot reuse them behind kernels still running on
    it; with no stream given the current stream is used as is.  CPU-only:
    torch's stream context and allocator are replaced by recorders."""
    import contextlib
    import torch
    from segment_causal_attention_amd import _lib
    events = []

    class Ext:
        def __init__(self, handle):
            self.handle = handle

    @contextlib.contextmanager
    def stream_ctx(s):
        events.append(("enter", s))
        yield
        events.append(("exit", s))

    real_empty = torch.empty

    def empty(*a, **k):
        events.append(("alloc",))
        k.pop("device", None)
        return real_empty(*a, **k)

    monkeypatch.setattr(torch.cuda, "ExternalStream", Ext)
    monkeypatch.setattr(torch.cuda, "stream", stream_ctx)
    monkeypatch.setattr(torch, "empty", empty)
    with pytest.raises(ValueError):             # a host tensor is no device workspace
        _lib._workspace(100, "cpu", None, 0x1234)
    assert [e[0] for e in events] == ["enter", "alloc", "exit"]
    assert isinstance(events[0][1], Ext) and events[0][1].handle == 0x1234
    events.clear()
    obj = object()
    with pytest.raises(ValueError):
        _lib._workspace(100, "cpu", None, obj)
    assert [e[0] for e in events] == ["enter", "alloc", "exit"] and events[0][1] is obj
    events.clear()
    with pytest.raises(ValueError):
        _lib._workspace(100, "cpu", None, None)
    assert events == [("alloc",)]
