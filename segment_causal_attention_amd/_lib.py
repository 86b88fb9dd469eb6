"""ctypes binding of libnomas (C ABI in include/nomas.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libnomas.so.  Device tensors are torch tensors (bf16 tensors may be
torch.bfloat16 or int16 holding the raw bits); torch supplies the memory and
the current stream.  There is no fallback: if the library is missing, every
call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnomas.so")

OK, EINVAL, ECAPACITY, EHIP, EUNSUPPORTED = 0, -1, -2, -3, -4
HEAD_DIM = 128
MAX_SEGS = 64
MAX_CAM = 128
MAX_SPLIT = 4
MAX_SEL_RANGES = 64
SM_SCALE = 1.0 / math.sqrt(HEAD_DIM)

SYMBOLS = ("nomas_rope3d", "nomas_kv_quant_append", "nomas_seg_attn", "nomas_seg_attn_workspace",
           "nomas_seg_attn_sel", "nomas_seg_attn_sel_workspace", "nomas_gqa_attn", "nomas_gqa_attn_workspace",
           "nomas_seg_attn_bwd", "nomas_seg_attn_bwd_workspace",
           "nomas_w8a16_linear", "nomas_w8a16_linear_workspace", "nomas_w8a16_linear_noalloc",
           "nomas_cam_tokens", "nomas_cam_xattn", "nomas_cam_xattn_workspace", "nomas_rope_table", "nomas_strerror",
           "nomas_version", "nomas_shutdown")


class NomasError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (where, strerror(code), code))


class Seg(ctypes.Structure):
    _fields_ = [("n_text", ctypes.c_int32), ("t0", ctypes.c_int32), ("T", ctypes.c_int32),
                ("Hg", ctypes.c_int32), ("Wg", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_D = ctypes.c_double


def lib() -> ctypes.CDLL:
    """Load libnomas.so (built in-tree by segment_causal_attention_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libnomas.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.nomas_rope3d.argtypes = [_P, _P, ctypes.POINTER(Seg), _I, _I, _P]
        L.nomas_kv_quant_append.argtypes = [_P, _P, _I64, _I, _P, _P, _P, _P, _I64, ctypes.POINTER(_I64), _P]
        L.nomas_seg_attn.argtypes = [_P, _P, _P, ctypes.POINTER(Seg), _I, _P, _P, _P, _P, _I64, _I64, _I, _F,
                                     _P, _P, _I, _P, _I64, _P]
        L.nomas_seg_attn_workspace.argtypes = [ctypes.POINTER(Seg), _I, _I64, _I, _I]
        L.nomas_seg_attn_workspace.restype = _I64
        L.nomas_seg_attn_sel.argtypes = [_P, _P, _P, ctypes.POINTER(Seg), _I, _P, _P, _P, _P, _I64, _I64, _P, _P, _I,
                                         _F, _P, _P, _I, _P, _I64, _P]
        L.nomas_seg_attn_sel_workspace.argtypes = [ctypes.POINTER(Seg), _I, _I64, _P, _P, _I, _I]
        L.nomas_seg_attn_sel_workspace.restype = _I64
        L.nomas_gqa_attn.argtypes = [_P, _P, _P, _I64, _I, _I, _F, _P, _P, _P, _I64, _P]
        L.nomas_gqa_attn_workspace.argtypes = [_I64, _I, _I]
        L.nomas_gqa_attn_workspace.restype = _I64
        L.nomas_seg_attn_bwd.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.POINTER(Seg), _I, _I, _F, _P, _P, _P, _P,
                                         _I64, _P]
        L.nomas_seg_attn_bwd_workspace.argtypes = [ctypes.POINTER(Seg), _I, _I]
        L.nomas_seg_attn_bwd_workspace.restype = _I64
        L.nomas_w8a16_linear.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P, _P, _I64, _P]
        L.nomas_w8a16_linear_workspace.argtypes = [_I64, _I64]
        L.nomas_w8a16_linear_workspace.restype = _I64
        L.nomas_w8a16_linear_noalloc.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P, _P]
        L.nomas_cam_tokens.argtypes = [_P, _I, _D, _D, _P]
        L.nomas_cam_xattn.argtypes = [_P, _I64, _I, _P, _I, _P, _P, _F, _P, _P, _I64, _P]
        L.nomas_cam_xattn_workspace.argtypes = [_I, _I]
        L.nomas_cam_xattn_workspace.restype = _I64
        L.nomas_rope_table.argtypes = [_I, _I, _P, _P]
        L.nomas_strerror.argtypes = [_I]
        L.nomas_strerror.restype = ctypes.c_char_p
        L.nomas_shutdown.argtypes = []
        L.nomas_shutdown.restype = _I
        L.nomas_version.argtypes = []
        L.nomas_version.restype = ctypes.c_char_p
        for name in ("nomas_rope3d", "nomas_kv_quant_append", "nomas_seg_attn", "nomas_seg_attn_sel", "nomas_gqa_attn",
                     "nomas_seg_attn_bwd",
                     "nomas_w8a16_linear", "nomas_w8a16_linear_noalloc",
                     "nomas_cam_tokens",
                     "nomas_cam_xattn", "nomas_rope_table"):
            getattr(L, name).restype = _I
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().nomas_strerror(int(code)).decode()


def version() -> str:
    return lib().nomas_version().decode()


def shutdown() -> None:
    """Drop the library's per-device host state (nomas_shutdown)."""
    _check(lib().nomas_shutdown(), "nomas_shutdown")


def _check(rc: int, where: str):
    if rc != OK:
        raise NomasError(rc, where)


def seg_array(segs):
    """A ctypes array of nomas_seg from (n_text, t0, T, Hg, Wg) tuples or objects with astuple()."""
    tup = [tuple(s.astuple()) if hasattr(s, "astuple") else tuple(s) for s in segs]
    arr = (Seg * max(1, len(tup)))()
    for i, t in enumerate(tup):
        arr[i] = Seg(*[int(v) for v in t])
    return arr, len(tup)


def seg_tokens(segs) -> int:
    n = 0
    for s in segs:
        t = tuple(s.astuple()) if hasattr(s, "astuple") else tuple(s)
        n += t[0] + t[2] * t[3] * t[4]
    return n


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _torch_stream(stream):
    """The torch stream object for `stream` (None: the current stream; an
    int: a raw hipStream_t handle, wrapped without taking ownership)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def _alloc_on(stream):
    """Context for the tensors a call allocates (outputs, workspace).

    PyTorch's caching allocator hands a freed block to the next allocation on
    the stream the block was allocated on, ordered by that stream alone.  A
    workspace allocated on the current stream but written by kernels queued
    on another stream could therefore be reused while those kernels still
    run.  Allocating under the call's own stream makes the reuse wait behind
    the call's kernels."""
    import contextlib
    import torch
    if stream is None:
        return contextlib.nullcontext()
    return torch.cuda.stream(_torch_stream(stream))


def _workspace(need, device, workspace, stream):
    """The caller's workspace (checked), or a new one on the call's stream."""
    import torch
    if workspace is None:
        with _alloc_on(stream):
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if not workspace.is_cuda or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device uint8 tensor")
    return workspace


def _dev(t, name, shape=None, elem=2):
    if t is None:
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.element_size() != elem:
        raise ValueError("%s must have %d-byte elements" % (name, elem))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI, without the prefix)


def rope3d(x, segs, out=None, stream=None):
    """3D RoPE of x [L][H][128] (bf16) -> out (new tensor unless given; may be x)."""
    import torch
    L, H = x.shape[0], x.shape[1]
    _dev(x, "x", (seg_tokens(segs), H, HEAD_DIM))
    if out is None:
        with _alloc_on(stream):
            out = torch.empty_like(x)
    _dev(out, "out", x.shape)
    arr, n = seg_array(segs)
    _check(lib().nomas_rope3d(_ptr(x), _ptr(out), arr, n, H, _stream(stream)), "nomas_rope3d")
    return out


def kv_quant_append(k_rot, v, k_codes, v_codes, k_scale, v_scale, length: int, stream=None) -> int:
    """Quantise k_rot, v [L][H][128] into the cache at `length`; returns the new length."""
    L, H = k_rot.shape[0], k_rot.shape[1]
    _dev(k_rot, "k_rot", (L, H, HEAD_DIM))
    _dev(v, "v", (L, H, HEAD_DIM))
    cap = k_codes.shape[1]
    _dev(k_codes, "k_codes", (H, cap, HEAD_DIM), 1)
    _dev(v_codes, "v_codes", (H, cap, HEAD_DIM), 1)
    _dev(k_scale, "k_scale", (H, cap), 4)
    _dev(v_scale, "v_scale", (H, cap), 4)
    ln = _I64(int(length))
    _check(lib().nomas_kv_quant_append(_ptr(k_rot), _ptr(v), L, H, _ptr(k_codes), _ptr(v_codes),
                                       _ptr(k_scale), _ptr(v_scale), cap, ctypes.byref(ln), _stream(stream)),
           "nomas_kv_quant_append")
    return int(ln.value)


def sel_arrays(sel, n_segs):
    """History selection -> (sel_off int32 [n+1], sel_ranges int64 [2r]) host
    arrays; sel is one list of (start, end) cache-token ranges per segment."""
    if len(sel) != n_segs:
        raise ValueError("sel needs one range list per new segment (%d), got %d" % (n_segs, len(sel)))
    off = np.zeros(n_segs + 1, np.int32)
    flat = []
    for a, ranges in enumerate(sel):
        for lo, hi in ranges:
            flat += [int(lo), int(hi)]
        off[a + 1] = len(flat) // 2
    return off, np.array(flat if flat else [0, 0], np.int64)


def seg_attn_workspace(new_segs, cache_len: int, H: int, n_split: int = 0, sel=None) -> int:
    """Bytes of device workspace seg_attn needs on the current device (host only)."""
    arr, n = seg_array(new_segs)
    if sel is None:
        nbytes = lib().nomas_seg_attn_workspace(arr, n, int(cache_len), int(H), int(n_split))
    else:
        off, rng = sel_arrays(sel, n)
        nbytes = lib().nomas_seg_attn_sel_workspace(arr, n, int(cache_len), off.ctypes.data, rng.ctypes.data, int(H),
                                                    int(n_split))
    if nbytes < 0:
        raise NomasError(int(nbytes), "nomas_seg_attn_workspace")
    return int(nbytes)


def seg_attn(q, k_new, v_new, new_segs, k_codes=None, v_codes=None, k_scale=None, v_scale=None,
             cache_len: int = 0, sm_scale: float = SM_SCALE, out=None, lse=None, workspace=None, n_split: int = 0,
             stream=None, sel=None):
    """Segment-causal attention; returns out [Ln][H][128] bf16 (lse filled if given).
    q and k_new are taken before RoPE (rotated inside).  workspace:
    a device uint8 tensor of at least seg_attn_workspace(...) bytes, allocated
    here when not given.  n_split: 0 = the library's choice of key-range parts,
    1..4 forces that many.  sel: None (whole cache) or, per new segment, a
    list of (start, end) cache-token ranges it may see (nomas_seg_attn_sel)."""
    import torch
    Ln, H = q.shape[0], q.shape[1]
    shp = (seg_tokens(new_segs), H, HEAD_DIM)
    _dev(q, "q", shp)
    _dev(k_new, "k_new", shp)
    _dev(v_new, "v_new", shp)
    cap = 0
    if cache_len > 0:
        cap = k_codes.shape[1]
        _dev(k_codes, "k_codes", (H, cap, HEAD_DIM), 1)
        _dev(v_codes, "v_codes", (H, cap, HEAD_DIM), 1)
        _dev(k_scale, "k_scale", (H, cap), 4)
        _dev(v_scale, "v_scale", (H, cap), 4)
    elif k_codes is not None:
        cap = k_codes.shape[1]
    if out is None:
        with _alloc_on(stream):
            out = torch.empty_like(q)
    _dev(out, "out", shp)
    if lse is not None:
        _dev(lse, "lse", (H, Ln), 4)
    need = seg_attn_workspace(new_segs, cache_len, H, n_split, sel)
    workspace = _workspace(need, q.device, workspace, stream)
    arr, n = seg_array(new_segs)
    if sel is None:
        _check(lib().nomas_seg_attn(_ptr(q), _ptr(k_new), _ptr(v_new), arr, n, _ptr(k_codes), _ptr(v_codes),
                                    _ptr(k_scale), _ptr(v_scale), cap, int(cache_len), H, float(sm_scale),
                                    _ptr(out), _ptr(lse), int(n_split), _ptr(workspace), workspace.numel(),
                                    _stream(stream)),
               "nomas_seg_attn")
    else:
        off, rng = sel_arrays(sel, n)
        _check(lib().nomas_seg_attn_sel(_ptr(q), _ptr(k_new), _ptr(v_new), arr, n, _ptr(k_codes), _ptr(v_codes),
                                        _ptr(k_scale), _ptr(v_scale), cap, int(cache_len), off.ctypes.data,
                                        rng.ctypes.data, H, float(sm_scale), _ptr(out), _ptr(lse), int(n_split),
                                        _ptr(workspace), workspace.numel(), _stream(stream)),
               "nomas_seg_attn_sel")
    return out


def seg_attn_bwd_workspace(segs, H: int) -> int:
    """Bytes of device workspace seg_attn_bwd needs (host only)."""
    arr, n = seg_array(segs)
    nbytes = lib().nomas_seg_attn_bwd_workspace(arr, n, int(H))
    if nbytes < 0:
        raise NomasError(int(nbytes), "nomas_seg_attn_bwd_workspace")
    return int(nbytes)


def seg_attn_bwd(q, k, v, out, lse, d_out, segs, sm_scale: float = SM_SCALE, dq=None, dk=None, dv=None,
                 workspace=None, stream=None):
    """Gradients of packed segment-causal attention (seg_attn with several
    segments and no cache): q, k (before RoPE), v, the forward's out and lse,
    and d_out; returns (dq, dk, dv), float32 [L][H][128]."""
    import torch
    L, H = q.shape[0], q.shape[1]
    shp = (seg_tokens(segs), H, HEAD_DIM)
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (d_out, "d_out")):
        _dev(t, name, shp)
    _dev(lse, "lse", (H, L), 4)
    grads = []
    for g, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if g is None:
            with _alloc_on(stream):
                g = torch.empty(shp, dtype=torch.float32, device=q.device)
        _dev(g, name, shp, 4)
        grads.append(g)
    need = seg_attn_bwd_workspace(segs, H)
    workspace = _workspace(need, q.device, workspace, stream)
    arr, n = seg_array(segs)
    _check(lib().nomas_seg_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(d_out), arr, n, H,
                                    float(sm_scale), _ptr(grads[0]), _ptr(grads[1]), _ptr(grads[2]),
                                    _ptr(workspace), workspace.numel(), _stream(stream)), "nomas_seg_attn_bwd")
    return tuple(grads)


def gqa_attn_workspace(L: int, Hq: int, Hkv: int) -> int:
    """Bytes of device workspace gqa_attn needs (host only)."""
    nbytes = lib().nomas_gqa_attn_workspace(int(L), int(Hq), int(Hkv))
    if nbytes < 0:
        raise NomasError(int(nbytes), "nomas_gqa_attn_workspace")
    return int(nbytes)


def gqa_attn(q, k, v, sm_scale: float = SM_SCALE, out=None, lse=None, workspace=None, stream=None):
    """Decoder window attention with grouped KV heads: q [L][Hq][128],
    k, v [L][Hkv][128] (bf16); every token attends to every token; query head
    h uses KV head h // (Hq // Hkv).  Returns out [L][Hq][128]."""
    import torch
    L, Hq, Hkv = q.shape[0], q.shape[1], k.shape[1]
    _dev(q, "q", (L, Hq, HEAD_DIM))
    _dev(k, "k", (L, Hkv, HEAD_DIM))
    _dev(v, "v", (L, Hkv, HEAD_DIM))
    if out is None:
        with _alloc_on(stream):
            out = torch.empty_like(q)
    _dev(out, "out", q.shape)
    if lse is not None:
        _dev(lse, "lse", (Hq, L), 4)
    need = gqa_attn_workspace(L, Hq, Hkv)
    workspace = _workspace(need, q.device, workspace, stream)
    _check(lib().nomas_gqa_attn(_ptr(q), _ptr(k), _ptr(v), L, Hq, Hkv, float(sm_scale), _ptr(out), _ptr(lse),
                                _ptr(workspace), workspace.numel(), _stream(stream)), "nomas_gqa_attn")
    return out


def w8a16_linear_workspace(K: int, N: int) -> int:
    """Bytes of device workspace w8a16_linear needs (host only)."""
    nbytes = lib().nomas_w8a16_linear_workspace(int(K), int(N))
    if nbytes < 0:
        raise NomasError(int(nbytes), "nomas_w8a16_linear_workspace")
    return int(nbytes)


def w8a16_linear(x, w_codes, w_scale, out=None, workspace=None, stream=None):
    """y = x . W^T with INT8 weights (codes [N][K] int8, scales [N] float32)
    and BF16 math; x [M][K] bf16 -> y [M][N] bf16."""
    import torch
    M, K = x.shape
    N = w_codes.shape[0]
    _dev(x, "x", (M, K))
    _dev(w_codes, "w_codes", (N, K), 1)
    _dev(w_scale, "w_scale", (N,), 4)
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _dev(out, "out", (M, N))
    need = w8a16_linear_workspace(K, N)
    workspace = _workspace(need, x.device, workspace, stream)
    _check(lib().nomas_w8a16_linear(_ptr(x), M, K, _ptr(w_codes), _ptr(w_scale), N, _ptr(out), _ptr(workspace),
                                    workspace.numel(), _stream(stream)), "nomas_w8a16_linear")
    return out


W8A16_NOALLOC_MAX_BYTES = 32 << 20


def w8a16_linear_noalloc(x, w_codes, w_scale, out, stream=None):
    """w8a16_linear without a workspace (nomas_w8a16_linear_noalloc): the
    library's static per-device scratch holds the dequantised weights, so the
    call allocates nothing; `out` [M][N] must be given.  Calls that overlap
    in time on one device share that scratch and race."""
    M, K = x.shape
    N = w_codes.shape[0]
    _dev(x, "x", (M, K))
    _dev(w_codes, "w_codes", (N, K), 1)
    _dev(w_scale, "w_scale", (N,), 4)
    _dev(out, "out", (M, N))
    _check(lib().nomas_w8a16_linear_noalloc(_ptr(x), M, K, _ptr(w_codes), _ptr(w_scale), N, _ptr(out),
                                            _stream(stream)), "nomas_w8a16_linear_noalloc")
    return out


def cam_tokens(c2w, translation_scale: float = 1.0, rotation_scale: float = 2.5) -> np.ndarray:
    """Host: c2w [N][4][4] float64 -> camera tokens [N/4][64] float32."""
    c = np.ascontiguousarray(c2w, dtype=np.float64)
    N = c.shape[0]
    out = np.zeros((N // 4, 64), np.float32)
    _check(lib().nomas_cam_tokens(c.ctypes.data, N, float(translation_scale), float(rotation_scale),
                                  out.ctypes.data), "nomas_cam_tokens")
    return out


def cam_xattn_workspace(H: int, Nc: int) -> int:
    """Bytes of device workspace cam_xattn needs (host only)."""
    nbytes = lib().nomas_cam_xattn_workspace(int(H), int(Nc))
    if nbytes < 0:
        raise NomasError(int(nbytes), "nomas_cam_xattn_workspace")
    return int(nbytes)


def cam_xattn(q, cam, w_k, w_v, sm_scale: float = SM_SCALE, out=None, workspace=None, stream=None):
    """Camera cross-attention of q [Lq][H][128] over cam [Nc][64] (float32,
    device).  workspace: a device uint8 tensor of at least
    cam_xattn_workspace(H, Nc) bytes, allocated here when not given."""
    import torch
    Lq, H = q.shape[0], q.shape[1]
    _dev(q, "q", (Lq, H, HEAD_DIM))
    Nc = cam.shape[0]
    _dev(cam, "cam", (Nc, 64), 4)
    _dev(w_k, "w_k", (64, H * HEAD_DIM))
    _dev(w_v, "w_v", (64, H * HEAD_DIM))
    if out is None:
        with _alloc_on(stream):
            out = torch.empty_like(q)
    _dev(out, "out", q.shape)
    workspace = _workspace(cam_xattn_workspace(H, Nc), q.device, workspace, stream)
    _check(lib().nomas_cam_xattn(_ptr(q), Lq, H, _ptr(cam), Nc, _ptr(w_k), _ptr(w_v), float(sm_scale),
                                 _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)), "nomas_cam_xattn")
    return out


def rope_table(axis: int, npos: int):
    """Host copy of the library's float32 RoPE table: (cos, sin) [npos][d/2]."""
    d = 16 if axis == 0 else 56
    c = np.zeros((npos, d // 2), np.float32)
    s = np.zeros((npos, d // 2), np.float32)
    _check(lib().nomas_rope_table(axis, npos, c.ctypes.data, s.ctypes.data), "nomas_rope_table")
    return c, s
