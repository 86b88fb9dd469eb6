"""numpy float64 definitions of the segment-causal attention path (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Nothing here is tuned;
each function is the plain definition, cut into independent (head, query
block) pieces only so that large inputs fit in memory.

Pages cited (by title and section):
  [CW] comfyui-wiki news, "Hy-Nomas：腾讯混元交互式世界模型，8 步生成 720p 可控视频":
       "一个世界，分段生成" (segment-autoregressive, causal between segments,
       attends to the K/V cache of every earlier segment), "相机控制作为一等输入"
       (c2w [N,4,4], normalised, grouped per 4 frames, 64-d, cross-attention,
       translation scale 1.0 / rotation scale 2.5), "模型内部" table (16 heads x
       128, 3D RoPE [16,56,56] theta 256, patch 1x1x1, DCAE-V f32t4c32),
       "单张 4090 配置" (cached keys and values stored INT8, attention computed
       in BF16).
  [HW] huaweicloud blog "Hy-Nomas:8B 参数、单张 4090 跑 60 秒可控世界",
       section 2.1 (text/video K,V of each segment cached and passed on; the two
       streams interact in every block) and the section 3.5 table (INT8 weights
       and INT8 KV cache, BF16 compute).

Readings where the pages are silent (each is listed in the design notes):
  * RoPE pairs are interleaved (2i, 2i+1) inside each axis chunk, chunks in the
    order t, h, w; omega_i = 256^(-2i/d); text tokens are not rotated; t is
    the absolute latent-frame index, h and w start at 0.
  * INT8: symmetric, one fp32 scale per (token, head) s = fl32(absmax/127),
    codes rne(x/s) with the exact quotient, clamped to [-127, 127]; an all-zero
    row has s = 0 and codes 0.  Keys are cached after RoPE.
  * "Attention computed in BF16": the operands that enter the two attention
    products are BF16 values -- rotated Q and K rounded to BF16, cached K/V
    dequantised as bf16(fl32(code * scale)).  Scores, softmax and sums are
    exact here (float64).
  * Gradients (packed training, [HW] 2.3): the bf16 rounding of the rotated
    q and k is a cast whose derivative is the identity; the backward pass is
    otherwise the exact chain rule of the exact forward.
  * Camera tokens: poses made relative to the first frame of the turn,
    translation x translation_scale, rotation angle x rotation_scale
    (axis-angle), 4 consecutive 4x4 matrices flattened row-major into 64
    values.  The embedding is a BF16 linear layer: Kc = bf16(bf16(cam) @ Wk),
    Vc = bf16(bf16(cam) @ Wv); every video query attends to every camera
    token of its turn.
"""
from __future__ import annotations

import math

import numpy as np

D = 128
THETA = 256.0
AXES = (16, 56, 56)          # channel widths for t, h, w
AXIS_OFFSETS = (0, 16, 72)
QMAX = 127

__all__ = [
    "D", "THETA", "AXES", "AXIS_OFFSETS", "QMAX",
    "bf16_bits_to_f64", "bf16_round", "f64_to_bf16_bits",
    "token_positions", "rope_omega", "rope_table_f32", "rope3d", "rope3d_pos",
    "quantise", "dequant", "dequant_bf16", "build_cache",
    "values", "seg_ends", "attend", "seg_attn", "seg_attn_bwd", "gqa_attn", "w8a16_linear", "cam_tokens", "cam_kv", "cam_xattn",
]


# ----------------------------------------------------------------------------
# bfloat16 values


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 values (exact)."""
    return (np.asarray(b).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def values(x) -> np.ndarray:
    """Tensor values as float64: uint16 arrays are bfloat16 bit patterns,
    floating-point arrays are taken as they are (finite-difference checks
    perturb inputs by amounts no bfloat16 can hold)."""
    x = np.asarray(x)
    return bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits: write x = m * 2^e with m in [0.5, 1);
    the rounded value is rint(m * 256) * 2^(e - 8) (rint is half-to-even and
    m * 256 is exact).  Results are returned as float64.  Finite normal
    range only, which is all the workloads produce.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 values that are already bfloat16 values -> uint16 bits."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# token layout  ([CW] 模型内部: patch 1x1x1, 880 tokens per 1280x704 latent frame;
#                [HW] 2.1: text and video streams processed jointly)


def token_positions(segs):
    """For the concatenation of segments (n_text, t0, T, Hg, Wg): per token a
    video flag and the (t, h, w) latent-grid position.  Each segment lists its
    n_text text tokens first, then its video tokens in (t, h, w) row-major
    order with t in [t0, t0+T)."""
    vids, ts, hs, ws = [], [], [], []
    for s in segs:
        n_text, t0, T, Hg, Wg = (int(v) for v in tuple(s.astuple() if hasattr(s, "astuple") else s))
        nv = T * Hg * Wg
        idx = np.arange(nv, dtype=np.int64)
        vids.append(np.concatenate([np.zeros(n_text, bool), np.ones(nv, bool)]))
        ts.append(np.concatenate([np.zeros(n_text, np.int64), t0 + idx // (Hg * Wg)]))
        hs.append(np.concatenate([np.zeros(n_text, np.int64), (idx // Wg) % Hg]))
        ws.append(np.concatenate([np.zeros(n_text, np.int64), idx % Wg]))
    if not vids:
        z = np.zeros(0, np.int64)
        return np.zeros(0, bool), z, z, z
    return np.concatenate(vids), np.concatenate(ts), np.concatenate(hs), np.concatenate(ws)


# ----------------------------------------------------------------------------
# 3D RoPE  ([CW] 模型内部: 3D RoPE, sizes [16, 56, 56], theta 256)


def rope_omega(axis: int) -> np.ndarray:
    """Angular frequencies of one axis chunk: omega_i = theta^(-2i/d), i < d/2."""
    d = AXES[axis]
    i = np.arange(d // 2, dtype=np.float64)
    return THETA ** (-2.0 * i / d)


def rope_table_f32(axis: int, npos: int):
    """cos and sin of p * omega_i for positions p < npos, rounded to float32.
    Used only to check that the library's own table holds the same numbers."""
    phi = np.arange(npos, dtype=np.float64)[:, None] * rope_omega(axis)[None, :]
    return np.cos(phi).astype(np.float32), np.sin(phi).astype(np.float32)


def rope3d_pos(x, vid, t, h, w, inverse=False) -> np.ndarray:
    """Rotate x [L][H][128] (float64) by the 3D RoPE angles of each token.

    Channel chunk a (t: [0,16), h: [16,72), w: [72,128)) of width d holds d/2
    pairs (2i, 2i+1); pair i turns by phi = p_a * omega_i:
        (x0, x1) -> (x0 cos phi - x1 sin phi, x0 sin phi + x1 cos phi).
    Text tokens (vid False) are left unchanged.  inverse=True turns by -phi,
    the transpose of the rotation (how a gradient goes back through it).
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    if not np.any(vid):
        return out
    pos = (t, h, w)
    xv = x[vid]
    ov = xv.copy()
    for a in range(3):
        off, d = AXIS_OFFSETS[a], AXES[a]
        phi = pos[a][vid].astype(np.float64)[:, None] * rope_omega(a)[None, :]
        c = np.cos(phi)[:, None, :]
        s = -np.sin(phi)[:, None, :] if inverse else np.sin(phi)[:, None, :]
        x0 = xv[:, :, off:off + d:2]
        x1 = xv[:, :, off + 1:off + d:2]
        ov[:, :, off:off + d:2] = x0 * c - x1 * s
        ov[:, :, off + 1:off + d:2] = x0 * s + x1 * c
    out[vid] = ov
    return out


def rope3d(x, segs) -> np.ndarray:
    """3D RoPE of the tokens of ``segs`` (concatenated) -- see rope3d_pos."""
    return rope3d_pos(x, *token_positions(segs))


# ----------------------------------------------------------------------------
# INT8 KV storage  ([CW] 单张 4090 配置 and [HW] 3.5: cached K/V stored INT8)


def quantise(x):
    """Symmetric absmax INT8 quantisation of each 128-value row of x.

    a = max|x_i|; s = fl32(a / 127); q_i = clamp(rne(x_i / s), -127, 127).
    The quotient is taken in float64: for bfloat16 x and float32 s its error
    is below 2^-46 while x/s lies at least 2^-25 away from any half-integer it
    is not equal to, so rounding it gives the exact rne.  a / 127 in float64
    never lands on a float32 rounding midpoint (1/127 has a 7-periodic binary
    expansion), so the float32 cast rounds the exact quotient.
    Returns (codes int8 [..., 128], scales float32 [...]).  a = 0 -> s = 0.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.max(np.abs(x), axis=-1)
    s = (a / float(QMAX)).astype(np.float32)
    sd = s.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(sd > 0, x / np.where(sd > 0, sd, 1.0), 0.0)
    q = np.clip(np.rint(r), -QMAX, QMAX).astype(np.int8)
    return q, s


def dequant(codes, scale) -> np.ndarray:
    """Exact dequantisation q * s (a 7-bit by 24-bit product fits float64)."""
    return np.asarray(codes).astype(np.float64) * np.asarray(scale, dtype=np.float64)[..., None]


def dequant_bf16(codes, scale) -> np.ndarray:
    """The BF16 operand of a cached key or value: bf16(fl32(q * s))."""
    p = np.asarray(codes).astype(np.float32) * np.asarray(scale, dtype=np.float32)[..., None]
    return bf16_round(p.astype(np.float64))


def build_cache(k_hist_bits, v_hist_bits, hist_segs, cap=None):
    """History K/V (bf16 bits, pre-RoPE keys, [Lc][H][128]) -> INT8 cache in
    head-major layout: codes [H][cap][128], scales [H][cap].  Keys are rotated
    at their history positions and rounded to BF16 before quantisation."""
    k = bf16_bits_to_f64(k_hist_bits)
    v = bf16_bits_to_f64(v_hist_bits)
    Lc, H, _ = k.shape
    cap = Lc if cap is None else cap
    kc = np.zeros((H, cap, D), np.int8)
    vc = np.zeros((H, cap, D), np.int8)
    ks = np.zeros((H, cap), np.float32)
    vs = np.zeros((H, cap), np.float32)
    pos = token_positions(hist_segs)
    for h in range(H):
        kr = bf16_round(rope3d_pos(k[:, h:h + 1, :], *pos))[:, 0, :]
        kc[h, :Lc], ks[h, :Lc] = quantise(kr)
        vc[h, :Lc], vs[h, :Lc] = quantise(v[:, h, :])
    return kc, vc, ks, vs


# ----------------------------------------------------------------------------
# segment-causal attention  ([CW] 一个世界，分段生成; [HW] 2.1)


def seg_ends(new_segs) -> np.ndarray:
    """Exclusive end (token index into the new tokens) of each new segment."""
    n = [int((s.astuple() if hasattr(s, "astuple") else s)[0]) +
         int(np.prod((s.astuple() if hasattr(s, "astuple") else s)[2:5])) for s in new_segs]
    return np.cumsum(np.asarray(n, dtype=np.int64))


def attend(qr, K, V, sm_scale):
    """Softmax attention of rows qr [n][128] over keys K [m][128], values
    V [m][128], all float64: s = sm_scale * <q, k>, p = softmax(s), o = p V,
    lse = ln sum exp(s)."""
    S = (qr @ K.T) * float(sm_scale)
    mx = S.max(axis=1, keepdims=True)
    E = np.exp(S - mx)
    l = E.sum(axis=1)
    O = (E @ V) / l[:, None]
    return O, mx[:, 0] + np.log(l)


def seg_attn(q_bits, k_new_bits, v_new_bits, new_segs, k_codes, v_codes, k_scale, v_scale,
             cache_len, sm_scale, rows=None, heads=None, bf16_operands=True, block=None, sel=None):
    """Segment-causal attention of the new tokens.

    Query i of new segment a attends to every cached token (the INT8 history of
    all earlier segments) and to the new tokens of segments 0..a (bidirectional
    inside its own segment, never to a later segment).

    sel (history selection): None, or per new segment a list of (start, end)
    ranges of cache tokens; segment a then attends to the cache tokens in its
    ranges instead of the whole cache.  The pages let the history a segment
    looks at be a chosen subset of the earlier frames: the most recent latent
    frames or frames sampled by temporal_context ([HW] section 3.5 table;
    [CW] 单张 4090 配置), chosen by the kind of action ([HW] section 2.2).
    Reading: the caller names the cache tokens; the allowed set is their
    union with the new tokens of segments 0..a.

    q, k_new, v_new: bf16 bits [Ln][H][128]; q and k_new are pre-RoPE.
    k_codes, v_codes: int8 [H][cap][128]; k_scale, v_scale: float32 [H][cap];
    the first cache_len entries are valid (cached keys are post-RoPE).
    Returns out [len(rows)][len(heads)][128] and lse [len(heads)][len(rows)]
    (natural log), float64.  With bf16_operands the rotated q/k and the
    dequantised cache enter the products as BF16 values; otherwise exactly.
    """
    q = np.asarray(q_bits)
    Ln, H, _ = q.shape
    rows = np.arange(Ln) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(H)) if heads is None else list(heads)
    ends = seg_ends(new_segs)
    assert ends[-1] == Ln, "token counts disagree with the segment descriptors"
    seg_of = np.searchsorted(ends, rows, side="right")
    pos = token_positions(new_segs)
    rnd = bf16_round if bf16_operands else (lambda a: a)
    deq = dequant_bf16 if bf16_operands else dequant
    Lc = int(cache_len)
    out = np.zeros((len(rows), len(heads), D))
    lse = np.zeros((len(heads), len(rows)))
    for hi, h in enumerate(heads):
        Kc = deq(k_codes[h, :Lc], k_scale[h, :Lc]) if Lc else np.zeros((0, D))
        Vc = deq(v_codes[h, :Lc], v_scale[h, :Lc]) if Lc else np.zeros((0, D))
        kmax = int(ends[seg_of.max()]) if len(rows) else 0
        kn = values(k_new_bits[:kmax, h:h + 1, :])
        Kn = rnd(rope3d_pos(kn, *(p[:kmax] for p in pos)))[:, 0, :]
        Vn = values(v_new_bits[:kmax, h, :])
        qs = values(q[rows, h:h + 1, :])
        Qr = rnd(rope3d_pos(qs, *(p[rows] for p in pos)))[:, 0, :]
        for a in np.unique(seg_of):
            mine = np.nonzero(seg_of == a)[0]
            e = int(ends[a])
            if sel is None:
                Ka, Va = Kc, Vc
            else:
                idx = np.array([j for (lo, hi) in sel[a] for j in range(int(lo), int(hi))], dtype=np.int64)
                assert len(idx) == 0 or (idx.min() >= 0 and idx.max() < Lc), "selection outside the cache"
                Ka, Va = Kc[idx], Vc[idx]
            K = np.concatenate([Ka, Kn[:e]])
            V = np.concatenate([Va, Vn[:e]])
            blk = block or int(max(8, min(256, (1 << 24) // max(1, len(K)))))
            for lo in range(0, len(mine), blk):
                r = mine[lo:lo + blk]
                o, l = attend(Qr[r], K, V, sm_scale)
                out[r, hi] = o
                lse[hi, r] = l
    return out, lse


def seg_attn_bwd(q_bits, k_bits, v_bits, do_bits, segs, sm_scale, rows=None, heads=None,
                 bf16_operands=True, want_kv=True, block=None, keys=None):
    """Gradients of packed segment-causal attention (training direction).

    The packed training sequence of the segment-forcing LoRA recipe
    ([HW] section 2.3: packed sequences of up to 360,000 tokens) is a chain of
    segments with the block-causal mask of seg_attn and no cache: query i of
    segment a attends to the tokens of segments 0..a.  For a loss whose
    gradient with respect to the attention output is dO, the chain rule
    through softmax attention gives, per head, with the allowed keys only:
        S = sm_scale Qr Kr^T,  P = softmax_row(S),  O = P V
        dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
        dS = P * (dP - D),  dQr = sm_scale dS Kr,  dKr = sm_scale dS^T Qr
    and through the rotation (Qr = R q, Kr = R k, R orthogonal per token):
        dq = R^T dQr,  dk = R^T dKr.
    Reading: the bf16 rounding of the rotated q and k (bf16_operands) is a
    cast whose derivative is taken as the identity; P and every sum are exact.

    q, k, v, dO: [Ln][H][128], bf16 bits (uint16) or float64 values; q and k
    before RoPE.  Returns (dq, dk, dv): dq [len(rows)][len(heads)][128] and,
    with want_kv, dk and dv [Ln][len(heads)][128] (else None), float64.

    keys (key-subset mode, for long sequences): token indices whose dk and dv
    are wanted.  The gradient of key j sums over the queries that see it
    (segments at or after j's), and each of those needs its whole softmax row
    (P over all its keys, O for D), so those rows are formed in full; only
    the columns of the chosen keys are kept for dP, dS, dk and dv.  Returns
    (None, dk, dv) with dk, dv [len(keys)][len(heads)][128]; dq is not formed.
    """
    q = np.asarray(q_bits)
    Ln, H, _ = q.shape
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(Ln) if rows is None else np.asarray(rows, dtype=np.int64)
    ends = seg_ends(segs)
    assert ends[-1] == Ln, "token counts disagree with the segment descriptors"
    pos = token_positions(segs)
    rnd = bf16_round if bf16_operands else (lambda a: a)
    sc = float(sm_scale)
    if keys is not None:
        kidx = np.asarray(keys, dtype=np.int64)
        assert len(kidx) and kidx.min() >= 0 and kidx.max() < Ln, "keys outside the sequence"
        want_kv = True
        first = int(np.searchsorted(ends, kidx.min(), side="right"))
        need = np.arange(0 if first == 0 else int(ends[first - 1]), Ln)   # queries that see a chosen key
    else:
        kidx = np.arange(Ln)
        # query rows whose softmax rows are needed: all of them for dk and dv
        need = np.arange(Ln) if want_kv else rows
    seg_of = np.searchsorted(ends, need, side="right")
    dq_r = np.zeros((Ln, len(heads), D)) if keys is None else None
    dk_r = np.zeros((len(kidx), len(heads), D)) if want_kv else None
    dv = np.zeros((len(kidx), len(heads), D)) if want_kv else None
    for hi, h in enumerate(heads):
        Qr = rnd(rope3d_pos(values(q[:, h:h + 1, :]), *pos))[:, 0, :]
        Kr = rnd(rope3d_pos(values(np.asarray(k_bits)[:, h:h + 1, :]), *pos))[:, 0, :]
        V = values(np.asarray(v_bits)[:, h, :])
        dO = values(np.asarray(do_bits)[:, h, :])
        for a in np.unique(seg_of):
            mine = need[seg_of == a]
            e = int(ends[a])
            K, Va = Kr[:e], V[:e]
            vis = np.nonzero(kidx < e)[0]         # chosen keys this segment's queries see
            cols = kidx[vis] if keys is not None else slice(None)
            blk = block or int(max(8, min(256, (1 << 23) // max(1, e))))
            for lo in range(0, len(mine), blk):
                r = mine[lo:lo + blk]
                S = sc * (Qr[r] @ K.T)
                E = np.exp(S - S.max(axis=1, keepdims=True))
                P = E / E.sum(axis=1, keepdims=True)
                O = P @ Va
                Dr = np.sum(dO[r] * O, axis=1)
                dP = dO[r] @ Va[cols].T
                dS = P[:, cols] * (dP - Dr[:, None])
                if keys is None:
                    dq_r[r, hi] = sc * (dS @ K)
                if want_kv:
                    dk_r[vis, hi] += sc * (dS.T @ Qr[r])
                    dv[vis, hi] += P[:, cols].T @ dO[r]
        del Qr, Kr, V, dO
    dq = None if keys is not None else rope3d_pos(dq_r[rows], *(p[rows] for p in pos), inverse=True)
    if not want_kv:
        return dq, None, None
    dk = rope3d_pos(dk_r, *(p[kidx] for p in pos), inverse=True)
    return dq, dk, dv


# ----------------------------------------------------------------------------
# decoder window attention  ([CW] 模型内部: the PixelUMM decoder has 32 query
# heads and 8 KV heads over a 4096-wide hidden state and reconstructs RGB from
# 4 x 16 x 16 tubelets on 10-latent-frame windows that overlap by 5 frames)


def gqa_attn(q_bits, k_bits, v_bits, sm_scale, rows=None, heads=None):
    """Attention of one decoder window with grouped KV heads.

    q: bf16 bits [L][Hq][128]; k, v: bf16 bits [L][Hkv][128], Hq a multiple
    of Hkv.  Query head h uses KV head h // (Hq / Hkv).  Reading (the pages
    give no mask or positions for the decoder): every token of the window
    attends to every token of it, the operands are the BF16 values as given
    (positions, if any, already applied), sm_scale is an argument.
    Returns out [len(rows)][len(heads)][128] and lse [len(heads)][len(rows)],
    float64 (lse in natural log)."""
    q = np.asarray(q_bits)
    L, Hq, _ = q.shape
    Hkv = np.asarray(k_bits).shape[1]
    assert Hq % Hkv == 0, "query heads must be a multiple of the KV heads"
    grp = Hq // Hkv
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    out = np.zeros((len(rows), len(heads), D))
    lse = np.zeros((len(heads), len(rows)))
    for hi, h in enumerate(heads):
        K = bf16_bits_to_f64(k_bits[:, h // grp, :])
        V = bf16_bits_to_f64(v_bits[:, h // grp, :])
        Q = bf16_bits_to_f64(q[rows, h, :])
        blk = int(max(8, min(256, (1 << 24) // max(1, L))))
        for lo in range(0, len(rows), blk):
            o, l = attend(Q[lo:lo + blk], K, V, sm_scale)
            out[lo:lo + blk, hi] = o
            lse[hi, lo:lo + blk] = l
    return out, lse


# ----------------------------------------------------------------------------
# INT8-weight linear layers  ([CW] 单张 4090 配置 and [HW] section 3.5 table:
# the DiT weights are stored INT8 while the linear layers compute in BF16;
# [CW] 模型内部: hidden size 2048)


def w8a16_linear(x_bits, w_codes, w_scale, rows=None):
    """y = x . W^T with INT8-stored weights and BF16 math.

    x: bf16 bits [M][K]; w_codes: int8 [N][K]; w_scale: float32 [N], one
    scale per output channel (the build's reading: the pages fix only INT8
    storage; the scale layout follows the KV cache's, one fp32 scale per
    row).  Each weight enters the product as the BF16 value
    bf16(fl32(code * scale)), as cached keys do; products and sums are exact
    here (float64).  Returns y [len(rows)][N] float64."""
    x = bf16_bits_to_f64(np.asarray(x_bits) if rows is None else np.asarray(x_bits)[np.asarray(rows)])
    W = dequant_bf16(w_codes, w_scale)
    return x @ W.T


# ----------------------------------------------------------------------------
# camera conditioning  ([CW] 相机控制作为一等输入; 模型内部: extrinsics embedded
#                       and injected by cross-attention in the dual-stream blocks)


HALF_TURN_SKEW = 1e-12


def _log_rotation(R):
    """Axis (unit) and angle in [0, pi] of a rotation matrix.

    For R = exp(ang [a]x) = cos(ang) I + sin(ang) [a]x + (1 - cos(ang)) a a^T
    the skew part is v = sin(ang) a and the symmetric part minus cos(ang) I
    is (1 - cos(ang)) a a^T.  Up to a right angle the axis is v / |v|.  Past
    it, sin(ang) shrinks towards zero at pi, so the axis magnitudes come from
    the symmetric part (accurate there, 1 - cos(ang) >= 1) and only the sign
    from v, whose largest-axis component keeps its sign until v vanishes.
    At a half turn a and -a give the same rotation (but not once the angle is
    scaled), and v is zero up to rounding; where that component of v is no
    larger than HALF_TURN_SKEW (1e-12, far above the rounding of products of
    orthonormal double matrices) the axis is taken with its largest component
    positive."""
    R = np.asarray(R, dtype=np.float64)
    v = 0.5 * np.array([R[2, 1] - R[1, 2], R[0, 2] - R[2, 0], R[1, 0] - R[0, 1]])
    s = float(np.linalg.norm(v))
    c = 0.5 * (float(np.trace(R)) - 1.0)
    ang = math.atan2(s, c)
    if c >= 0.0:
        if s == 0.0:                # the identity: angle 0, any axis
            return np.array([1.0, 0.0, 0.0]), 0.0
        return v / s, ang
    A = (0.5 * (R + R.T) - c * np.eye(3)) / (1.0 - c)      # = a a^T
    j = int(np.argmax(np.diag(A)))
    a = A[:, j] / math.sqrt(A[j, j])                        # component j positive
    if v[j] < -HALF_TURN_SKEW:
        a = -a
    return a / np.linalg.norm(a), ang


def _exp_rotation(axis, ang):
    x, y, z = axis
    K = np.array([[0, -z, y], [z, 0, -x], [-y, x, 0]], dtype=np.float64)
    return np.eye(3) + math.sin(ang) * K + (1.0 - math.cos(ang)) * (K @ K)


def cam_tokens(c2w, translation_scale=1.0, rotation_scale=2.5) -> np.ndarray:
    """64-d camera tokens of one turn from its c2w matrices [N][4][4].

    Each pose is made relative to the first frame (R0^T R_k, R0^T (t_k - t0)),
    its translation is multiplied by translation_scale and its rotation angle
    (axis-angle) by rotation_scale; groups of 4 consecutive frames give 4 x 16
    row-major values.  Returns float64 [N/4][64]."""
    c2w = np.asarray(c2w, dtype=np.float64)
    N = c2w.shape[0]
    assert N % 4 == 0, "the camera path must hold a multiple of 4 frames"
    R0, t0 = c2w[0, :3, :3], c2w[0, :3, 3]
    mats = np.zeros((N, 4, 4))
    for k in range(N):
        Rr = R0.T @ c2w[k, :3, :3]
        tr = R0.T @ (c2w[k, :3, 3] - t0)
        axis, ang = _log_rotation(Rr)
        mats[k, :3, :3] = _exp_rotation(axis, rotation_scale * ang)
        mats[k, :3, 3] = translation_scale * tr
        mats[k, 3, 3] = 1.0
    return mats.reshape(N // 4, 64)


def cam_kv(cam, w_k_bits, w_v_bits, H, bf16_operands=True):
    """Camera keys and values [Nc][H][128]: the camera embedding is a linear
    layer, and linear layers run in BF16 ([CW] 单张 4090 配置), so the tokens
    cam [Nc][64] are rounded to bf16, multiplied exactly by the bf16 weights
    [64][H*128], and the products rounded to bf16 as attention operands."""
    cam = np.asarray(cam, dtype=np.float64)
    if bf16_operands:
        cam = bf16_round(cam)
    Kc = cam @ bf16_bits_to_f64(w_k_bits)
    Vc = cam @ bf16_bits_to_f64(w_v_bits)
    if bf16_operands:
        Kc, Vc = bf16_round(Kc), bf16_round(Vc)
    Nc = cam.shape[0]
    return Kc.reshape(Nc, H, D), Vc.reshape(Nc, H, D)


def cam_xattn(q_bits, cam, w_k_bits, w_v_bits, sm_scale, rows=None, bf16_operands=True):
    """Camera cross-attention: every video query of the turn attends to all
    Nc camera tokens, per head (no RoPE).  q: bf16 bits [Lq][H][128];
    cam [Nc][64] (the float32 token values).  Returns float64 [rows][H][128]."""
    q = np.asarray(q_bits)
    Lq, H, _ = q.shape
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    Kc, Vc = cam_kv(cam, w_k_bits, w_v_bits, H, bf16_operands)
    out = np.zeros((len(rows), H, D))
    for h in range(H):
        qh = bf16_bits_to_f64(q[rows, h, :])
        for lo in range(0, len(rows), 4096):
            o, _ = attend(qh[lo:lo + 4096], Kc[:, h, :], Vc[:, h, :], sm_scale)
            out[lo:lo + 4096, h] = o
    return out
