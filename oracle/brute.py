"""Pure-Python brute force for tiny inputs (oracle pins).

TEST INFRASTRUCTURE ONLY.  Written separately from nomas_ref (no numpy, no
shared helpers) so that agreement between the two pins the vectorised code:
loops over (token, head, channel), math.fsum for every sum, and
fractions.Fraction for every rounding decision.  Same definitions and readings
as nomas_ref (see its docstring for the page citations).
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

D = 128


# ----------------------------------------------------------------------------
# exact rounding with rationals


def _round_to_bits(x: Fraction, mant_bits: int) -> Fraction:
    """Round a rational to the nearest value with ``mant_bits`` significant
    bits, ties to even (no exponent limits: normal range only)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # normalise so that 2^(mant_bits-1) <= a * 2^-e' < 2^mant_bits
    while a >= Fraction(2) ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    ulp = Fraction(2) ** (e - mant_bits + 1)
    return sign * round(a / ulp) * ulp     # round() on Fraction is half-to-even


def round_bf16(x) -> float:
    return float(_round_to_bits(Fraction(x), 8))


def round_f32(x) -> float:
    return float(_round_to_bits(Fraction(x), 24))


def bf16_from_bits(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]


# ----------------------------------------------------------------------------
# token layout and RoPE


def positions(segs):
    """List of (is_video, t, h, w) per token of the concatenated segments."""
    out = []
    for (n_text, t0, T, Hg, Wg) in segs:
        out += [(False, 0, 0, 0)] * n_text
        for t in range(T):
            for h in range(Hg):
                for w in range(Wg):
                    out.append((True, t0 + t, h, w))
    return out


def rope_vec(x, pos):
    """Rotate one 128-channel vector; pos = (is_video, t, h, w)."""
    vid, t, h, w = pos
    y = list(x)
    if not vid:
        return y
    off = 0
    for p, d in zip((t, h, w), (16, 56, 56)):
        for i in range(d // 2):
            ang = p * 256.0 ** (-2.0 * i / d)
            c, s = math.cos(ang), math.sin(ang)
            a, b = x[off + 2 * i], x[off + 2 * i + 1]
            y[off + 2 * i] = a * c - b * s
            y[off + 2 * i + 1] = a * s + b * c
        off += d
    return y


# ----------------------------------------------------------------------------
# quantiser


def quantise_row(x):
    """(codes, scale) of one row by exact rational arithmetic."""
    a = max(abs(Fraction(v)) for v in x)
    if a == 0:
        return [0] * len(x), 0.0
    s = _round_to_bits(a / 127, 24)
    codes = [max(-127, min(127, round(Fraction(v) / s))) for v in x]
    return codes, float(s)


# ----------------------------------------------------------------------------
# attention


def softmax_attend(qv, keys, vals, sm_scale):
    """(output vector, lse, probabilities) of one query over lists of keys/values."""
    sc = [sm_scale * math.fsum(a * b for a, b in zip(qv, k)) for k in keys]
    mx = max(sc)
    ex = [math.exp(s - mx) for s in sc]
    tot = math.fsum(ex)
    p = [e / tot for e in ex]
    o = [math.fsum(p[j] * vals[j][c] for j in range(len(vals))) for c in range(len(qv))]
    return o, mx + math.log(tot), p


def seg_attn(q, k_new, v_new, new_segs, cache_k, cache_v, sm_scale, bf16_operands=True, sel=None):
    """Brute-force segment-causal attention.

    q, k_new, v_new: nested lists [Ln][H][128] of floats (bf16 values, q/k
    pre-RoPE).  cache_k, cache_v: nested lists [H][Lc] of (codes, scale) rows.
    sel: None (every segment sees the whole cache) or, per new segment, a list
    of (start, end) cache-token ranges it may see (huaweicloud blog, section
    2.2 and the section 3.5 table; comfyui-wiki, 单张 4090 配置: the history a
    segment looks at is a chosen subset of the earlier frames).
    Returns out [Ln][H][128], lse [H][Ln], probs [H][Ln][keys]."""
    Ln, H = len(q), len(q[0])
    pos = positions(new_segs)
    ends, acc = [], 0
    for s in new_segs:
        acc += s[0] + s[2] * s[3] * s[4]
        ends.append(acc)
    rnd = round_bf16 if bf16_operands else (lambda v: v)

    def deq(codes, scale):
        if bf16_operands:
            return [round_bf16(round_f32(Fraction(c) * Fraction(scale))) for c in codes]
        return [float(Fraction(c) * Fraction(scale)) for c in codes]

    out = [[None] * H for _ in range(Ln)]
    lse = [[0.0] * Ln for _ in range(H)]
    probs = [[None] * Ln for _ in range(H)]
    for h in range(H):
        Kc = [deq(c, s) for (c, s) in cache_k[h]]
        Vc = [deq(c, s) for (c, s) in cache_v[h]]
        Kn = [[rnd(v) for v in rope_vec(k_new[j][h], pos[j])] for j in range(Ln)]
        Vn = [list(v_new[j][h]) for j in range(Ln)]
        for i in range(Ln):
            a = next(n for n, e in enumerate(ends) if i < e)
            qv = [rnd(v) for v in rope_vec(q[i][h], pos[i])]
            seen = range(len(Kc)) if sel is None else [j for (lo, hi) in sel[a] for j in range(lo, hi)]
            o, l, p = softmax_attend(qv, [Kc[j] for j in seen] + Kn[:ends[a]], [Vc[j] for j in seen] + Vn[:ends[a]],
                                     sm_scale)
            out[i][h], lse[h][i], probs[h][i] = o, l, p
    return out, lse, probs


def cam_xattn(q, cam, w_k, w_v, H, sm_scale, bf16_operands=True):
    """Brute-force camera cross-attention; q [Lq][H][128], cam [Nc][64],
    w_k/w_v [64][H*128] (floats).  Returns out [Lq][H][128]."""
    rnd = round_bf16 if bf16_operands else (lambda v: v)
    Nc = len(cam)
    cam = [[rnd(v) for v in row] for row in cam]
    Kc = [[rnd(math.fsum(cam[n][i] * w_k[i][c] for i in range(64))) for c in range(H * D)] for n in range(Nc)]
    Vc = [[rnd(math.fsum(cam[n][i] * w_v[i][c] for i in range(64))) for c in range(H * D)] for n in range(Nc)]
    out = []
    for qi in q:
        row = []
        for h in range(H):
            keys = [k[h * D:(h + 1) * D] for k in Kc]
            vals = [v[h * D:(h + 1) * D] for v in Vc]
            o, _, _ = softmax_attend(qi[h], keys, vals, sm_scale)
            row.append(o)
        out.append(row)
    return out
