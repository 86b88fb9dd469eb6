// Internal definitions shared by the libnomas kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nomas.h"

namespace nomas {

constexpr int D = NOMAS_HEAD_DIM;       // channels per head
constexpr int NPAIR_T = 8;              // RoPE pairs on the t axis (16 channels)
constexpr int NPAIR_HW = 28;            // RoPE pairs on the h and w axes (56 channels)

// A segment as the kernels see it: its first token index in the concatenated
// token array plus the descriptor fields.
struct SegDev {
    int32_t start, n_text, t0, T, Hg, Wg;
    float inv_hw, inv_w;      // 1/(Hg*Wg) and 1/Wg, for the float-estimated divisions below
};

struct SegTable {
    int32_t n;
    SegDev s[NOMAS_MAX_SEGS];
};

// Device addresses of the per-device RoPE tables.  One float32 and one
// float64 array each hold the three axis tables back to back: t at entry 0
// ([NOMAS_MAX_T][8]), h at ROPE_H0 and w at ROPE_W0 ([NOMAS_MAX_HW][28]
// each); entry (p, i) of an axis holds (cos, sin) of p * 256^(-2i/d).
constexpr int ROPE_H0 = NOMAS_MAX_T * NPAIR_T;
constexpr int ROPE_W0 = ROPE_H0 + NOMAS_MAX_HW * NPAIR_HW;
constexpr int ROPE_N = ROPE_W0 + NOMAS_MAX_HW * NPAIR_HW;
struct RopeTables {
    const float2* f32;
    const double2* f64;
};

// First table entry for the 4 channel pairs held by the 8-channel group
// `grp` (0..15) of a token at (t, h, w): groups 0-1 turn with t, 2-8 with h,
// 9-15 with w (the axis chunks are multiples of 8 channels).  Integer
// selects only, so lanes holding different groups do not diverge.
__device__ __forceinline__ int rope_entry(int grp, int t, int h, int w) {
    const int tt = t * NPAIR_T + 4 * grp;
    const int hh = ROPE_H0 + h * NPAIR_HW + 4 * (grp - 2);
    const int ww = ROPE_W0 + w * NPAIR_HW + 4 * (grp - 9);
    return grp < 2 ? tt : (grp < 9 ? hh : ww);
}

// Builds the tables on the current device on first use; returns NOMAS_OK or
// NOMAS_EHIP.  Thread-safe.
int rope_tables(RopeTables* out);

// Host-side float64 angle of pair i on an axis of width d at position p.
double rope_angle(int p, int i, int d);

// ----------------------------------------------------------------------------
// device helpers

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float nm_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 nm_bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16x2 (a in the low half), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    nm_f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, nm_bf16x2));
}

// Combine a per-lane value with the one in the other half of the wave
// (lane l and l^32) through v_permlane32_swap: the two returned registers hold
// the low and the high half broadcast, so a symmetric op of the pair gives the
// reduction over {l, l^32} in every lane.
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier that orders LDS only.  __syncthreads() is a full
// workgroup fence, which also waits for every outstanding global load; the
// key-tile prefetches must stay in flight across the per-tile barrier, and
// only the LDS tile writes need to be visible to the other waves.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// n / d for 0 <= n < 2^24, d >= 1, from a float estimate with inv = 1/d:
// the estimate is off by at most one, which one compare-and-step fixes.
__device__ __forceinline__ int fdiv(int n, int d, float inv) {
    int q = (int)((float)n * inv);
    int r = n - q * d;
    q += (r >= d) ? 1 : 0;
    q -= (r < 0) ? 1 : 0;
    return q;
}

// (t, h, w) of video token `loc` (counted from the first video token) of segment s.
__device__ __forceinline__ void video_pos(const SegDev& s, int loc, int& t, int& h, int& w) {
    const int hw = s.Hg * s.Wg;
    const int tt = fdiv(loc, hw, s.inv_hw);
    const int rem = loc - tt * hw;
    const int hh = fdiv(rem, s.Wg, s.inv_w);
    t = s.t0 + tt;
    h = hh;
    w = rem - hh * s.Wg;
}

// Position of token `idx` of the concatenated segments in `st`:
// video flag and (t, h, w).
__device__ __forceinline__ bool token_pos(const SegTable& st, int idx, int& t, int& h, int& w) {
    int a = 0;
    while (a + 1 < st.n && st.s[a + 1].start <= idx) ++a;
    const SegDev& s = st.s[a];
    const int loc = idx - s.start - s.n_text;
    if (loc < 0) { t = h = w = 0; return false; }
    video_pos(s, loc, t, h, w);
    return true;
}

// Rotate the 4 channel pairs held in a 16-byte group of 8 bf16 values at
// channels [8*grp, 8*grp+8) of a token at (t, h, w); float32 arithmetic with
// the float32 table, result rounded to bf16.
__device__ __forceinline__ uint4 rope_group_f32(uint4 x, int grp, int t, int h, int w,
                                                const RopeTables& rt) {
    const float4* tab = reinterpret_cast<const float4*>(rt.f32 + rope_entry(grp, t, h, w));
    const float4 c01 = tab[0], c23 = tab[1];      // (cos, sin) of pairs 0, 1 and 2, 3
    const float cs[8] = {c01.x, c01.y, c01.z, c01.w, c23.x, c23.y, c23.z, c23.w};
    const uint32_t in[4] = {x.x, x.y, x.z, x.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float c = cs[2 * i], sn = cs[2 * i + 1];
        const float x0 = bf16lo(in[i]), x1 = bf16hi(in[i]);
        o[i] = pack_bf16(x0 * c - x1 * sn, x0 * sn + x1 * c);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// float64 -> bf16, rounded once: truncating to float32 and setting the
// sticky bit when inexact (round-to-odd) keeps the final round-to-nearest-
// even to bf16 exact.
__device__ __forceinline__ uint32_t f64_to_bf16(double d) {
    float f = __double2float_rz(d);
    uint32_t b = __float_as_uint(f);
    if ((double)f != d) b |= 1u;
    b += 0x7fffu + ((b >> 16) & 1u);
    return b >> 16;
}

// one channel pair (x0, x1) rotated in float64 with separately rounded
// products (no fma contraction), each output rounded once to bf16
__device__ __forceinline__ uint32_t rot_pair_f64(uint32_t in, double2 cs) {
#pragma clang fp contract(off)
    double x0 = (double)bf16lo(in), x1 = (double)bf16hi(in);
    double y0 = x0 * cs.x - x1 * cs.y;
    double y1 = x0 * cs.y + x1 * cs.x;
    return f64_to_bf16(y0) | (f64_to_bf16(y1) << 16);
}

// 8 channels [8*grp, 8*grp+8) of token tok of the segments in st, rotated
// by 3D RoPE in float64 and rounded once to bf16; text tokens unchanged.
__device__ __forceinline__ uint4 rope_chunk_f64(uint4 w, int grp, int tok, const SegTable& st, const RopeTables& rt) {
    int t, h, ww;
    if (token_pos(st, tok, t, h, ww)) {
        const double2* tab = rt.f64 + rope_entry(grp, t, h, ww);
        w.x = rot_pair_f64(w.x, tab[0]);
        w.y = rot_pair_f64(w.y, tab[1]);
        w.z = rot_pair_f64(w.z, tab[2]);
        w.w = rot_pair_f64(w.w, tab[3]);
    }
    return w;
}

}  // namespace nomas
