// Segment-causal joint attention over the lifelong INT8 KV cache plus the
// current segment(s), for gfx950.
//
// What it computes (comfyui-wiki news page on Hy-Nomas, section 一个世界，分段生成;
// huaweicloud blog, section 2.1): query i of new segment a attends to every
// cached token and to the new tokens of segments 0..a, never to a later
// segment.  Cached K/V are INT8 with one fp32 scale per (token, head); the
// attention itself runs in BF16 (comfyui-wiki, 单张 4090 配置): cached entries
// enter the products as bf16(fl32(code*scale)), new Q/K are rotated by 3D RoPE
// (comfyui-wiki, 模型内部: [16, 56, 56], theta 256) on load and rounded to bf16.
//
// Kernel shape.  One workgroup = 4 waves x 64 query rows = 256 rows of one
// head, all inside one new segment, so every row allows the same keys:
// the cache [0, Lc) and the new tokens [0, end of its segment).  Later
// segments are never loaded.  Keys stream through LDS in tiles of 64,
// double-buffered: while the waves run the MFMAs of tile j from one buffer,
// the registers already hold tile j+1 from HBM, which is then dequantised
// (cache: int8 * scale -> bf16) or rotated (new keys: RoPE -> bf16) once per
// workgroup and written to the other buffer.  V is written transposed
// ([channel][key]) so that both products read 16 contiguous bytes per lane.
//
// Both products put the query on the MFMA's N side (v_mfma_f32_32x32x16_bf16):
//   S^T (keys x queries) = K (keys x d) . Q^T       A = K from LDS, B = Q in regs
//   O^T (d x queries)   += V^T (d x keys) . P^T     A = V^T from LDS, B = P in regs
// so the accumulator lane of S^T, P^T and O^T is the query itself: the
// running max, the sum and the rescale of O are lane-local, the two lane
// halves (l, l^32) hold disjoint keys of the same query, and P goes from the
// S^T accumulator straight into the B operand of the PV product: the keys a
// lane holds for a 16-key chunk are 16c + {4g..4g+3, 8+4g..8+4g+3} (g = lane
// half), and V^T is stored in LDS with each 16-key chunk permuted to
// [0-3, 8-11, 4-7, 12-15] so those 8 keys are contiguous.
// Softmax is online in base 2 (scale folded into one fma) with a lazy
// rescale: O and the sum are rescaled only when a row's max grows by more
// than 8 (a factor 256), which keeps every exponent bounded.
#include "common.hpp"

namespace nomas {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 64;              // keys per tile
constexpr int NW = 8;               // waves per workgroup (2 per SIMD)
constexpr int QW = 32;              // query rows per wave
constexpr int BM = NW * QW;         // query rows per workgroup
constexpr int NT = NW * 64;         // threads per workgroup
constexpr int KSTR = D + 8;         // LDS row stride of the K tile (bf16), padded
constexpr int VSTR = BN + 8;        // LDS row stride of the V^T tile (bf16), padded

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int8_t* kc;
    const int8_t* vc;
    const float* ks;
    const float* vs;
    uint16_t* out;
    float* lse;
    int64_t cap;
    int32_t Lc, Ln, H, ntq;         // ntq: query tiles per head
    float scale_log2;               // sm_scale * log2(e)
    int32_t tile0[NOMAS_MAX_SEGS + 1];   // first query tile of each new segment
    SegTable segs;
    RopeTables rt;
};

// This thread's share of one key tile on its way from HBM to LDS.
//   K: thread owns key row tid/8, channels 16*(tid%8) .. +16
//   V: thread owns keys 4*(tid%16) .. +4, channels 4*(tid/16) .. +4
struct Prefetch {
    uint4 a[2];       // K: cache 16 codes in a[0]; new 16 bf16 in a[0..1]
    uint32_t b[8];    // V: cache 4 keys x 4 codes in b[0..3]; new 4 keys x 4 bf16 in b[0..7]
    float sc[5];      // cache scales: K of the row, V of the 4 keys
};

// position (in the permuted V^T row) of key k, k a multiple of 4 inside a tile
__device__ __forceinline__ int vperm(int k) {
    int w = k & 15;
    int p = (w == 4) ? 8 : (w == 8) ? 4 : w;
    return (k & ~15) + p;
}

__device__ __forceinline__ float i8(uint32_t word, int byte) {
    return (float)(int8_t)(word >> (8 * byte));
}

// Loads are never guarded: key indices are clamped into the allowed range
// ([0, Lc) for the cache, [0, kend) for new keys), so every address is valid
// and the clamped rows are keys this workgroup may see anyway.  Keys past the
// range only occur in a tail tile, where their scores are masked to -inf and
// their probabilities are exactly 0.
__device__ __forceinline__ void load_tile(const AttnArgs& A, int head, int t, int nc, int kend, int tid,
                                          Prefetch& p) {
    const int krow = tid >> 3, kpart = tid & 7;
    const int kg = tid & 15, dq = tid >> 4;
    if (t < nc) {
        const int key0 = t * BN, last = A.Lc - 1;
        const int8_t* kc = A.kc + (int64_t)head * A.cap * D;
        const int8_t* vc = A.vc + (int64_t)head * A.cap * D;
        const float* ks = A.ks + (int64_t)head * A.cap;
        const float* vs = A.vs + (int64_t)head * A.cap;
        const int key = min(key0 + krow, last);
        p.a[0] = *reinterpret_cast<const uint4*>(kc + (int64_t)key * D + 16 * kpart);
        p.sc[0] = ks[key];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kv = min(key0 + 4 * kg + i, last);
            p.b[i] = *reinterpret_cast<const uint32_t*>(vc + (int64_t)kv * D + 4 * dq);
            p.sc[1 + i] = vs[kv];
        }
    } else {
        const int key0 = (t - nc) * BN, last = kend - 1;
        const int64_t rs = (int64_t)A.H * D;
        const uint16_t* kb = A.k + head * D;
        const uint16_t* vb = A.v + head * D;
        const int key = min(key0 + krow, last);
        const uint4* src = reinterpret_cast<const uint4*>(kb + key * rs + 16 * kpart);
        p.a[0] = src[0];
        p.a[1] = src[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kv = min(key0 + 4 * kg + i, last);
            const uint2 w = *reinterpret_cast<const uint2*>(vb + kv * rs + 4 * dq);
            p.b[2 * i] = w.x;
            p.b[2 * i + 1] = w.y;
        }
    }
}

__device__ __forceinline__ void store_tile(const AttnArgs& A, int t, int nc, int kend, int tid, Prefetch& p,
                                           uint16_t* Ks, uint16_t* Vt) {
    const int krow = tid >> 3, kpart = tid & 7;
    const int kg = tid & 15, dq = tid >> 4;
    uint4* kdst = reinterpret_cast<uint4*>(Ks + krow * KSTR + 16 * kpart);
    const int col = vperm(4 * kg);
    if (t < nc) {
        // K: 16 codes * scale -> bf16
        const float s = p.sc[0];
        const uint32_t w[4] = {p.a[0].x, p.a[0].y, p.a[0].z, p.a[0].w};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = pack_bf16(i8(w[i], 0) * s, i8(w[i], 1) * s);
            o[2 * i + 1] = pack_bf16(i8(w[i], 2) * s, i8(w[i], 3) * s);
        }
        kdst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        kdst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        // V: 4 keys x 4 channels, transposed: one 4-key run per channel
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float x0 = i8(p.b[0], d) * p.sc[1], x1 = i8(p.b[1], d) * p.sc[2];
            const float x2 = i8(p.b[2], d) * p.sc[3], x3 = i8(p.b[3], d) * p.sc[4];
            *reinterpret_cast<uint2*>(Vt + (4 * dq + d) * VSTR + col) = make_uint2(pack_bf16(x0, x1), pack_bf16(x2, x3));
        }
    } else {
        const int key = min((t - nc) * BN + krow, kend - 1);
        int tt, h, w;
        bool vid;
        if (A.segs.n == 1) {
            const int loc = key - A.segs.s[0].n_text;
            vid = loc >= 0;
            if (vid) video_pos(A.segs.s[0], loc, tt, h, w);
        } else {
            vid = token_pos(A.segs, key, tt, h, w);
        }
        if (vid) {
            p.a[0] = rope_group_f32(p.a[0], 2 * kpart, tt, h, w, A.rt);
            p.a[1] = rope_group_f32(p.a[1], 2 * kpart + 1, tt, h, w, A.rt);
        }
        kdst[0] = p.a[0];
        kdst[1] = p.a[1];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int wi = d >> 1;
            const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t p01 = __builtin_amdgcn_perm(p.b[2 + wi], p.b[wi], sel);
            const uint32_t p23 = __builtin_amdgcn_perm(p.b[6 + wi], p.b[4 + wi], sel);
            *reinterpret_cast<uint2*>(Vt + (4 * dq + d) * VSTR + col) = make_uint2(p01, p23);
        }
    }
}

// One 64-key tile for the 32 query rows of this wave: S^T = K.Q^T, online
// softmax, O^T += V^T.P^T.  MASK: keys at or beyond `lim` are excluded.
template <bool MASK>
__device__ __forceinline__ void tile_step(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                          const bf16x8 (&qf)[8], f32x16 (&o)[4], float& m, float& lsum,
                                          float c, int lim, int g, int l32) {
    f32x16 s[2];
    const f32x16 zero = {};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const uint16_t* kr = K + (32 * kb + l32) * KSTR + 8 * g;
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kr), qf[0], zero, 0, 0, 0);
#pragma unroll
        for (int kk = 1; kk < 8; ++kk)
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kr + 16 * kk), qf[kk],
                                                            s[kb], 0, 0, 0);
    }
    if (MASK) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (32 * kb + 8 * (r >> 2) + 4 * g + (r & 3) >= lim) s[kb][r] = -INFINITY;
    }
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
    mx = half_max(mx);
    const float mn = mx * c;
    if (__any(mn > m + 8.0f)) {
        const float mnew = fmaxf(m, mn);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m = mnew;
    }
    const float nm = -m;
    bf16x8 pb[4];
    const nm_bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        uint32_t pk[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, nm));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], c, nm));
            pk[r >> 1] = pack_bf16(p0, p1);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(nm_bf16x2, pk[r >> 1]), ones, lsum, false);
        }
        pb[2 * kb] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
        pb[2 * kb + 1] = __builtin_bit_cast(bf16x8, u32x4{pk[4], pk[5], pk[6], pk[7]});
    }
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(V + (32 * db + l32) * VSTR + 16 * ch + 8 * g);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ch], o[db], 0, 0, 0);
        }
    }
}

__global__ __launch_bounds__(NT) void seg_attn_kernel(const AttnArgs A) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VSTR];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int head = blockIdx.x / A.ntq;
    const int qt = blockIdx.x - head * A.ntq;

    int a = 0;
    while (a + 1 < A.segs.n && A.tile0[a + 1] <= qt) ++a;
    const SegDev& sg = A.segs.s[a];
    const int seg_end = sg.start + sg.n_text + sg.T * sg.Hg * sg.Wg;
    const int r0 = sg.start + (qt - A.tile0[a]) * BM;
    const int r1 = min(r0 + BM, seg_end);
    const int kend = seg_end;                 // new keys [0, kend) are allowed
    const float c = A.scale_log2;

    // ---- Q fragments with RoPE: lane holds query row l32 of this wave,
    //      channels 16kk + 8g .. +8 (the B operand of S^T = K.Q^T)
    bf16x8 qf[8];
    {
        // rows past the tile's end read the last row (never stored)
        const int row = min(r0 + wave * QW + l32, r1 - 1);
        int t = 0, h = 0, w = 0;
        const bool vid = token_pos(A.segs, row, t, h, w);
        const uint4* src = reinterpret_cast<const uint4*>(A.q + ((int64_t)row * A.H + head) * D);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            uint4 x = src[2 * kk + g];
            if (vid) x = rope_group_f32(x, 2 * kk + g, t, h, w, A.rt);
            qf[kk] = __builtin_bit_cast(bf16x8, u32x4{x.x, x.y, x.z, x.w});
        }
    }

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float m = -INFINITY, lsum = 0.0f;

    const int nc = (A.Lc + BN - 1) / BN;
    const int nt = nc + (kend + BN - 1) / BN;

    // Prefetch registers always hold the next tile to be written to LDS.  Loads
    // are unconditional (tile indices clamped to the last tile, a harmless
    // reload) and sit in straight-line code, so no wait for them is needed
    // before their consumer one iteration later.
    Prefetch pf;
    load_tile(A, head, 0, nc, kend, tid, pf);
    store_tile(A, 0, nc, kend, tid, pf, Ks[0], Vt[0]);
    load_tile(A, head, min(1, nt - 1), nc, kend, tid, pf);
    lds_barrier();

    auto step = [&](int j) {
        const int buf = j & 1;
        const int lim = (j < nc) ? min(BN, A.Lc - j * BN) : min(BN, kend - (j - nc) * BN);
        if (lim == BN) tile_step<false>(Ks[buf], Vt[buf], qf, o, m, lsum, c, lim, g, l32);
        else tile_step<true>(Ks[buf], Vt[buf], qf, o, m, lsum, c, lim, g, l32);
    };
    auto refill = [&](int j) {
        // tile j+1 into the buffer tile j-1 used (every wave is past it), then
        // request tile j+2; in the last iteration this rewrites an unused buffer
        const int buf = j & 1;
        store_tile(A, min(j + 1, nt - 1), nc, kend, tid, pf, Ks[buf ^ 1], Vt[buf ^ 1]);
        load_tile(A, head, min(j + 2, nt - 1), nc, kend, tid, pf);
    };
    // Odd waves refill before their tile math, even waves after it, so the two
    // waves sharing a SIMD alternate between MFMA and VALU work.
    if (wave & 1) {
        for (int j = 0; j < nt; ++j) {
            refill(j);
            step(j);
            lds_barrier();
        }
    } else {
        for (int j = 0; j < nt; ++j) {
            step(j);
            refill(j);
            lds_barrier();
        }
    }

    // ---- epilogue: O / l -> bf16; lse = (m + log2 l) ln 2
    const float lt = half_sum(lsum);
    const float inv = 1.0f / lt;
    const int row = r0 + wave * QW + l32;
    if (row < r1) {
        uint16_t* dst = A.out + ((int64_t)row * A.H + head) * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint2*>(dst + 32 * db + 8 * i + 4 * g) =
                    make_uint2(pack_bf16(o[db][4 * i] * inv, o[db][4 * i + 1] * inv),
                               pack_bf16(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv));
        if (A.lse && g == 0) A.lse[(int64_t)head * A.Ln + row] = (m + __log2f(lt)) * 0.69314718055994531f;
    }
}

int launch_seg_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const SegTable& segs,
                    int Ln, const int8_t* kc, const int8_t* vc, const float* ks, const float* vs,
                    int64_t cap, int Lc, int H, float sm_scale, uint16_t* out, float* lse,
                    const RopeTables& rt, hipStream_t stream) {
    AttnArgs A{};
    A.q = q; A.k = k; A.v = v;
    A.kc = kc; A.vc = vc; A.ks = ks; A.vs = vs;
    A.out = out; A.lse = lse;
    A.cap = cap; A.Lc = Lc; A.Ln = Ln; A.H = H;
    A.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
    int nt = 0;
    for (int i = 0; i < segs.n; ++i) {
        A.tile0[i] = nt;
        const SegDev& s = segs.s[i];
        const int ntok = s.n_text + s.T * s.Hg * s.Wg;
        nt += (ntok + BM - 1) / BM;
    }
    A.tile0[segs.n] = nt;
    A.ntq = nt;
    A.segs = segs;
    A.rt = rt;
    if (nt == 0) return NOMAS_OK;
    const int64_t blocks = (int64_t)nt * H;
    hipLaunchKernelGGL(seg_attn_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, A);
    return hipGetLastError() == hipSuccess ? NOMAS_OK : NOMAS_EHIP;
}

}  // namespace nomas
