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
constexpr int NW = 4;               // waves per workgroup
constexpr int QW = 64;              // query rows per wave
constexpr int BM = NW * QW;         // query rows per workgroup
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

// Registers that carry the next key tile from HBM to LDS.
struct Prefetch {
    uint4 a[4];     // K: cache 2 x 16 codes; new 4 x 8 bf16
    uint4 b[4];     // V: cache 4 keys x 8 codes (in .x/.y of b[0..1] pairs); new 4 keys x 8 bf16
    float sc[5];    // cache scales: K of this thread's row, V of its 4 keys
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

__device__ __forceinline__ void load_cache_tile(const AttnArgs& A, int head, int key0, int tid, Prefetch& p) {
    const int64_t hb = (int64_t)head * A.cap;
    {
        const int krow = tid >> 2, kpart = tid & 3;
        const int key = key0 + krow;
        if (key < A.Lc) {
            const uint4* src = reinterpret_cast<const uint4*>(A.kc + (hb + key) * D + 32 * kpart);
            p.a[0] = src[0];
            p.a[1] = src[1];
            p.sc[0] = A.ks[hb + key];
        } else {
            p.a[0] = p.a[1] = make_uint4(0, 0, 0, 0);
            p.sc[0] = 0.0f;
        }
    }
    {
        const int kg = tid & 15, dg = tid >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = key0 + 4 * kg + i;
            uint2 w = make_uint2(0, 0);
            float s = 0.0f;
            if (key < A.Lc) {
                w = *reinterpret_cast<const uint2*>(A.vc + (hb + key) * D + 8 * dg);
                s = A.vs[hb + key];
            }
            if (i & 1) { p.b[i >> 1].z = w.x; p.b[i >> 1].w = w.y; }
            else { p.b[i >> 1].x = w.x; p.b[i >> 1].y = w.y; }
            p.sc[1 + i] = s;
        }
    }
}

__device__ __forceinline__ void store_cache_tile(const Prefetch& p, uint16_t* Ks, uint16_t* Vt, int tid) {
    {
        const int krow = tid >> 2, kpart = tid & 3;
        const float s = p.sc[0];
        uint32_t wv[8] = {p.a[0].x, p.a[0].y, p.a[0].z, p.a[0].w, p.a[1].x, p.a[1].y, p.a[1].z, p.a[1].w};
        uint32_t o[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            o[2 * i] = pack_bf16(i8(wv[i], 0) * s, i8(wv[i], 1) * s);
            o[2 * i + 1] = pack_bf16(i8(wv[i], 2) * s, i8(wv[i], 3) * s);
        }
        uint4* dst = reinterpret_cast<uint4*>(Ks + krow * KSTR + 32 * kpart);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    }
    {
        const int kg = tid & 15, dg = tid >> 4;
        // key i's 8 codes: lo word / hi word
        uint32_t lo[4] = {p.b[0].x, p.b[0].z, p.b[1].x, p.b[1].z};
        uint32_t hi[4] = {p.b[0].y, p.b[0].w, p.b[1].y, p.b[1].w};
        const int col = vperm(4 * kg);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = i8(d < 4 ? lo[i] : hi[i], d & 3) * p.sc[1 + i];
            *reinterpret_cast<uint2*>(Vt + (8 * dg + d) * VSTR + col) =
                make_uint2(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]));
        }
    }
}

__device__ __forceinline__ void load_new_tile(const AttnArgs& A, int head, int key0, int kend, int tid, Prefetch& p) {
    {
        const int krow = tid >> 2, kpart = tid & 3;
        const int key = key0 + krow;
        if (key < kend) {
            const uint4* src = reinterpret_cast<const uint4*>(A.k + ((int64_t)key * A.H + head) * D + 32 * kpart);
#pragma unroll
            for (int i = 0; i < 4; ++i) p.a[i] = src[i];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) p.a[i] = make_uint4(0, 0, 0, 0);
        }
    }
    {
        const int kg = tid & 15, dg = tid >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = key0 + 4 * kg + i;
            p.b[i] = (key < kend)
                         ? *reinterpret_cast<const uint4*>(A.v + ((int64_t)key * A.H + head) * D + 8 * dg)
                         : make_uint4(0, 0, 0, 0);
        }
    }
}

__device__ __forceinline__ void store_new_tile(const AttnArgs& A, Prefetch& p, int key0, int kend,
                                               uint16_t* Ks, uint16_t* Vt, int tid) {
    {
        const int krow = tid >> 2, kpart = tid & 3;
        const int key = key0 + krow;
        int t, h, w;
        if (key < kend && token_pos(A.segs, key, t, h, w)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) p.a[i] = rope_group_f32(p.a[i], 4 * kpart + i, t, h, w, A.rt);
        }
        uint4* dst = reinterpret_cast<uint4*>(Ks + krow * KSTR + 32 * kpart);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = p.a[i];
    }
    {
        const int kg = tid & 15, dg = tid >> 4;
        const int col = vperm(4 * kg);
        uint32_t wv[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) { wv[i][0] = p.b[i].x; wv[i][1] = p.b[i].y; wv[i][2] = p.b[i].z; wv[i][3] = p.b[i].w; }
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const int c = d >> 1;
            const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
            uint32_t p01 = __builtin_amdgcn_perm(wv[1][c], wv[0][c], sel);
            uint32_t p23 = __builtin_amdgcn_perm(wv[3][c], wv[2][c], sel);
            *reinterpret_cast<uint2*>(Vt + (8 * dg + d) * VSTR + col) = make_uint2(p01, p23);
        }
    }
}

__global__ __launch_bounds__(256, 1) void seg_attn_kernel(const AttnArgs A) {
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

    // ---- Q fragments with RoPE: lane holds query (l32) and channels 16kk+8g..+8
    bf16x8 qf[2][8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int row = r0 + wave * QW + qb * 32 + l32;
        int t = 0, h = 0, w = 0;
        const bool valid = row < r1;
        const bool vid = valid && token_pos(A.segs, row, t, h, w);
        const uint4* src = reinterpret_cast<const uint4*>(A.q + ((int64_t)row * A.H + head) * D);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            uint4 x = valid ? src[2 * kk + g] : make_uint4(0, 0, 0, 0);
            if (vid) x = rope_group_f32(x, 2 * kk + g, t, h, w, A.rt);
            qf[qb][kk] = __builtin_bit_cast(bf16x8, u32x4{x.x, x.y, x.z, x.w});
        }
    }

    f32x16 o[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.0f;
    float m[2] = {-INFINITY, -INFINITY};
    float lsum[2] = {0.0f, 0.0f};

    const int nc = (A.Lc + BN - 1) / BN;
    const int nt = nc + (kend + BN - 1) / BN;

    Prefetch pf;
    if (nc > 0) { load_cache_tile(A, head, 0, tid, pf); store_cache_tile(pf, Ks[0], Vt[0], tid); }
    else { load_new_tile(A, head, 0, kend, tid, pf); store_new_tile(A, pf, 0, kend, Ks[0], Vt[0], tid); }
    __syncthreads();

    for (int j = 0; j < nt; ++j) {
        const int buf = j & 1;
        const int jn = j + 1;
        if (jn < nt) {
            if (jn < nc) load_cache_tile(A, head, jn * BN, tid, pf);
            else load_new_tile(A, head, (jn - nc) * BN, kend, tid, pf);
        }
        const int lim = (j < nc) ? min(BN, A.Lc - j * BN) : min(BN, kend - (j - nc) * BN);

        // ---- S^T = K . Q^T
        const uint16_t* K = Ks[buf];
        f32x16 s[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(K + (32 * kb + l32) * KSTR + 16 * kk + 8 * g);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qb][kk], s[kb][qb], 0, 0, 0);
            }
        }
        if (lim < BN) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (key >= lim) { s[kb][0][r] = -INFINITY; s[kb][1][r] = -INFINITY; }
                }
        }

        // ---- online softmax (base 2), P packed to bf16 in the B-operand layout
        bf16x8 pb[2][4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mn = mx * c;
            if (__any(mn > m[qb] + 8.0f)) {
                const float mnew = fmaxf(m[qb], mn);
                const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
                lsum[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
                m[qb] = mnew;
            }
            const float nm = -m[qb];
            float acc = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                uint32_t pk[8];
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r], c, nm));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r + 1], c, nm));
                    acc += p0 + p1;
                    pk[r >> 1] = pack_bf16(p0, p1);
                }
                pb[qb][2 * kb] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
                pb[qb][2 * kb + 1] = __builtin_bit_cast(bf16x8, u32x4{pk[4], pk[5], pk[6], pk[7]});
            }
            lsum[qb] += acc;
        }

        // ---- O^T += V^T . P^T
        const uint16_t* V = Vt[buf];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const bf16x8 va = *reinterpret_cast<const bf16x8*>(V + (32 * db + l32) * VSTR + 16 * ch + 8 * g);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qb][ch], o[qb][db], 0, 0, 0);
            }
        }

        if (jn < nt) {
            if (jn < nc) store_cache_tile(pf, Ks[buf ^ 1], Vt[buf ^ 1], tid);
            else store_new_tile(A, pf, (jn - nc) * BN, kend, Ks[buf ^ 1], Vt[buf ^ 1], tid);
        }
        __syncthreads();
    }

    // ---- epilogue: O / l -> bf16; lse = (m + log2 l) ln 2
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = lsum[qb] + __shfl_xor(lsum[qb], 32);
        const float inv = 1.0f / lt;
        const int row = r0 + wave * QW + qb * 32 + l32;
        if (row < r1) {
            uint16_t* dst = A.out + ((int64_t)row * A.H + head) * D;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int d0 = 32 * db + 8 * i + 4 * g;
                    const f32x16& ov = o[qb][db];
                    *reinterpret_cast<uint2*>(dst + d0) =
                        make_uint2(pack_bf16(ov[4 * i] * inv, ov[4 * i + 1] * inv),
                                   pack_bf16(ov[4 * i + 2] * inv, ov[4 * i + 3] * inv));
                }
            if (A.lse && g == 0) A.lse[(int64_t)head * A.Ln + row] = (m[qb] + __log2f(lt)) * 0.69314718055994531f;
        }
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
    hipLaunchKernelGGL(seg_attn_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, A);
    return hipGetLastError() == hipSuccess ? NOMAS_OK : NOMAS_EHIP;
}

}  // namespace nomas
