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

// This thread's share of one key tile on its way from HBM to LDS.  Both
// kinds of tile fill all four registers, so the two load paths join without
// copies:
//   K: key row tid/8, channels 16*(tid%8) .. +16
//   V: keys 4*(tid%16) .. +4, channels 4*(tid/16) .. +4
//   cache tile: a0 = 16 K codes, a1.x = K scale, b0 = 4 keys x 4 V codes,
//               b1 = the 4 V scales
//   new tile:   a0, a1 = 16 K values (bf16), b0, b1 = 4 keys x 4 V values
struct Prefetch {
    uint4 a0, a1, b0, b1;
};

// Buffer descriptors of the key/value ranges one workgroup may read.  Each
// covers exactly the allowed keys, so a read past them returns zeros: tail
// keys of the last tile come back as zero vectors (their scores are masked)
// and tokens of later segments are never read.
struct Bufs {
    __amdgpu_buffer_rsrc_t kc, vc, ks, vs, k, v;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// position (in the permuted V^T row) of key k, k a multiple of 4 inside a tile
__device__ __forceinline__ int vperm(int k) {
    int w = k & 15;
    int p = (w == 4) ? 8 : (w == 8) ? 4 : w;
    return (k & ~15) + p;
}

__device__ __forceinline__ float i8(uint32_t word, int byte) {
    return (float)(int8_t)(word >> (8 * byte));
}

// Which keys a tile holds.  Full tiles come first (cache, then new keys),
// the at most two partial tiles (cache tail, new-key tail) last.
struct TileRef {
    bool cache;
    int key0, lim;      // first key, number of valid keys
};

__device__ __forceinline__ TileRef tile_at(int j, int Lc, int kend) {
    const int ncf = Lc / BN, nnf = kend / BN;
    if (j < ncf) return {true, j * BN, BN};
    if (j < ncf + nnf) return {false, (j - ncf) * BN, BN};
    if (j == ncf + nnf && Lc % BN) return {true, ncf * BN, Lc - ncf * BN};
    return {false, nnf * BN, kend - nnf * BN};
}

__device__ __forceinline__ void load_tile(const Bufs& B, const TileRef& T, uint32_t rs, int tid, Prefetch& p) {
    const uint32_t krow = tid >> 3, kpart = tid & 7;
    const uint32_t kg = tid & 15, dq = tid >> 4;
    if (T.cache) {
        const uint32_t key = T.key0 + krow;
        const uint32_t kv = T.key0 + 4 * kg;
        p.a0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(B.kc, key * D + 16 * kpart, 0, 0));
        p.a1 = make_uint4(__builtin_amdgcn_raw_buffer_load_b32(B.ks, 4 * key, 0, 0), 0u, 0u, 0u);
        const uint32_t vo = kv * D + 4 * dq;
        p.b0 = make_uint4(__builtin_amdgcn_raw_buffer_load_b32(B.vc, vo, 0, 0),
                          __builtin_amdgcn_raw_buffer_load_b32(B.vc, vo + D, 0, 0),
                          __builtin_amdgcn_raw_buffer_load_b32(B.vc, vo + 2 * D, 0, 0),
                          __builtin_amdgcn_raw_buffer_load_b32(B.vc, vo + 3 * D, 0, 0));
        p.b1 = make_uint4(__builtin_amdgcn_raw_buffer_load_b32(B.vs, 4 * kv, 0, 0),
                          __builtin_amdgcn_raw_buffer_load_b32(B.vs, 4 * kv + 4, 0, 0),
                          __builtin_amdgcn_raw_buffer_load_b32(B.vs, 4 * kv + 8, 0, 0),
                          __builtin_amdgcn_raw_buffer_load_b32(B.vs, 4 * kv + 12, 0, 0));
    } else {
        const uint32_t key = T.key0 + krow;
        const uint32_t kv = T.key0 + 4 * kg;
        const uint32_t ko = key * rs + 32 * kpart;
        p.a0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(B.k, ko, 0, 0));
        p.a1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(B.k, ko + 16, 0, 0));
        const uint32_t vo = kv * rs + 8 * dq;
        const auto v0 = __builtin_amdgcn_raw_buffer_load_b64(B.v, vo, 0, 0);
        const auto v1 = __builtin_amdgcn_raw_buffer_load_b64(B.v, vo + rs, 0, 0);
        const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(B.v, vo + 2 * rs, 0, 0);
        const auto v3 = __builtin_amdgcn_raw_buffer_load_b64(B.v, vo + 3 * rs, 0, 0);
        p.b0 = make_uint4(v0[0], v0[1], v1[0], v1[1]);
        p.b1 = make_uint4(v2[0], v2[1], v3[0], v3[1]);
    }
}

__device__ __forceinline__ void store_tile(const AttnArgs& A, const TileRef& T, int kend, int tid, Prefetch& p,
                                           uint16_t* Ks, uint16_t* Vt) {
    const int krow = tid >> 3, kpart = tid & 7;
    const int kg = tid & 15, dq = tid >> 4;
    uint4* kdst = reinterpret_cast<uint4*>(Ks + krow * KSTR + 16 * kpart);
    const int col = vperm(4 * kg);
    if (T.cache) {
        // K: 16 codes * scale -> bf16
        const float s = __uint_as_float(p.a1.x);
        const uint32_t w[4] = {p.a0.x, p.a0.y, p.a0.z, p.a0.w};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = pack_bf16(i8(w[i], 0) * s, i8(w[i], 1) * s);
            o[2 * i + 1] = pack_bf16(i8(w[i], 2) * s, i8(w[i], 3) * s);
        }
        kdst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        kdst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        // V: 4 keys x 4 channels, transposed: one 4-key run per channel
        const float s0 = __uint_as_float(p.b1.x), s1 = __uint_as_float(p.b1.y);
        const float s2 = __uint_as_float(p.b1.z), s3 = __uint_as_float(p.b1.w);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float x0 = i8(p.b0.x, d) * s0, x1 = i8(p.b0.y, d) * s1;
            const float x2 = i8(p.b0.z, d) * s2, x3 = i8(p.b0.w, d) * s3;
            *reinterpret_cast<uint2*>(Vt + (4 * dq + d) * VSTR + col) = make_uint2(pack_bf16(x0, x1), pack_bf16(x2, x3));
        }
    } else {
        // K rows past the allowed range read as zeros and stay zero (no rotation)
        const int key = T.key0 + krow;
        int tt, h, w;
        bool vid;
        if (A.segs.n == 1) {
            const int loc = key - A.segs.s[0].n_text;
            vid = loc >= 0 && key < kend;
            if (vid) video_pos(A.segs.s[0], loc, tt, h, w);
        } else {
            vid = key < kend && token_pos(A.segs, key, tt, h, w);
        }
        if (vid) {
            p.a0 = rope_group_f32(p.a0, 2 * kpart, tt, h, w, A.rt);
            p.a1 = rope_group_f32(p.a1, 2 * kpart + 1, tt, h, w, A.rt);
        }
        kdst[0] = p.a0;
        kdst[1] = p.a1;
        // V: word j of key i holds channels 4dq + 2j, +1
        const uint32_t wv[4][2] = {{p.b0.x, p.b0.y}, {p.b0.z, p.b0.w}, {p.b1.x, p.b1.y}, {p.b1.z, p.b1.w}};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int wi = d >> 1;
            const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t p01 = __builtin_amdgcn_perm(wv[1][wi], wv[0][wi], sel);
            const uint32_t p23 = __builtin_amdgcn_perm(wv[3][wi], wv[2][wi], sel);
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
    // keep several K fragments in flight ahead of the MFMAs that use them
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);       // 6 LDS reads
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
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
    const int head = __builtin_amdgcn_readfirstlane(blockIdx.x / A.ntq);
    const int qt = __builtin_amdgcn_readfirstlane(blockIdx.x - head * A.ntq);

    int a = 0;
    while (a + 1 < A.segs.n && A.tile0[a + 1] <= qt) ++a;
    const SegDev& sg = A.segs.s[a];
    // workgroup-uniform values, kept in scalar registers so that tile choices
    // are scalar branches and tile bases are scalar addresses
    const int seg_end = __builtin_amdgcn_readfirstlane(sg.start + sg.n_text + sg.T * sg.Hg * sg.Wg);
    const int r0 = __builtin_amdgcn_readfirstlane(sg.start + (qt - A.tile0[a]) * BM);
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

    const int nc = __builtin_amdgcn_readfirstlane((A.Lc + BN - 1) / BN);
    const int nt = __builtin_amdgcn_readfirstlane(nc + (kend + BN - 1) / BN);

    Bufs B;
    {
        const size_t hb = (size_t)head * A.cap;
        B.kc = make_rsrc(A.kc + hb * D, (uint32_t)A.Lc * D);
        B.vc = make_rsrc(A.vc + hb * D, (uint32_t)A.Lc * D);
        B.ks = make_rsrc(A.ks + hb, (uint32_t)A.Lc * 4);
        B.vs = make_rsrc(A.vs + hb, (uint32_t)A.Lc * 4);
        // new tokens [0, kend) of this head: rows of H*128 bf16, this head's 128 at the front
        const uint32_t bytes = (uint32_t)(kend - 1) * (uint32_t)A.H * D * 2 + D * 2;
        B.k = make_rsrc(A.k + head * D, bytes);
        B.v = make_rsrc(A.v + head * D, bytes);
    }
    const uint32_t rs = (uint32_t)A.H * D * 2;      // bytes per new-token row

    // Prefetch registers always hold the next tile to be written to LDS.  Loads
    // are unconditional (tile indices clamped to the last tile, a harmless
    // reload) and sit in straight-line code, so no wait for them is needed
    // before their consumer one iteration later.
    const int nfull = __builtin_amdgcn_readfirstlane(A.Lc / BN + kend / BN);
    Prefetch pf;
    load_tile(B, tile_at(0, A.Lc, kend), rs, tid, pf);
    store_tile(A, tile_at(0, A.Lc, kend), kend, tid, pf, Ks[0], Vt[0]);
    load_tile(B, tile_at(min(1, nt - 1), A.Lc, kend), rs, tid, pf);
    lds_barrier();

    auto refill = [&](int j) {
        // tile j+1 into the buffer tile j-1 used (every wave is past it), then
        // request tile j+2; in the last iteration this rewrites an unused buffer
        const int buf = j & 1;
        store_tile(A, tile_at(min(j + 1, nt - 1), A.Lc, kend), kend, tid, pf, Ks[buf ^ 1], Vt[buf ^ 1]);
        load_tile(B, tile_at(min(j + 2, nt - 1), A.Lc, kend), rs, tid, pf);
    };
    // Odd waves refill before their tile math, even waves after it, so the two
    // waves sharing a SIMD alternate between MFMA and VALU work.  Full tiles
    // run without any masking; the partial tiles come last, in a loop of
    // their own.
    if (wave & 1) {
        for (int j = 0; j < nfull; ++j) {
            refill(j);
            tile_step<false>(Ks[j & 1], Vt[j & 1], qf, o, m, lsum, c, BN, g, l32);
            lds_barrier();
        }
    } else {
        for (int j = 0; j < nfull; ++j) {
            tile_step<false>(Ks[j & 1], Vt[j & 1], qf, o, m, lsum, c, BN, g, l32);
            refill(j);
            lds_barrier();
        }
    }
    for (int j = nfull; j < nt; ++j) {
        const int lim = tile_at(j, A.Lc, kend).lim;
        tile_step<true>(Ks[j & 1], Vt[j & 1], qf, o, m, lsum, c, lim, g, l32);
        refill(j);
        lds_barrier();
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
