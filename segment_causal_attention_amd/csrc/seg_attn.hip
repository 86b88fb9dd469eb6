// Segment-causal joint attention over the lifelong INT8 KV cache plus the
// current segment(s), for gfx950.
//
// What it computes (comfyui-wiki news page on Hy-Nomas, section 一个世界，分段生成;
// huaweicloud blog, section 2.1): query i of new segment a attends to every
// cached token and to the new tokens of segments 0..a, never to a later
// segment.  Cached K/V are INT8 with one fp32 scale per (token, head); the
// attention itself runs in BF16 (comfyui-wiki, 单张 4090 配置): cached entries
// enter the products as bf16(fl32(code*scale)); queries are rotated by 3D
// RoPE (comfyui-wiki, 模型内部: [16, 56, 56], theta 256) on load and rounded
// to bf16; new keys arrive already rotated (the rows the cache append stores).
//
// Kernel shape.  One workgroup = 8 waves x 32 query rows = 256 rows of one
// head, all inside one new segment, so every row allows the same keys:
// the cache [0, Lc) and the new tokens [0, end of its segment).  Later
// segments are never loaded.  Keys stream through three LDS buffers in tiles
// of 64.  Tile j+2 is converted (cache: int8 * scale -> bf16; new keys: bf16
// copy, V transposed) once per workgroup while the waves work on tiles j and
// j+1, and each wave runs a software pipeline across tiles: the S^T products
// of tile j+1 issue between the softmax instructions of tile j, and the O^T
// products of tile j between the conversion instructions of tile j+2, so
// every wave always has independent vector work between its matrix
// instructions.  One LDS barrier per tile; HBM loads for tile j+3 are in
// flight across it.  V^T is stored [channel][key] so that both products
// read 16 contiguous bytes per lane.
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
#include <type_traits>

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
#ifndef PF_DIST
#define PF_DIST 4
#endif
constexpr int FD = PF_DIST;         // LDS fragment reads issued this many products ahead

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

// Which keys a tile holds.  Cache tiles come first, [0, nc), then the new
// keys' tiles; the last tile of each run may be partial.
struct TileRef {
    bool cache;
    int key0, lim;      // first key, number of valid keys
};

__device__ __forceinline__ TileRef tile_at(int j, int Lc, int nc, int kend) {
    if (j < nc) return {true, j * BN, min(BN, Lc - j * BN)};
    return {false, (j - nc) * BN, min(BN, kend - (j - nc) * BN)};
}

// What a stretch of steps knows about its tiles at compile time: all cache,
// all new keys, or either (a scalar branch per tile).  Each kind issues one
// fixed sequence of loads, so the wait before a conversion counts exactly
// the loads issued after it.
enum TileKind { KIND_CACHE = 0, KIND_NEW = 1, KIND_ANY = 2 };

template <int KIND>
__device__ __forceinline__ void load_tile(const Bufs& B, const TileRef& T, uint32_t rs, int tid, Prefetch& p) {
    const uint32_t krow = tid >> 3, kpart = tid & 7;
    const uint32_t kg = tid & 15, dq = tid >> 4;
    if (KIND == KIND_CACHE || (KIND == KIND_ANY && T.cache)) {
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

// Per-wave state carried across key tiles.
struct WaveState {
    bf16x8 qf[8];        // Q^T fragments (B operand): query l32, channels 16kk + 8g .. +8
    f32x16 o[4];         // O^T accumulators: channels 32db + 8i + 4g + j, query l32
    float m, lsum;       // running max (base 2, scaled) and partial row sum of this lane half
};

// Nothing is scheduled across this point: it pins the order of the slots of
// the pipelined loop body.
#define SLOT_FENCE() __builtin_amdgcn_sched_barrier(0)

// A operand of the i-th S^T product of a tile: key block i%2, channels 16(i/2)
__device__ __forceinline__ bf16x8 kfrag(const uint16_t* K, int krd, int i) {
    return *reinterpret_cast<const bf16x8*>(K + krd + 32 * (i & 1) * KSTR + 16 * (i >> 1));
}
// A operand of the i-th O^T product of a tile: channel block i%4, key chunk i/4
__device__ __forceinline__ bf16x8 vfrag(const uint16_t* V, int vrd, int i) {
    return *reinterpret_cast<const bf16x8*>(V + vrd + 32 * (i & 3) * VSTR + 16 * (i >> 2));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Scores of keys at or past lim (partial tiles) -> -inf.  Register r of block
// kb holds key 32kb + 8(r/4) + 4g + r%4.
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int lim, int g) {
    const int limg = lim - 4 * g;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (32 * kb + 8 * (r >> 2) + (r & 3) >= limg) s[kb][r] = -INFINITY;
            if ((r & 3) == 3) SLOT_FENCE();
        }
}

__device__ __forceinline__ float max_part(const f32x16 (&s)[2], int r0, int r1, float mx) {
#pragma unroll
    for (int r = r0; r < r1; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
    return mx;
}

// Row max of the tile (both lane halves) against the running max; O and the
// sum are rescaled only when the max grows by more than 8 (a factor 256).
__device__ __forceinline__ void update_max(float mx, WaveState& w, float c) {
    mx = half_max(mx);
    const float mn = mx * c;
    if (__any(mn > w.m + 8.0f)) {
        const float mnew = fmaxf(w.m, mn);
        const float alpha = __builtin_amdgcn_exp2f(w.m - mnew);
        w.lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) w.o[db][r] *= alpha;
        w.m = mnew;
    }
}

// Probability pair q (0..15) of the tile: keys of registers 2(q%8), +1 of
// block q/8, exp2(s c - m) rounded to bf16 and packed; the row sum is taken
// over the same bf16 values.  Words 4ch .. 4ch+3 form the B operand of key
// chunk ch of the O^T product.
__device__ __forceinline__ void prob_pair(const f32x16 (&s)[2], int q, WaveState& w, float c, uint32_t (&pk)[16]) {
    const nm_bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    const int kb = q >> 3, r = 2 * (q & 7);
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -w.m));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], c, -w.m));
    pk[q] = pack_bf16(p0, p1);
    w.lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(nm_bf16x2, pk[q]), ones, w.lsum, false);
}

__device__ __forceinline__ bf16x8 pchunk(const uint32_t (&pk)[16], int ch) {
    return __builtin_bit_cast(bf16x8, u32x4{pk[4 * ch], pk[4 * ch + 1], pk[4 * ch + 2], pk[4 * ch + 3]});
}

// ---------------------------------------------------------------------------
// HBM tile -> LDS tile, in units small enough to sit between two matrix
// instructions.  Thread tid writes K row tid/8, channels 16(tid%8) .. +16 and
// V^T channels 4(tid/16) .. +4 at keys 4(tid%16) .. +4.

struct StoreDst {
    uint4* k;            // K row tid/8, channels 16(tid%8)
    uint16_t* v;         // V^T row 4(tid/16), permuted column of key 4(tid%16)
};

__device__ __forceinline__ StoreDst store_dst(uint16_t* Ks, uint16_t* Vt, int tid) {
    return {reinterpret_cast<uint4*>(Ks + (tid >> 3) * KSTR + 16 * (tid & 7)), Vt + 4 * (tid >> 4) * VSTR + vperm(4 * (tid & 15))};
}

// cache tile, K: word u (4 codes) of the 16, times the key's scale; the two
// 16-byte halves are written after words 1 and 3
__device__ __forceinline__ void cache_k_unit(int u, const Prefetch& p, uint32_t (&o)[4], const StoreDst& d) {
    const float s = __uint_as_float(p.a1.x);
    const uint32_t w = u == 0 ? p.a0.x : u == 1 ? p.a0.y : u == 2 ? p.a0.z : p.a0.w;
    o[2 * (u & 1)] = pack_bf16(i8(w, 0) * s, i8(w, 1) * s);
    o[2 * (u & 1) + 1] = pack_bf16(i8(w, 2) * s, i8(w, 3) * s);
    if (u & 1) d.k[u >> 1] = make_uint4(o[0], o[1], o[2], o[3]);
}

// cache tile, V: channel dq of the thread's 4, over its 4 keys
__device__ __forceinline__ void cache_v_unit(int dq, const Prefetch& p, const StoreDst& d) {
    const float x0 = i8(p.b0.x, dq) * __uint_as_float(p.b1.x), x1 = i8(p.b0.y, dq) * __uint_as_float(p.b1.y);
    const float x2 = i8(p.b0.z, dq) * __uint_as_float(p.b1.z), x3 = i8(p.b0.w, dq) * __uint_as_float(p.b1.w);
    *reinterpret_cast<uint2*>(d.v + dq * VSTR) = make_uint2(pack_bf16(x0, x1), pack_bf16(x2, x3));
}

// new-key tile, V: word pairs of the 4 keys regrouped per channel
__device__ __forceinline__ void new_v_unit(int dq, const Prefetch& p, const StoreDst& d) {
    const uint32_t sel = (dq & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t w0 = (dq >> 1) ? p.b0.y : p.b0.x, w1 = (dq >> 1) ? p.b0.w : p.b0.z;
    const uint32_t w2 = (dq >> 1) ? p.b1.y : p.b1.x, w3 = (dq >> 1) ? p.b1.w : p.b1.z;
    *reinterpret_cast<uint2*>(d.v + dq * VSTR) =
        make_uint2(__builtin_amdgcn_perm(w1, w0, sel), __builtin_amdgcn_perm(w3, w2, sel));
}

// new-key tile, K: the 16 rotated bf16 values copied as they are
__device__ __forceinline__ void new_k_unit(int half, const Prefetch& p, const StoreDst& d) {
    d.k[half] = half ? p.a1 : p.a0;
}

// Whole-tile store, unscheduled (prologue).
__device__ __forceinline__ void store_tile(const TileRef& T, int tid, const Prefetch& p, uint16_t* Ks, uint16_t* Vt) {
    const StoreDst d = store_dst(Ks, Vt, tid);
    if (T.cache) {
        uint32_t o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) cache_k_unit(u, p, o, d);
#pragma unroll
        for (int dq = 0; dq < 4; ++dq) cache_v_unit(dq, p, d);
    } else {
        new_k_unit(0, p, d);
        new_k_unit(1, p, d);
#pragma unroll
        for (int dq = 0; dq < 4; ++dq) new_v_unit(dq, p, d);
    }
}

// ---------------------------------------------------------------------------
// The pipelined step j.  The S^T products of tile j+1 (K from LDS) run
// interleaved with the row max and probabilities of tile j; then the O^T
// products of tile j run interleaved with the conversion of tile j+2 (HBM
// data already in registers) into the third LDS buffer.  Every slot holds
// one matrix instruction, the LDS read of the operand two slots ahead and a
// short run of independent vector work, so each wave keeps issuing while its
// matrix instructions execute.

template <int KIND>
__device__ __forceinline__ void pipelined_step(const uint16_t* Kn, const uint16_t* V, uint16_t* K2, uint16_t* V2,
                                               bool cache2, int lim, int tid, int krd, int vrd, const Prefetch& pf,
                                               WaveState& w, f32x16 (&s)[2], f32x16 (&sn)[2], float c, int g) {
    if (KIND != KIND_ANY) cache2 = KIND == KIND_CACHE;
    if (lim < BN) mask_tile(s, lim, g);
    uint32_t pk[16];
    {
        const f32x16 zero = {};
        bf16x8 kf[16];
#pragma unroll
        for (int i = 0; i < FD; ++i) kf[i] = kfrag(Kn, krd, i);
        SLOT_FENCE();
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + FD < 16) kf[i + FD] = kfrag(Kn, krd, i + FD);
            sn[i & 1] = mfma(kf[i], w.qf[i >> 1], i < 2 ? zero : sn[i & 1]);
            if (i == 0) mx = max_part(s, 0, 8, fmaxf(s[0][0], s[1][0]));
            else if (i == 1) mx = max_part(s, 8, 16, mx);
            else if (i == 2) update_max(mx, w, c);
            else prob_pair(s, i - 3, w, c, pk);
            SLOT_FENCE();
        }
    }
    // O^T products of tile j with the conversion of tile j+2; the tile kind
    // is a scalar branch inside each slot, so the accumulators never pass
    // through a join
    const StoreDst d = store_dst(K2, V2, tid);
    bf16x8 vf[16];
#pragma unroll
    for (int i = 0; i < FD; ++i) vf[i] = vfrag(V, vrd, i);
    SLOT_FENCE();
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (i + FD < 16) vf[i + FD] = vfrag(V, vrd, i + FD);
        w.o[i & 3] = mfma(vf[i], pchunk(pk, i >> 2), w.o[i & 3]);
        if (i < 3) {
            prob_pair(s, 13 + i, w, c, pk);
        } else if (i < 7) {
            if (cache2) cache_k_unit(i - 3, pf, o, d);
            else new_v_unit(i - 3, pf, d);
        } else if (i < 11) {
            if (cache2) cache_v_unit(i - 7, pf, d);
            else if (i < 9) new_k_unit(i - 7, pf, d);
        }
        SLOT_FENCE();
    }
}

__global__ __launch_bounds__(NT) void seg_attn_kernel(const AttnArgs A) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[3][BN * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[3][D * VSTR];

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
    WaveState ws;
    {
        // rows past the tile's end read the last row (never stored)
        const int row = min(r0 + wave * QW + l32, r1 - 1);
        int t = 0, h = 0, w = 0;
        if (!token_pos(A.segs, row, t, h, w)) t = h = w = 0;   // text: identity rotation
        const uint4* src = reinterpret_cast<const uint4*>(A.q + ((int64_t)row * A.H + head) * D);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const uint4 x = rope_group_f32(src[2 * kk + g], 2 * kk + g, t, h, w, A.rt);
            ws.qf[kk] = __builtin_bit_cast(bf16x8, u32x4{x.x, x.y, x.z, x.w});
        }
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) ws.o[db][r] = 0.0f;
    ws.m = -INFINITY;
    ws.lsum = 0.0f;

    const int nc = __builtin_amdgcn_readfirstlane((A.Lc + BN - 1) / BN);   // cache tiles
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
    const int krd = l32 * KSTR + 8 * g;             // this lane's K / V^T fragment offsets
    const int vrd = l32 * VSTR + 8 * g;

    // Three LDS buffers: step j reads K of tile j+1 and V of tile j and
    // writes tile j+2.  Two prefetch register sets alternate between steps:
    // the set converted in step j was loaded in step j-2, two steps ahead of
    // its use.  Loads are unconditional (tile indices clamped to the last
    // tile, a harmless reload) and straight-line.
    auto tile = [&](int j) { return tile_at(min(j, nt - 1), A.Lc, nc, kend); };
    Prefetch pa, pb;
    load_tile<KIND_ANY>(B, tile(0), rs, tid, pa);
    load_tile<KIND_ANY>(B, tile(1), rs, tid, pb);
    store_tile(tile(0), tid, pa, Ks[0], Vt[0]);
    load_tile<KIND_ANY>(B, tile(2), rs, tid, pa);
    store_tile(tile(1), tid, pb, Ks[1], Vt[1]);
    load_tile<KIND_ANY>(B, tile(3), rs, tid, pb);
    lds_barrier();

    f32x16 sa[2], sb[2];
    {
        const f32x16 zero = {};
#pragma unroll
        for (int i = 0; i < 16; ++i) sa[i & 1] = mfma(kfrag(Ks[0], krd, i), ws.qf[i >> 1], i < 2 ? zero : sa[i & 1]);
    }
    // Step j: scores of tile j in x, next tile's scores into y; LDS buffer b0
    // holds tile j; pf holds tile j+2 and is refilled with tile j+4.  Steps
    // past the last tile see a fully masked tile and change nothing.  Steps
    // go in pairs, so the score and prefetch sets swap roles without copies.
    auto step = [&](auto kind, int j, int b0, f32x16 (&x)[2], f32x16 (&y)[2], Prefetch& pf) {
        constexpr int K = decltype(kind)::value;
        const int b1 = b0 == 2 ? 0 : b0 + 1;
        const int b2 = b1 == 2 ? 0 : b1 + 1;
        const int lim = j < nt ? tile(j).lim : 0;
        pipelined_step<K>(Ks[b1], Vt[b0], Ks[b2], Vt[b2], tile(j + 2).cache, lim, tid, krd, vrd, pf, ws, x, y, c, g);
        load_tile<K>(B, tile(j + 4), rs, tid, pf);
        lds_barrier();
        return b1;
    };
    const std::integral_constant<int, KIND_CACHE> cache_kind;
    const std::integral_constant<int, KIND_NEW> new_kind;
    const std::integral_constant<int, KIND_ANY> any_kind;
    // all outstanding loads complete before a specialised stretch, so its
    // waits are counted from its own loads only
    const auto drain = [] { __builtin_amdgcn_s_waitcnt(0x0f70); };   // vmcnt(0)
    int j = 0, b = 0;
    if (j + 5 < nc) {
        drain();
        for (; j + 5 < nc; j += 2) {          // tiles j .. j+5 all from the cache
            b = step(cache_kind, j, b, sa, sb, pa);
            b = step(cache_kind, j + 1, b, sb, sa, pb);
        }
    }
    for (; j < nt && !(j + 2 >= nc && j + 5 < nt); j += 2) {
        b = step(any_kind, j, b, sa, sb, pa);
        b = step(any_kind, j + 1, b, sb, sa, pb);
    }
    if (j + 5 < nt) {
        drain();
        for (; j + 5 < nt; j += 2) {          // tiles j+2 .. j+5 all new keys
            b = step(new_kind, j, b, sa, sb, pa);
            b = step(new_kind, j + 1, b, sb, sa, pb);
        }
    }
    for (; j < nt; j += 2) {
        b = step(any_kind, j, b, sa, sb, pa);
        b = step(any_kind, j + 1, b, sb, sa, pb);
    }

    // ---- epilogue: O / l -> bf16; lse = (m + log2 l) ln 2
    const float lt = half_sum(ws.lsum);
    const float inv = 1.0f / lt;
    const int row = r0 + wave * QW + l32;
    if (row < r1) {
        uint16_t* dst = A.out + ((int64_t)row * A.H + head) * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint2*>(dst + 32 * db + 8 * i + 4 * g) =
                    make_uint2(pack_bf16(ws.o[db][4 * i] * inv, ws.o[db][4 * i + 1] * inv),
                               pack_bf16(ws.o[db][4 * i + 2] * inv, ws.o[db][4 * i + 3] * inv));
        if (A.lse && g == 0) A.lse[(int64_t)head * A.Ln + row] = (ws.m + __log2f(lt)) * 0.69314718055994531f;
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
