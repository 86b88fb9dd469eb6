// Backward pass of packed segment-causal attention, for gfx950.
//
// What it computes.  Segment-forcing training packs a long video into one
// sequence of segments (huaweicloud blog, section 2.3: packed length up to
// 360,000 tokens) under the block-causal mask of the forward pass (comfyui-
// wiki news page, 一个世界，分段生成): query i of segment a attends to the
// tokens of segments 0..a.  Given dO, the gradient of the loss with respect to
// the attention output, and the forward's output O and log-sum-exp, per head
// and over the allowed pairs only:
//   S = sm_scale Qr Kr^T,  P = exp(S - lse),  dV = P^T dO,  dP = dO V^T,
//   D_i = sum_c dO_ic O_ic,  dS = P * (dP - D),
//   dQr = sm_scale dS Kr,  dKr = sm_scale dS^T Qr,
// then dq = R^T dQr and dk = R^T dKr back through the 3D RoPE rotation R.
// Qr and Kr are the rotated bf16 operands of the forward pass, rebuilt here
// bit for bit; P and dS enter their products as bf16, products accumulate in
// fp32 and the three gradients are returned in fp32.
//
// Layout.  Every segment starts a new 64-token tile, so a tile never mixes
// segments and the mask is whole tiles: query tiles of segment a see the key
// tiles of segments 0..a and nothing else.  Padding tokens past a segment's
// end are zero (keys, values, queries, dO) with lse = +inf, and contribute
// exactly zero to every gradient, so no kernel masks anything.  A pack kernel
// writes two images per tile, each a byte image of what an attention kernel
// wants in LDS:
//   query tile (35,840 B): Q rows [64][136] and dO rows [64][136] bf16, then
//     -lse / sm_scale and -D of the tile's tokens (fp32 [64] each).
//   key tile (34,816 B): K rows and V rows [64][136] bf16.
// Row strides are padded by 16 bytes, and within each 16-token block token
// 4a + b sits at row 4b + a, so that the plain row reads and the transposing
// reads below both hit distinct LDS banks.
//
// Two attention kernels, both on v_mfma_f32_32x32x16_bf16, 8 waves of 32
// tokens per workgroup, tiles copied into LDS by buffer-to-LDS DMA, four
// buffers deep:
//   dK/dV kernel, key on the MFMA's N side (one lane column = one key):
//     S = Q K^T and dP = dO V^T (A = Q, dO rows from LDS; B = the wave's K, V
//     held in registers), then dV^T += dO^T P and dK^T += Q^T dS (A = dO^T,
//     Q^T read from the same rows by the LDS transpose read; B = P, dS
//     straight from the accumulators).  It walks the query tiles of its
//     segment and every later one.
//   dQ kernel, query on the N side: S^T = K Q^T and dP^T = V dO^T (A = K, V
//     rows; B = the wave's Q, dO in registers), then dQ^T += K^T dS^T (K^T
//     by the transpose read).  It walks the key tiles of segments 0..a.
// S and dP are recomputed by both kernels instead of exchanging dQ partials
// between workgroups; at training lengths the pairs outnumber the tokens by
// five orders of magnitude, so any per-pair or per-block-pair exchange would
// be bound by HBM.
#include <algorithm>
#include <cstring>
#include <type_traits>

#include "common.hpp"

namespace nomas {
namespace {

typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef short s4v __attribute__((ext_vector_type(4)));

constexpr int TB = 64;                          // tokens per image tile
constexpr int RSTR = D + 8;                     // row stride (bf16) of [token][channel] images
constexpr int ROWIMG = TB * RSTR * 2;           // 17408
constexpr int QI_DO = ROWIMG;                   // query image: dO rows
constexpr int QI_LSE = 2 * ROWIMG;              //              -lse / sm_scale, fp32 [64]
constexpr int QI_D = 2 * ROWIMG + 4 * TB;       //              -D, fp32 [64]
constexpr int QIMG = 35 * 1024;                 // 35840 (35,328 used)
constexpr int KI_V = ROWIMG;                    // key image: V rows
constexpr int KIMG = 2 * ROWIMG;                // 34816
constexpr int QIMG_KB = QIMG / 1024;            // 35 one-kilobyte DMA copies
constexpr int KIMG_KB = KIMG / 1024;            // 34
static_assert(QIMG % 1024 == 0 && KIMG % 1024 == 0 && QI_D + 4 * TB <= QIMG, "tile images are copied in 1 KB pieces");

constexpr int NW = 8;                           // waves per workgroup (2 per SIMD)
constexpr int NT = NW * 64;
constexpr int WT = 32;                          // tokens per wave
constexpr int WG_TILES = NW * WT / TB;          // image tiles per workgroup (4)
constexpr int KBUF = 4;                         // key-tile buffers of the dQ kernel
constexpr int QBUF = 4;                         // query-tile buffers of the dK/dV kernel
constexpr int PACK_NT = 256;

// image row of token k of a tile: token 4a + b of each 16-token block at row 4b + a
__device__ __forceinline__ int trow(int k) { return (k & ~15) | ((k & 3) << 2) | ((k >> 2) & 3); }

__device__ __forceinline__ f16v mma(b8 a, b8 b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ b8 ldfrag(const uint8_t* p) { return *reinterpret_cast<const b8*>(p); }

__device__ __forceinline__ b8 chunk4(const uint32_t* w) {
    return __builtin_bit_cast(b8, u4v{w[0], w[1], w[2], w[3]});
}

// one kilobyte of an image into LDS (lane l's 16 bytes at LDS byte m0 + 16 l)
__device__ __forceinline__ void dma1k(uint32_t m0, uint32_t voff, u4v rs, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(m0), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void dma_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Segments and tiles as the kernels see them.  Tile t of a head's images
// belongs to segment a with tile0[a] <= t < tile0[a+1]; workgroups of the
// attention kernels come in the segment order `order`, segment order[i]
// owning blocks blk0[i] .. blk0[i+1]-1 (head-major, then its workgroups).
struct BwdPlan {
    int32_t nseg, T;                            // segments; tiles per head
    int32_t tile0[NOMAS_MAX_SEGS + 1];
    int32_t order[NOMAS_MAX_SEGS];
    int32_t blk0[NOMAS_MAX_SEGS + 1];
};

__device__ __forceinline__ int seg_end(const SegDev& s) { return s.start + s.n_text + s.T * s.Hg * s.Wg; }

// ---------------------------------------------------------------------------
// pack kernel: blockIdx = (tile, head, 0 query image | 1 key image)

struct PackBwdArgs {
    const uint16_t *q, *k, *v, *o, *dout;
    const float* lse;
    uint8_t *qimg, *kimg;
    int32_t Ln, H;
    float sm_scale;
    BwdPlan pl;
    SegTable segs;
    RopeTables rt;
};
static_assert(sizeof(PackBwdArgs) <= 4000, "kernel arguments are passed by value");

__global__ __launch_bounds__(PACK_NT) void bwd_pack_kernel(const PackBwdArgs P) {
    const int t = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const bool is_q = blockIdx.z == 0;
    int a = 0;
    while (a + 1 < P.pl.nseg && P.pl.tile0[a + 1] <= t) ++a;
    const SegDev& sg = P.segs.s[a];
    const int x0 = sg.start + (t - P.pl.tile0[a]) * TB;
    const int end = seg_end(sg);
    uint8_t* img = is_q ? P.qimg + ((size_t)h * P.pl.T + t) * QIMG : P.kimg + ((size_t)h * P.pl.T + t) * KIMG;

    // thread = (token, quarter of the channels): chunks 4 qd .. 4 qd + 3 of 8 channels
    const int row = tid >> 2, qd = tid & 3;
    const int tok = x0 + row;
    const bool valid = tok < end;
    const size_t src = ((size_t)(valid ? tok : 0) * P.H + h) * D;
    uint4 a0[4], a1[4];
    float dsum = 0.0f;
    if (is_q) {
        int tt = 0, hh = 0, ww = 0;
        if (!(valid && token_pos(P.segs, tok, tt, hh, ww))) tt = hh = ww = 0;   // text: identity rotation
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 4 * qd + j;
            if (valid) {
                // queries rotated exactly as the forward kernel rotates them
                a0[j] = rope_group_f32(reinterpret_cast<const uint4*>(P.q + src)[c], c, tt, hh, ww, P.rt);
                a1[j] = reinterpret_cast<const uint4*>(P.dout + src)[c];
                const uint4 ow = reinterpret_cast<const uint4*>(P.o + src)[c];
                const uint32_t dw[4] = {a1[j].x, a1[j].y, a1[j].z, a1[j].w};
                const uint32_t owv[4] = {ow.x, ow.y, ow.z, ow.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dsum = fmaf(bf16lo(dw[e]), bf16lo(owv[e]), fmaf(bf16hi(dw[e]), bf16hi(owv[e]), dsum));
            } else {
                a0[j] = a1[j] = make_uint4(0, 0, 0, 0);
            }
        }
        dsum += __shfl_xor(dsum, 1);
        dsum += __shfl_xor(dsum, 2);
        // -lse / sm_scale (so that P = 2^(sm_scale log2(e) (s + it))) and -D
        if (qd == 0) {
            reinterpret_cast<float*>(img + QI_LSE)[row] = valid ? -P.lse[(size_t)h * P.Ln + tok] / P.sm_scale : -INFINITY;
            reinterpret_cast<float*>(img + QI_D)[row] = valid ? -dsum : 0.0f;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 4 * qd + j;
            // keys rotated in float64 exactly as the forward pack kernel does
            a0[j] = valid ? rope_chunk_f64(reinterpret_cast<const uint4*>(P.k + src)[c], c, tok, P.segs, P.rt)
                          : make_uint4(0, 0, 0, 0);
            a1[j] = valid ? reinterpret_cast<const uint4*>(P.v + src)[c] : make_uint4(0, 0, 0, 0);
        }
    }
    // the two row images (Q, dO or K, V), padding zero
    uint4* r0 = reinterpret_cast<uint4*>(img + trow(row) * RSTR * 2);
    uint4* r1 = reinterpret_cast<uint4*>(img + ROWIMG + trow(row) * RSTR * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        r0[4 * qd + j] = a0[j];
        r1[4 * qd + j] = a1[j];
    }
    if (qd == 0) {
        r0[D / 8] = make_uint4(0, 0, 0, 0);
        r1[D / 8] = make_uint4(0, 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// attention kernels

struct BwdArgs {
    const uint8_t* qimg;
    const uint8_t* kimg;
    float *dq, *dk, *dv;
    int32_t Ln, H;
    float c;                        // sm_scale * log2(e)
    float sm_scale;
    BwdPlan pl;
    SegTable segs;
    RopeTables rt;
};
static_assert(sizeof(BwdArgs) <= 4000, "kernel arguments are passed by value");

// Workgroup -> (segment, head, first tile).  A workgroup (8 waves) covers
// NTL = 4 tiles of one segment; wave w takes tile tile0 + NTL wg + w/2,
// tokens 32 (w%2) .. +32 of it.  Waves past the segment's last tile repeat
// that tile and store nothing.
struct WgPos {
    int a, head, tile, row;
    bool live;
};
template <int NTL>
__device__ __forceinline__ WgPos wg_pos(const BwdPlan& pl, int wave) {
    const int b = blockIdx.x;
    int i = 0;
    while (i + 1 < pl.nseg && pl.blk0[i + 1] <= b) ++i;
    WgPos p;
    p.a = __builtin_amdgcn_readfirstlane(pl.order[i]);
    const int nt = pl.tile0[p.a + 1] - pl.tile0[p.a];
    const int nwg = (nt + NTL - 1) / NTL;
    const int local = b - pl.blk0[i];
    p.head = __builtin_amdgcn_readfirstlane(local / nwg);
    const int wg = local - p.head * nwg;
    const int tl = NTL * wg + (wave >> 1);
    p.live = tl < nt;
    p.tile = pl.tile0[p.a] + min(tl, nt - 1);
    p.row = WT * (wave & 1);
    return p;
}

// The transpose of the RoPE rotation applied to 4 channels 8 grp + 4 g .. +3
// (two pairs) of a token at (t, h, w), text tokens unchanged; x scaled by s.
__device__ __forceinline__ float4 unrotate4(float4 x, float s, bool vid, int grp, int g, int t, int h, int w,
                                            const RopeTables& rt) {
    x.x *= s; x.y *= s; x.z *= s; x.w *= s;
    if (!vid) return x;
    const float4 cs = *reinterpret_cast<const float4*>(rt.f32 + rope_entry(grp, t, h, w) + 2 * g);
    return make_float4(x.x * cs.x + x.y * cs.y, x.y * cs.x - x.x * cs.y,
                       x.z * cs.z + x.w * cs.w, x.w * cs.z - x.z * cs.w);
}

// Q / dO / K / V row fragment: token `r`, channels 16 s + 8 g
__device__ __forceinline__ b8 rowfrag(const uint8_t* img, int r, int s, int g) {
    return ldfrag(img + trow(r) * RSTR * 2 + 32 * s + 16 * g);
}
// Transposed fragment (A operand of dO^T, Q^T or K^T) from a row image in
// LDS: lane (channel ch0 + l32, half g) gets tokens 16 k16 + 4 g + 0..3 and
// 16 k16 + 8 + 4 g + 0..3, the token order in which the B operand leaves the
// accumulators.  ds_read_b64_tr_b16 works on groups of 16 lanes: lane 4e + m
// of a group names 4 consecutive elements of row e, and lane r of the group
// receives element r of rows 0..3.  So lane 4e + m of group (g, h) names
// token 16 k16 + 4 g + e (+8 for the second read), channels ch0 + 16 h + 4 m.
__device__ __forceinline__ b8 trfrag(const uint8_t* img, int ch0, int k16, int lane) {
    const int e = (lane >> 2) & 3, g = lane >> 5;
    const int ch = ch0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // trow(16 k16 + 4 g + e) = 16 k16 + 4 e + g; the +8 token is two rows on
    uint8_t* p = const_cast<uint8_t*>(img) + (16 * k16 + 4 * e + g) * RSTR * 2 + 2 * ch;
    const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)p);
    const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(p + 2 * RSTR * 2));
    return __builtin_bit_cast(b8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Nothing is scheduled across this point: it pins the order of the slots of
// the pipelined loop bodies (one matrix instruction each, plus the LDS read
// of a later operand and a few vector instructions).
#define SLOT() __builtin_amdgcn_sched_barrier(0)
constexpr int FD = 2;               // LDS operand reads issued this many products ahead (dQ)
constexpr int KFD = 1;              // the same for dK/dV (its registers hold P in fp32 for dS)

// ---- dQ: lane = query --------------------------------------------------------
//
// Per key tile and wave (32 queries x 64 keys, 48 products): the products of
// key block 0 (S^T and dP^T alternating) with the dS of the previous tile's
// block 1 in their slots, those of key block 1 with the dS of block 0 in
// theirs, then the dQ^T products of the previous tile's block 1 and of this
// tile's block 0: one score per slot and stage throughout, so that the
// vector work of each score hides behind a product.  Tiles are copied two
// ahead, so the previous tile's buffer is still intact.

__global__ __launch_bounds__(NT) void bwd_dq_kernel(const BwdArgs A) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[KBUF * KIMG];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const WgPos wp = wg_pos<WG_TILES>(A.pl, wave);
    const int qrow = wp.row + l32;
    const uint8_t* qi = A.qimg + ((size_t)wp.head * A.pl.T + wp.tile) * QIMG;
    b8 qf[8], df[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        qf[s] = rowfrag(qi, qrow, s, g);
        df[s] = rowfrag(qi + QI_DO, qrow, s, g);
    }
    // lse2 = lse log2(e) and D of this lane's query
    const float lse2 = -A.c * reinterpret_cast<const float*>(qi + QI_LSE)[qrow];
    const float dd = -reinterpret_cast<const float*>(qi + QI_D)[qrow];
    f16v acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

    // key tiles 0 .. tile0[a+1]-1: segments 0..a
    const int nk = __builtin_amdgcn_readfirstlane(A.pl.tile0[wp.a + 1]);
    const uint64_t kbase = (uint64_t)(uintptr_t)A.kimg + (uint64_t)wp.head * A.pl.T * KIMG;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto copy = [&](int j) {
        const uint64_t base = kbase + (uint64_t)min(j, nk - 1) * KIMG;
        const u4v rs = {(uint32_t)base, (uint32_t)(base >> 32) & 0xffffu, (uint32_t)KIMG, 0x00020000u};
        const uint32_t m = lds0 + (uint32_t)(j % KBUF) * KIMG;
#pragma unroll
        for (int p = 0; p < (KIMG_KB + NW - 1) / NW; ++p) {
            const int kb = wv + NW * p;
            if (kb < KIMG_KB) dma1k(m + 1024 * kb, 16u * lane, rs, 1024u * kb);
        }
    };
    const float c = A.c;
    const f16v zero = {};
    f16v negd;              // -D: the initial dP^T accumulator, so that dP - D comes out of the products
#pragma unroll
    for (int r = 0; r < 16; ++r) negd[r] = -dd;
    // The fourth buffer starts zeroed: the first tile's products for "the
    // previous tile's block 1" read it, with dS = 0, before any tile lands there.
    {
        uint4* z = reinterpret_cast<uint4*>(lds + (KBUF - 1) * KIMG);
        for (int i = tid; i < KIMG / 16; i += NT) z[i] = make_uint4(0, 0, 0, 0);
    }
    copy(0);
    copy(1);
    // Block 1 of a tile is finished in the next tile's slots, so its scores
    // (s[1], dp[1]) and then its dS (pk[8..15]) carry over; before the first
    // tile they give dS = 0 (2^(-1e30 c - lse) = 0, times dP - D = 0).
    f16v s[2], dp[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        s[1][r] = -1e30f;
        dp[1][r] = 0.0f;
    }
    uint32_t pk[16];
    float tx[8];
    float pe = 0.0f;
    // score e (0..31; block e / 16, register e % 16) through stage st:
    // 0: x = S c - lse2;  1: x = 2^x;  2: dS = x (dP - D), packed in pairs
    auto stage = [&](int st, int e) {
        const int kb = e >> 4, r = e & 15, i8 = e & 7;
        if (st == 0) {
            tx[i8] = fmaf(s[kb][r], c, -lse2);
        } else if (st == 1) {
            tx[i8] = __builtin_amdgcn_exp2f(tx[i8]);
        } else {
            const float v = tx[i8] * dp[kb][r];
            if (r & 1) pk[e >> 1] = pack_bf16(pe, v);
            else pe = v;
        }
    };
    // tile j lives in buffer j % 4, tile j-1 (whose block 1 is finished here)
    // in the one before; the loop is unrolled by 4 so that every LDS operand
    // address is the lane's base plus an immediate offset
    auto tile_step = [&](int j, auto bufc) {
        constexpr int bi = decltype(bufc)::value;
        constexpr int bp = (bi + KBUF - 1) % KBUF;
        // this wave's copies of tile j have landed once at most those of tile j+1 are in flight
        if (wv < KIMG_KB % NW) dma_wait<(KIMG_KB + NW - 1) / NW>();
        else dma_wait<KIMG_KB / NW>();
        lds_barrier();
        copy(j + 2);        // into the buffer of tile j-2, which every wave has finished
        const uint8_t* K = lds + bi * KIMG;
        const uint8_t* Kp = lds + bp * KIMG;
        // operand of product n: 0-31 S^T / dP^T of key blocks 0 and 1 of tile j
        // (even n: K rows, odd n: V rows; channel step (n % 16) / 2); 32-39
        // dQ^T of tile j-1's block 1 (channel block (n - 32) % 4, 16-key chunk
        // 2 + (n - 32) / 4); 40-47 dQ^T of tile j's block 0 (chunk (n - 40) / 4)
        auto afrag = [&](int n) {
            if (n < 32) return rowfrag(K + ((n & 1) ? KI_V : 0), 32 * (n >> 4) + l32, (n & 15) >> 1, g);
            if (n < 40) return trfrag(Kp, 32 * ((n - 32) & 3), 2 + ((n - 32) >> 2), lane);
            return trfrag(K, 32 * ((n - 40) & 3), (n - 40) >> 2, lane);
        };
        b8 fr[48];
#pragma unroll
        for (int n = 0; n < FD; ++n) fr[n] = afrag(n);
        SLOT();
#pragma unroll
        for (int n = 0; n < 48; ++n) {
            if (n + FD < 48) fr[n + FD] = afrag(n + FD);
            // raised wave priority over the S^T / dP^T products (-1% measured)
            if (n == 0) __builtin_amdgcn_s_setprio(2);
            if (n == 32) __builtin_amdgcn_s_setprio(0);
            // vector work first, one score per slot and stage: tile j-1's
            // block 1 in slots 0-17, tile j's block 0 in slots 16-33.  It reads
            // s[1] and dp[1] before this slot's product restarts their chains.
#pragma unroll
            for (int st = 0; st < 3; ++st) {
                const int e1 = n - st;
                if (e1 >= 0 && e1 < 16) stage(st, 16 + e1);
                const int e0 = n - 16 - st;
                if (e0 >= 0 && e0 < 16) stage(st, e0);
            }
            if (n < 32) {
                const int kb = n >> 4, m = n & 15;
                if (m & 1) dp[kb] = mma(fr[n], df[m >> 1], m < 2 ? negd : dp[kb]);
                else s[kb] = mma(fr[n], qf[m >> 1], m < 2 ? zero : s[kb]);
            } else if (n < 40) {
                const int m = n - 32;
                acc[m & 3] = mma(fr[n], chunk4(pk + 8 + 4 * (m >> 2)), acc[m & 3]);
            } else {
                const int m = n - 40;
                acc[m & 3] = mma(fr[n], chunk4(pk + 4 * (m >> 2)), acc[m & 3]);
            }
            SLOT();
        }
    };
    for (int j = 0; j < nk; j += KBUF) {
        tile_step(j, std::integral_constant<int, 0>{});
        if (j + 1 < nk) tile_step(j + 1, std::integral_constant<int, 1>{});
        if (j + 2 < nk) tile_step(j + 2, std::integral_constant<int, 2>{});
        if (j + 3 < nk) tile_step(j + 3, std::integral_constant<int, 3>{});
    }
    // the last tile's block 1: its dS and dQ^T products
    {
        const uint8_t* Kl = lds + ((nk - 1) % KBUF) * KIMG;
#pragma unroll
        for (int e1 = 0; e1 < 16; ++e1)
#pragma unroll
            for (int st = 0; st < 3; ++st) stage(st, 16 + e1);
#pragma unroll
        for (int m = 0; m < 8; ++m)
            acc[m & 3] = mma(trfrag(Kl, 32 * (m & 3), 2 + (m >> 2), lane), chunk4(pk + 8 + 4 * (m >> 2)), acc[m & 3]);
    }
    dma_wait<0>();

    // epilogue: dq = R^T (sm_scale dQ^T), fp32
    const SegDev& sg = A.segs.s[wp.a];
    const int tok = sg.start + (wp.tile - A.pl.tile0[wp.a]) * TB + qrow;
    if (wp.live && tok < seg_end(sg)) {
        int t = 0, h = 0, w = 0;
        const bool vid = token_pos(A.segs, tok, t, h, w);
        float* dst = A.dq + ((size_t)tok * A.H + wp.head) * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 x = make_float4(acc[db][4 * i], acc[db][4 * i + 1], acc[db][4 * i + 2], acc[db][4 * i + 3]);
                *reinterpret_cast<float4*>(dst + 32 * db + 8 * i + 4 * g) =
                    unrotate4(x, A.sm_scale, vid, 4 * db + i, g, t, h, w, A.rt);
            }
    }
}

// ---- dK, dV: lane = key ------------------------------------------------------
//
// Per query tile and wave (64 queries x 32 keys, 64 products) two halves of
// 32 queries, each: the S products, the dP products with P formed in their
// slots, the dV^T products with dS formed in theirs, the dK^T products.

__global__ __launch_bounds__(NT) void bwd_dkv_kernel(const BwdArgs A) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[QBUF * QIMG];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const WgPos wp = wg_pos<WG_TILES>(A.pl, wave);
    const int krow = wp.row + l32;
    const uint8_t* ki = A.kimg + ((size_t)wp.head * A.pl.T + wp.tile) * KIMG;
    b8 kf[8], vf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        kf[s] = rowfrag(ki, krow, s, g);
        vf[s] = rowfrag(ki + KI_V, krow, s, g);
    }
    f16v dk[4], dv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dk[i][r] = dv[i][r] = 0.0f;

    // query tiles tile0[a] .. T-1: segment a and every later one
    const int q0 = __builtin_amdgcn_readfirstlane(A.pl.tile0[wp.a]);
    const int nq = __builtin_amdgcn_readfirstlane(A.pl.T - q0);
    const uint64_t qbase = (uint64_t)(uintptr_t)A.qimg + ((uint64_t)wp.head * A.pl.T + q0) * QIMG;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto copy = [&](int j) {
        const uint64_t base = qbase + (uint64_t)min(j, nq - 1) * QIMG;
        const u4v rs = {(uint32_t)base, (uint32_t)(base >> 32) & 0xffffu, (uint32_t)QIMG, 0x00020000u};
        const uint32_t m = lds0 + (uint32_t)(j % QBUF) * QIMG;
#pragma unroll
        for (int p = 0; p < (QIMG_KB + NW - 1) / NW; ++p) {
            const int kb = wv + NW * p;
            if (kb < QIMG_KB) dma1k(m + 1024 * kb, 16u * lane, rs, 1024u * kb);
        }
    };
    const float c = A.c;
    copy(0);
    copy(1);
    copy(2);
    // tile j lives in buffer j % 4 (the buffer's base is added once per tile)
    auto tile_step = [&](int j, int bi) {
        // this wave's copies of tile j have landed once at most those of tiles j+1, j+2 are in flight
        if (wv < QIMG_KB % NW) dma_wait<2 * ((QIMG_KB + NW - 1) / NW)>();
        else dma_wait<2 * (QIMG_KB / NW)>();
        lds_barrier();
        copy(j + 3);        // into the buffer of tile j-1, which every wave has finished
        const uint8_t* Q = lds + bi * QIMG;
        // Per 32-query half u, 32 slots of one product each: S (slots 0-7),
        // dP (8-15) with P formed in their slots, dV^T (16-23) with dS formed
        // in theirs, dK^T (24-31).  Register r of S and dP holds query
        // 32 u + 8 (r/4) + 4 g + r%4, whose -lse/sm_scale and -D are the
        // initial accumulators, so S + pad gives P = 2^(c (S + pad)) and
        // dP - D comes out of the products.
        auto afrag = [&](int n) {
            const int u = n >> 5, m = n & 31;
            if (m < 16) return rowfrag(Q + (m < 8 ? 0 : QI_DO), 32 * u + l32, m & 7, g);
            const int ch = (m >> 2) & 1, db = m & 3;
            return trfrag(Q + (m < 24 ? QI_DO : 0), 32 * db, 2 * u + ch, lane);
        };
        auto pad16 = [&](int off, int u) {
            f16v x;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 v = *reinterpret_cast<const float4*>(Q + off + 4 * (32 * u + 8 * r4 + 4 * g));
                x[4 * r4] = v.x; x[4 * r4 + 1] = v.y; x[4 * r4 + 2] = v.z; x[4 * r4 + 3] = v.w;
            }
            return x;
        };
        f16v sc = pad16(QI_LSE, 0), dp;
        uint32_t pp[8], ps[8];
        b8 fr[64];
#pragma unroll
        for (int n = 0; n < KFD; ++n) fr[n] = afrag(n);
        SLOT();
        auto slot = [&](int n) {
            const int u = n >> 5, m = n & 31;
            if (n + KFD < 64) fr[n + KFD] = afrag(n + KFD);
            // raised wave priority over the S and dP products of each half
            if (m == 0) __builtin_amdgcn_s_setprio(2);
            if (m == 16) __builtin_amdgcn_s_setprio(0);
            if (m == 4) dp = pad16(QI_D, u);
            if (m == 28 && u == 0) sc = pad16(QI_LSE, 1);
            if (m < 8) sc = mma(fr[n], kf[m], sc);
            else if (m < 16) dp = mma(fr[n], vf[m - 8], dp);
            else if (m < 24) dv[m & 3] = mma(fr[n], chunk4(pp + 4 * ((m >> 2) & 1)), dv[m & 3]);
            else dk[m & 3] = mma(fr[n], chunk4(ps + 4 * ((m >> 2) & 1)), dk[m & 3]);
            // P of scores 2 (m - 9), +1 in slots 9-16
            if (m >= 9 && m < 17) {
                const int r = 2 * (m - 9);
                const float p0 = __builtin_amdgcn_exp2f(sc[r] * c), p1 = __builtin_amdgcn_exp2f(sc[r + 1] * c);
                sc[r] = p0;
                sc[r + 1] = p1;
                pp[r >> 1] = pack_bf16(p0, p1);
            }
            // dS = P (dP - D) of scores 2 (m - 17), +1 in slots 17-24
            if (m >= 17 && m < 25) {
                const int r = 2 * (m - 17);
                ps[r >> 1] = pack_bf16(sc[r] * dp[r], sc[r + 1] * dp[r + 1]);
            }
            SLOT();
        };
#pragma unroll
        for (int n = 0; n < 32; ++n) slot(n);
#pragma unroll
        for (int n = 32; n < 64; ++n) slot(n);
    };
    for (int j = 0; j < nq; ++j) tile_step(j, j & 3);
    dma_wait<0>();

    // epilogue: dk = R^T (sm_scale dK^T), dv, fp32
    const SegDev& sg = A.segs.s[wp.a];
    const int tok = sg.start + (wp.tile - A.pl.tile0[wp.a]) * TB + krow;
    if (wp.live && tok < seg_end(sg)) {
        int t = 0, h = 0, w = 0;
        const bool vid = token_pos(A.segs, tok, t, h, w);
        float* dkd = A.dk + ((size_t)tok * A.H + wp.head) * D;
        float* dvd = A.dv + ((size_t)tok * A.H + wp.head) * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = 32 * db + 8 * i + 4 * g;
                const float4 x = make_float4(dk[db][4 * i], dk[db][4 * i + 1], dk[db][4 * i + 2], dk[db][4 * i + 3]);
                *reinterpret_cast<float4*>(dkd + ch) = unrotate4(x, A.sm_scale, vid, 4 * db + i, g, t, h, w, A.rt);
                *reinterpret_cast<float4*>(dvd + ch) =
                    make_float4(dv[db][4 * i], dv[db][4 * i + 1], dv[db][4 * i + 2], dv[db][4 * i + 3]);
            }
    }
}

// tiles per head and the per-segment tile offsets
int64_t plan_tiles(const SegTable& st, BwdPlan* pl) {
    std::memset(pl, 0, sizeof(*pl));
    pl->nseg = st.n;
    int64_t t = 0;
    for (int a = 0; a < st.n; ++a) {
        pl->tile0[a] = (int32_t)t;
        const SegDev& s = st.s[a];
        const int64_t n = (int64_t)s.n_text + (int64_t)s.T * s.Hg * s.Wg;
        t += (n + TB - 1) / TB;
    }
    pl->tile0[st.n] = (int32_t)t;
    pl->T = (int32_t)t;
    return t;
}

// block ranges in the given segment order; returns the block count
int64_t plan_blocks(BwdPlan* pl, int H, bool late_first, int tiles_per_wg) {
    int64_t b = 0;
    for (int i = 0; i < pl->nseg; ++i) {
        const int a = late_first ? pl->nseg - 1 - i : i;
        pl->order[i] = a;
        pl->blk0[i] = (int32_t)b;
        const int nt = pl->tile0[a + 1] - pl->tile0[a];
        b += (int64_t)H * ((nt + tiles_per_wg - 1) / tiles_per_wg);
    }
    pl->blk0[pl->nseg] = (int32_t)b;
    return b;
}

}  // namespace

int64_t seg_attn_bwd_workspace_bytes(const SegTable& st, int H) {
    BwdPlan pl;
    return (int64_t)H * plan_tiles(st, &pl) * (QIMG + KIMG);
}

int launch_seg_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                        const float* lse, const uint16_t* dout, const SegTable& st, int Ln, int H, float sm_scale,
                        float* dq, float* dk, float* dv, void* workspace, const RopeTables& rt, hipStream_t stream) {
    BwdPlan pl;
    const int64_t T = plan_tiles(st, &pl);
    uint8_t* qimg = static_cast<uint8_t*>(workspace);
    uint8_t* kimg = qimg + (size_t)H * T * QIMG;
    PackBwdArgs P{q, k, v, o, dout, lse, qimg, kimg, Ln, H, sm_scale, pl, st, rt};
    hipLaunchKernelGGL(bwd_pack_kernel, dim3((unsigned)T, (unsigned)H, 2), dim3(PACK_NT), 0, stream, P);
    BwdArgs A{qimg, kimg, dq, dk, dv, Ln, H, sm_scale * 1.44269504088896341f, sm_scale, pl, st, rt};
    // dK/dV: early segments (the most query tiles) first
    const int64_t nb_kv = plan_blocks(&A.pl, H, false, WG_TILES);
    hipLaunchKernelGGL(bwd_dkv_kernel, dim3((unsigned)nb_kv), dim3(NT), 0, stream, A);
    // dQ: late segments (the most key tiles) first
    const int64_t nb_q = plan_blocks(&A.pl, H, true, WG_TILES);
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)nb_q), dim3(NT), 0, stream, A);
    return hipGetLastError() == hipSuccess ? NOMAS_OK : NOMAS_EHIP;
}

}  // namespace nomas
