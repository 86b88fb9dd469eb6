// Segment-causal joint attention over the lifelong INT8 KV cache plus the
// current segment(s), for gfx950.
//
// What it computes (comfyui-wiki news page on Hy-Nomas, section 一个世界，分段生成;
// huaweicloud blog, section 2.1): query i of new segment a attends to every
// cached token and to the new tokens of segments 0..a, never to a later
// segment.  Cached K/V are INT8 with one fp32 scale per (token, head); the
// attention itself runs in BF16 (comfyui-wiki, 单张 4090 配置): cached entries
// enter the products as bf16(fl32(code*scale)); queries and new keys are
// rotated by 3D RoPE (comfyui-wiki, 模型内部: [16, 56, 56], theta 256) and
// rounded to bf16: queries on load in float32, keys in the pack kernel in
// float64 (the same rows nomas_rope3d gives the cache append).
//
// Two kernels.  The pack kernel lays the keys a call can touch (the cache,
// then the new tokens) out as 64-key tiles, each a byte image of what the
// attention kernel wants in LDS: the K tile [key][channel] and the V^T tile
// [channel][key], bf16, rows padded against bank conflicts, cache entries
// dequantised, tail keys zero.  It is bound by HBM and runs once per call.
// The attention kernel then copies tile images into LDS with buffer-to-LDS
// DMA (no registers, no conversion, no LDS stores), three tiles ahead into
// four buffers, and spends its vector instructions on the softmax alone:
// on gfx950 an MFMA hides only a few vector instructions, so every one taken
// out of the key loop shortens it.
//
// Attention kernel shape.  One workgroup = 8 waves x 32 query rows = 256 rows
// of one head, all inside one new segment, so every row allows the same keys:
// the cache [0, Lc) and the new tokens [0, end of its segment), i.e. a prefix
// of the packed key range; later segments are masked in the last tile.  Each
// wave runs a software pipeline across tiles: the S^T products of tile j+1
// issue between the softmax instructions of tile j, then the O^T products of
// tile j.  One LDS barrier per tile.
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
#include <algorithm>
#include <cstring>

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
constexpr int KSTR = D + 8;         // row stride of the K tile image (bf16), padded
constexpr int VSTR = BN + 8;        // row stride of the V^T tile image (bf16), padded
constexpr int KIMG = BN * KSTR * 2;           // bytes of the K tile image
constexpr int VIMG = D * VSTR * 2;            // bytes of the V^T tile image
constexpr int TILE_BYTES = KIMG + VIMG;       // 35840
constexpr int TILE_KB = TILE_BYTES / 1024;    // 35 one-kilobyte DMA copies per tile
constexpr int NBUF = 4;             // LDS tile buffers
constexpr int FD = 2;               // LDS fragment reads issued this many products ahead
static_assert(TILE_BYTES % 1024 == 0, "tile images are copied in 1 KB pieces");

// position (in the permuted V^T row) of key k of a tile
__device__ __forceinline__ int vperm_key(int k) {
    const int w = k & 15;
    const int p = w < 4 ? w : w < 8 ? w + 4 : w < 12 ? w - 4 : w;
    return (k & ~15) + p;
}

__device__ __forceinline__ float i8(uint32_t word, int byte) {
    return (float)(int8_t)(word >> (8 * byte));
}

// ---------------------------------------------------------------------------
// Pack kernel: one workgroup of 256 threads builds the image of tile t of
// head h.  Key x of the packed range is cache token x for x < Lc, new token
// x - Lc for x < Lc + Ln (its key rotated by 3D RoPE in float64 and rounded
// once to bf16), and zero beyond.

// The packed key ranges.  Region r holds nsel[r] selected cache tokens (the
// ranges rng0[r] .. rng0[r+1]-1 of the range table, in order) followed by
// the new tokens [0, nnew[r]), and starts at tile tile0[r] of a head's
// images.  Without a history selection there is one region: the whole cache,
// then every new token.  Segments that see different cache tokens get
// regions of their own.
struct KeyPlan {
    int32_t nreg;
    int32_t tile0[NOMAS_MAX_SEGS + 1];          // tile0[nreg]: tiles per head
    int32_t nsel[NOMAS_MAX_SEGS];
    int32_t nnew[NOMAS_MAX_SEGS];
    int32_t rng0[NOMAS_MAX_SEGS + 1];
    int32_t rstart[NOMAS_MAX_SEL_RANGES];       // cache token of the range's first key
    int32_t rkey0[NOMAS_MAX_SEL_RANGES];        // packed key (within the region) of that token
};

struct PackArgs {
    const int8_t* kc;
    const int8_t* vc;
    const float* ks;
    const float* vs;
    const uint16_t* k;              // new keys before RoPE
    const uint16_t* v;
    uint8_t* img;
    float* knorm;                   // [H][ntk]: largest squared key norm of each tile
    int64_t cap;
    int32_t H, ntk;                 // H: key/value heads (of k, v and the cache); ntk: tiles per head
    KeyPlan kp;
    SegTable segs;                  // the new segments (positions of the new keys)
    RopeTables rt;
};
static_assert(sizeof(PackArgs) <= 4000, "kernel arguments are passed by value");

// Where packed key x of region r comes from: a cache token, a new token, or
// neither (zero padding past the region's end).
struct KeySrc {
    int32_t cache, fresh;
};
__device__ __forceinline__ KeySrc key_source(const KeyPlan& kp, int r, int x) {
    if (x < kp.nsel[r]) {
        int j = kp.rng0[r];
        while (j + 1 < kp.rng0[r + 1] && kp.rkey0[j + 1] <= x) ++j;
        return {kp.rstart[j] + (x - kp.rkey0[j]), -1};
    }
    x -= kp.nsel[r];
    return {-1, x < kp.nnew[r] ? x : -1};
}

constexpr int PACK_NT = 256;

// the 8 bf16 values of channels 8j .. 8j+7 of a packed key (as 4 words)
__device__ __forceinline__ uint4 key_chunk(const PackArgs& P, int h, KeySrc x, int j, bool is_v) {
    if (x.cache >= 0) {
        const size_t row = (size_t)h * P.cap + x.cache;
        const int8_t* codes = (is_v ? P.vc : P.kc) + row * D + 8 * j;
        const float s = (is_v ? P.vs : P.ks)[row];
        const uint2 w = *reinterpret_cast<const uint2*>(codes);
        return make_uint4(pack_bf16(i8(w.x, 0) * s, i8(w.x, 1) * s), pack_bf16(i8(w.x, 2) * s, i8(w.x, 3) * s),
                          pack_bf16(i8(w.y, 0) * s, i8(w.y, 1) * s), pack_bf16(i8(w.y, 2) * s, i8(w.y, 3) * s));
    }
    if (x.fresh >= 0) {
        const uint16_t* src = (is_v ? P.v : P.k) + ((size_t)x.fresh * P.H + h) * D + 8 * j;
        const uint4 w = *reinterpret_cast<const uint4*>(src);
        // new keys are rotated here exactly as nomas_rope3d rotates them
        return is_v ? w : rope_chunk_f64(w, j, x.fresh, P.segs, P.rt);
    }
    return make_uint4(0, 0, 0, 0);
}

__global__ __launch_bounds__(PACK_NT) void pack_kernel(const PackArgs P) {
    __shared__ __attribute__((aligned(16))) uint16_t vt[D * VSTR];     // the V^T image
    __shared__ uint32_t kmax;       // bits of the largest squared key norm (non-negative floats order as integers)
    const int t = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int r = 0;
    while (r + 1 < P.kp.nreg && P.kp.tile0[r + 1] <= t) ++r;
    const int x0 = (t - P.kp.tile0[r]) * BN;
    uint8_t* img = P.img + ((size_t)h * P.ntk + t) * TILE_BYTES;
    if (tid == 0) kmax = 0;
    __syncthreads();
    // K: thread = (key, quarter of the channels); its 64 bytes go straight to
    // the key's image row.  The key's squared norm as the attention kernel
    // sees it (bf16) goes into the row padding (first word, the rest zero) and
    // into the tile's maximum.
    {
        const int key = tid >> 2, qd = tid & 3;
        uint4 w[4];
        const KeySrc src = key_source(P.kp, r, x0 + key);
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = key_chunk(P, h, src, 4 * qd + j, false);
        float n2 = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t ww[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = __uint_as_float(ww[e] << 16), b = __uint_as_float(ww[e] & 0xffff0000u);
                n2 = fmaf(a, a, fmaf(b, b, n2));
            }
        }
        n2 += __shfl_xor(n2, 1);
        n2 += __shfl_xor(n2, 2);
        uint4* row = reinterpret_cast<uint4*>(img + key * KSTR * 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) row[4 * qd + j] = w[j];
        if (qd == 0) {
            row[D / 8] = make_uint4(__float_as_uint(n2), 0, 0, 0);
            atomicMax(&kmax, __float_as_uint(n2));
        }
    }
    // V^T through LDS: thread = (key pair, 16 channels); each channel row gets
    // one word holding both keys (adjacent columns under the chunk
    // permutation), consecutive lanes on consecutive words
    {
        const int kp = tid & 31, cg = tid >> 5;
        const KeySrc sa = key_source(P.kp, r, x0 + 2 * kp), sb = key_source(P.kp, r, x0 + 2 * kp + 1);
        const uint4 a[2] = {key_chunk(P, h, sa, 2 * cg, true), key_chunk(P, h, sa, 2 * cg + 1, true)};
        const uint4 b[2] = {key_chunk(P, h, sb, 2 * cg, true), key_chunk(P, h, sb, 2 * cg + 1, true)};
        uint32_t* col = reinterpret_cast<uint32_t*>(vt + vperm_key(2 * kp));
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t wa = (&a[e >> 3].x)[(e >> 1) & 3], wb = (&b[e >> 3].x)[(e >> 1) & 3];
            const uint32_t lo = (e & 1) ? wa >> 16 : wa & 0xffffu, hi = (e & 1) ? wb >> 16 : wb & 0xffffu;
            col[(16 * cg + e) * (VSTR / 2)] = lo | (hi << 16);
        }
    }
    // padding of the V^T rows (128): zero
    if (tid < D) *reinterpret_cast<uint4*>(vt + tid * VSTR + BN) = make_uint4(0, 0, 0, 0);
    __syncthreads();
    uint4* dst = reinterpret_cast<uint4*>(img + KIMG);
    for (int i = tid; i < VIMG / 16; i += PACK_NT) dst[i] = reinterpret_cast<const uint4*>(vt)[i];
    if (tid == 0) P.knorm[(size_t)h * P.ntk + t] = __uint_as_float(kmax);
}

// ---------------------------------------------------------------------------
// Attention kernel

struct AttnArgs {
    const uint16_t* q;
    const uint8_t* img;             // packed tile images
    const float* knorm;             // [H][ntk] largest squared key norm per tile
    uint16_t* out;
    float* lse;
    float* po;                      // split tiles: partial outputs O/l [split][nf][128] fp32 and
    float* plse;                    //   partial log2-sum-exp [split][nf], for the (head, row)
    int64_t f0, nf;                 //   pairs f = head * Ln + row in [f0, f0 + nf)
    int32_t Ln, H, ntq, ntk;        // H: query heads; ntq: query tiles per head, ntk: key tiles per KV head
    int32_t grp;                    // query heads per key/value head (head h reads KV head h / grp)
    int32_t nsplit;                 // key-range parts of a split query tile
    int32_t nmain;                  // blocks [0, nmain): whole query tiles; the rest split into nsplit parts
    int32_t xcd_runs;               // 1: each of the 8 XCDs takes a contiguous run of units (see below)
    float scale_log2;               // sm_scale * log2(e)
    int32_t tile0[NOMAS_MAX_SEGS + 1];   // first query tile of each new segment
    int32_t order[NOMAS_MAX_SEGS];       // segments in launch order (most keys first)
    int32_t lt0[NOMAS_MAX_SEGS + 1];     // first launch-order tile of each of them
    int32_t ktile0[NOMAS_MAX_SEGS];      // first key tile (of a head's images) of each segment's region
    int32_t nsel[NOMAS_MAX_SEGS];        // cache tokens each segment sees (its region's first keys)
    SegTable segs;
    RopeTables rt;
};
static_assert(sizeof(AttnArgs) <= 4000, "kernel arguments are passed by value");

// One kilobyte of a tile image into LDS: lane l's 16 bytes, read at byte
// voff + soff of the resource, land at LDS byte m0 + 16 l.  Written as inline
// assembly so that the compiler does not tie LDS reads to outstanding DMA
// (it would wait for every copy in flight); the key loop waits itself.
__device__ __forceinline__ void dma_1k(uint32_t m0, uint32_t voff, u32x4 rs, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(m0), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}

// wait until at most N buffer-to-LDS copies of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_dma() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
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

__device__ __forceinline__ bf16x8 pchunk(const uint32_t (&pk)[16], int ch) {
    return __builtin_bit_cast(bf16x8, u32x4{pk[4 * ch], pk[4 * ch + 1], pk[4 * ch + 2], pk[4 * ch + 3]});
}

// ---------------------------------------------------------------------------
// The pipelined step j: 32 slots, each holding one matrix instruction, the
// LDS read of the operand FD slots ahead and a few vector instructions.
// Slots 0-15 issue the S^T products of tile j+1, slots 16-31 the O^T
// products of tile j.  The row max of tile j+1 is taken after the last
// product, where the waves wait for one another anyway; each
// probability pair is formed over three slots (scale and shift, exp2, pack
// and sum) so that no slot holds a chain of dependent vector instructions.

// max of 16 values as a tree of three-input maxima
__device__ __forceinline__ float max16(const f32x16 (&s)[2], int r0) {
    float m[6];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int k = r0 + (3 * i) / 2;
        m[i] = (3 * i) % 2 == 0 ? fmaxf(fmaxf(s[0][k], s[1][k]), s[0][k + 1])
                                : fmaxf(fmaxf(s[1][k], s[0][k + 1]), s[1][k + 1]);
    }
    m[5] = s[1][r0 + 7];
    return fmaxf(fmaxf(fmaxf(m[0], m[1]), m[2]), fmaxf(fmaxf(m[3], m[4]), m[5]));
}

// probability pair q in three stages; t holds the pairs in flight
__device__ __forceinline__ void prob_stage(int stage, int q, const f32x16 (&s)[2], WaveState& w, float c,
                                           float (&t)[4][2], uint32_t (&pk)[16]) {
    const int kb = q >> 3, r = 2 * (q & 7);
    float* x = t[q & 3];
    if (stage == 0) {
        x[0] = fmaf(s[kb][r], c, -w.m);
        x[1] = fmaf(s[kb][r + 1], c, -w.m);
    } else if (stage == 1) {
        x[0] = __builtin_amdgcn_exp2f(x[0]);
        x[1] = __builtin_amdgcn_exp2f(x[1]);
    } else {
        const nm_bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        pk[q] = pack_bf16(x[0], x[1]);
        w.lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(nm_bf16x2, pk[q]), ones, w.lsum, false);
    }
}

// mx: row max of s (this lane half), taken at the end of the previous step;
// returns the row max of sn, taken after the last product of this step.
// FIXED: w.m is a bound that holds for the whole key range, so the step takes
// no maxima and never rescales.
template <bool FIXED>
__device__ __forceinline__ float pipelined_step(const uint16_t* Kn, const uint16_t* V, int lim, int krd, int vrd,
                                                WaveState& w, f32x16 (&s)[2], float mx, f32x16 (&sn)[2], float c,
                                                int g) {
    if (lim < BN) {
        mask_tile(s, lim, g);
        if (!FIXED) mx = fmaxf(max16(s, 0), max16(s, 8));
    }
    const f32x16 zero = {};
    uint32_t pk[16];
    float t[4][2];
    bf16x8 fr[32];
    auto frag = [&](int i) { return i < 16 ? kfrag(Kn, krd, i) : vfrag(V, vrd, i - 16); };
#pragma unroll
    for (int i = 0; i < FD; ++i) fr[i] = frag(i);
    SLOT_FENCE();
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        if (i + FD < 32) fr[i + FD] = frag(i + FD);
        // the S^T products and the first O^T products of the step issue at a
        // raised wave priority, so the SIMD's two waves drift apart in phase
        // (measured -1.3% against no priority change; ending at slot 16: -0.8%)
        if (i == 0) __builtin_amdgcn_s_setprio(2);
        if (i == 20) __builtin_amdgcn_s_setprio(0);
        if (i < 16) sn[i & 1] = mfma(fr[i], w.qf[i >> 1], i < 2 ? zero : sn[i & 1]);
        else w.o[i & 3] = mfma(fr[i], pchunk(pk, (i - 16) >> 2), w.o[i & 3]);
        // rescale of tile j
        if (!FIXED && i == 2) update_max(mx, w, c);
        // probabilities: pair q in slots 3+q, 4+q, 5+q
#pragma unroll
        for (int st = 0; st < 3; ++st)
            if (i - 3 - st >= 0 && i - 3 - st < 16) prob_stage(st, i - 3 - st, s, w, c, t, pk);
        SLOT_FENCE();
    }
    return FIXED ? 0.0f : fmaxf(max16(sn, 0), max16(sn, 8));
}

template <bool B> struct Fixed { static constexpr bool value = B; };

__global__ __launch_bounds__(NT) void seg_attn_kernel(const AttnArgs A) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * TILE_BYTES];
    __shared__ float kred[NW];      // per wave: largest squared key norm of the key range

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    // Units u = head * ntq + launch-order query tile.  Blocks [0, nmain)
    // are units 0 .. nmain-1 whole; the others are the remaining units split
    // into nsplit key-range parts, part-major, so that the workgroups that
    // share a key range run side by side.  The segments with the most keys
    // go first (packed calls: the last segment), so that the grid does not
    // end on a few long workgroups.
    // Workgroup b is dispatched to XCD b % 8.  With xcd_runs, index w of n
    // equal-work units runs unit (w % 8) * (n / 8) + w / 8, so each XCD walks
    // a contiguous run of units (about two heads at 16 heads) and its CUs
    // stream the same head's tile images through its own L2.
    auto runs = [&](int w, int n) {
        const int q8 = n >> 3;
        return (A.xcd_runs && w < 8 * q8) ? (w & 7) * q8 + (w >> 3) : w;
    };
    int unit, split, parts;
    if ((int)blockIdx.x < A.nmain) {
        unit = runs(blockIdx.x, A.nmain);
        split = 0;
        parts = 1;
    } else {
        const int t = blockIdx.x - A.nmain, r = A.ntq * A.H - A.nmain;
        split = t / r;
        unit = A.nmain + (A.nmain > 0 ? t - split * r : runs(t - split * r, r));
        parts = A.nsplit;
    }
    unit = __builtin_amdgcn_readfirstlane(unit);
    split = __builtin_amdgcn_readfirstlane(split);
    parts = __builtin_amdgcn_readfirstlane(parts);
    const int head = __builtin_amdgcn_readfirstlane(unit / A.ntq);
    const int li = __builtin_amdgcn_readfirstlane(unit - head * A.ntq);

    int oi = 0;
    while (oi + 1 < A.segs.n && A.lt0[oi + 1] <= li) ++oi;
    const int a = A.order[oi];
    const int qt = A.tile0[a] + (li - A.lt0[oi]);
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
    // squared norm of the rotated query as the products see it (bf16)
    float q2 = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const u32x4 x = __builtin_bit_cast(u32x4, ws.qf[kk]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = __uint_as_float(x[e] << 16), b = __uint_as_float(x[e] & 0xffff0000u);
            q2 = fmaf(a, a, fmaf(b, b, q2));
        }
    }
    q2 = half_sum(q2);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) ws.o[db][r] = 0.0f;
    ws.m = -INFINITY;
    ws.lsum = 0.0f;

    // keys [0, nkeys) of the packed range are allowed: the cache and the new
    // tokens up to the end of this segment
    const int nkeys = __builtin_amdgcn_readfirstlane(A.nsel[a] + kend);
    const int64_t kbase = (int64_t)(head / A.grp) * A.ntk + A.ktile0[a];   // this segment's region of the images
    const int nt_all = (nkeys + BN - 1) / BN;
    // this workgroup's part of the key tiles: [t0, t0 + nt)
    const int t0 = __builtin_amdgcn_readfirstlane((int)((int64_t)split * nt_all / parts));
    const int nt = __builtin_amdgcn_readfirstlane((int)((int64_t)(split + 1) * nt_all / parts) - t0);
    const int krd = l32 * KSTR + 8 * g;             // this lane's K / V^T fragment offsets
    const int vrd = l32 * VSTR + 8 * g;
    {
        // largest squared norm of the allowed keys of this range: the tile
        // maxima of its full tiles, the keys' own norms (row padding of the
        // image) in a last, partial tile
        const int nfull = nt > 0 ? min(nt, (nkeys - t0 * BN) / BN) : 0;    // t0 * BN < nkeys when nt > 0
        float k2 = 0.0f;
        for (int t = tid; t < nfull; t += NT) k2 = fmaxf(k2, A.knorm[kbase + t0 + t]);
        if (nfull < nt && tid < nkeys - (t0 + nfull) * BN)
            k2 = fmaxf(k2, *reinterpret_cast<const float*>(A.img + (kbase + t0 + nfull) * TILE_BYTES +
                                                           tid * KSTR * 2 + 2 * D));
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) k2 = fmaxf(k2, __shfl_xor(k2, off));
        if (lane == 0) kred[wave] = k2;
    }

    // ---- tile copies: wave w copies kilobytes w, w+8, ... of each image
    const int wv = __builtin_amdgcn_readfirstlane(wave) & (NW - 1);
    const uint64_t hbase = (uint64_t)(uintptr_t)A.img + (uint64_t)kbase * TILE_BYTES;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
    const uint32_t lane16 = 16u * lane;
    auto copy_tile = [&](int tile, int b) {
        const uint64_t base = hbase + (uint64_t)(t0 + min(tile, nt - 1)) * TILE_BYTES;
        const u32x4 rs = {(uint32_t)base, (uint32_t)(base >> 32) & 0xffffu, (uint32_t)TILE_BYTES, 0x00020000u};
#pragma unroll
        for (int k = 0; k < (TILE_KB + NW - 1) / NW; ++k) {
            const int kb = wv + NW * k;
            if (kb < TILE_KB) dma_1k(lds0 + b * TILE_BYTES + 1024 * kb, lane16, rs, 1024u * kb);
        }
    };
    // wait for this wave's copies of the tile before the last one issued
    auto wait_prev_tile = [&] {
        if (wv < TILE_KB % NW) wait_dma<(TILE_KB + NW - 1) / NW>();
        else wait_dma<TILE_KB / NW>();
    };
    auto kbuf = [&](int b) { return reinterpret_cast<const uint16_t*>(lds + b * TILE_BYTES); };
    auto vbuf = [&](int b) { return reinterpret_cast<const uint16_t*>(lds + b * TILE_BYTES + KIMG); };
    // Keys a row may not see get probability 0, but 0 x NaN is NaN: a later
    // segment's non-finite value in the last tile would still reach P.V.  So
    // the last tile's columns of such keys are zeroed in LDS, in its buffer
    // and in the buffer of the clamped copy that the padding step after an
    // odd tile count reads.
    const int lim_last = nt > 0 ? nkeys - (t0 + nt - 1) * BN : BN;    // allowed keys of the last tile
    auto zero_vt = [&](int b) {
        uint16_t* vt = reinterpret_cast<uint16_t*>(lds + b * TILE_BYTES + KIMG);
        for (int i = tid; i < D * BN; i += NT) {
            const int key = i & (BN - 1);
            if (key >= lim_last) vt[(i >> 6) * VSTR + vperm_key(key)] = 0;
        }
    };

    // Tile t lives in buffer t % 4.  Step j copies tile j+3 into the buffer
    // that tile j-1 left, works on tiles j and j+1, and ends once its copies
    // of tile j+2 have landed and every wave has reached the barrier.
    if (nt > 0) {       // a key-range part can be empty when there are fewer tiles than parts
    copy_tile(0, 0);
    copy_tile(1, 1);
    copy_tile(2, 2);
    wait_dma<0>();      // tiles 0 and 1 (and 2) of this wave
    lds_barrier();
    if (nt == 1 && lim_last < BN) {
        zero_vt(0);
        zero_vt(1);
        lds_barrier();
    }

    f32x16 sa[2], sb[2];
    {
        const f32x16 zero = {};
#pragma unroll
        for (int i = 0; i < 16; ++i) sa[i & 1] = mfma(kfrag(kbuf(0), krd, i), ws.qf[i >> 1], i < 2 ? zero : sa[i & 1]);
    }
    float ma = fmaxf(max16(sa, 0), max16(sa, 8)), mb = 0.0f;    // row maxima of the two score sets
    // Cauchy-Schwarz: every score of this row is at most |q| max|k|.  When
    // that bound lies within 64 (base 2) of the first tile's largest score,
    // it serves as the softmax shift for the whole range: no probability
    // exceeds 1 and the largest is at least 2^-64, far from underflow.  Else
    // the shift follows the running maximum.  The choice is per wave.
    float k2max = kred[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) k2max = fmaxf(k2max, kred[i]);
    const float bound = c * __builtin_sqrtf(q2 * k2max);
    const bool fixed = nkeys - t0 * BN >= BN && __all(bound - c * half_max(ma) <= 64.0f);
    if (fixed) ws.m = bound;
    // Step j: scores of tile j in x, next tile's scores into y.  Steps past
    // the last tile see a fully masked tile and change nothing; steps go in
    // pairs so the two score sets swap roles without copies.
    // fx: Fixed<> (the shift); tail: the step may have to zero a buffer
    auto step = [&](auto fx, auto tail, int j, f32x16 (&x)[2], float mx, f32x16 (&y)[2]) {
        const int b0 = j & 3, b1 = (j + 1) & 3;
        copy_tile(j + 3, (j + 3) & 3);
        const int lim = j < nt ? min(BN, nkeys - (t0 + j) * BN) : 0;
        const float my = pipelined_step<decltype(fx)::value>(kbuf(b1), vbuf(b0), lim, krd, vrd, ws, x, mx, y, c, g);
        // the last tile (landed, read from the next step on) and its copy
        if (decltype(tail)::value && lim_last < BN && (j == nt - 2 || (j == nt - 1 && (nt & 1)))) zero_vt(b1);
        wait_prev_tile();
        lds_barrier();
        return my;
    };
    // steps nt-2 and, for odd nt, nt-1 zero; they fall in the last one or two pairs
    const int jt = max(0, (nt & 1) ? nt - 3 : nt - 2);
    if (fixed) {
        int j = 0;
        for (; j < jt; j += 2) {
            step(Fixed<true>{}, Fixed<false>{}, j, sa, 0.0f, sb);
            step(Fixed<true>{}, Fixed<false>{}, j + 1, sb, 0.0f, sa);
        }
        for (; j < nt; j += 2) {
            step(Fixed<true>{}, Fixed<true>{}, j, sa, 0.0f, sb);
            step(Fixed<true>{}, Fixed<true>{}, j + 1, sb, 0.0f, sa);
        }
    } else {
        int j = 0;
        for (; j < jt; j += 2) {
            mb = step(Fixed<false>{}, Fixed<false>{}, j, sa, ma, sb);
            ma = step(Fixed<false>{}, Fixed<false>{}, j + 1, sb, mb, sa);
        }
        for (; j < nt; j += 2) {
            mb = step(Fixed<false>{}, Fixed<true>{}, j, sa, ma, sb);
            ma = step(Fixed<false>{}, Fixed<true>{}, j + 1, sb, mb, sa);
        }
    }
    wait_dma<0>();
    }

    // ---- epilogue: O / l -> bf16; lse = (m + log2 l) ln 2
    const float lt = half_sum(ws.lsum);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const int row = r0 + wave * QW + l32;
    if (row < r1 && parts > 1) {
        // partial result of this key range: O/l in fp32 and log2-sum-exp
        const int64_t f = (int64_t)head * A.Ln + row - A.f0;
        float* dst = A.po + ((int64_t)split * A.nf + f) * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<float4*>(dst + 32 * db + 8 * i + 4 * g) =
                    make_float4(ws.o[db][4 * i] * inv, ws.o[db][4 * i + 1] * inv, ws.o[db][4 * i + 2] * inv,
                                ws.o[db][4 * i + 3] * inv);
        if (g == 0) A.plse[(int64_t)split * A.nf + f] = lt > 0.0f ? ws.m + __log2f(lt) : -INFINITY;
    } else if (row < r1) {
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

// Merge of the key-range parts (log-sum-exp identity): for each (row, head)
// lse = log2 sum_s 2^lse_s, out = sum_s 2^(lse_s - lse) * (O/l)_s.
// 32 threads per (row, head), 4 channels each, over the pairs f = head * Ln
// + row >= f0: the split query tiles are the last units in head-major order,
// so their rows are a suffix of these pairs.
struct MergeArgs {
    const float* po;
    const float* plse;
    uint16_t* out;
    float* lse;
    int64_t f0;
    int32_t Ln, H, nsplit;
};

__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs M) {
    const int64_t f = M.f0 + (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    if (f >= (int64_t)M.Ln * M.H) return;
    const int head = (int)(f / M.Ln), row = (int)(f - (int64_t)head * M.Ln);
    const int64_t pair = (int64_t)row * M.H + head;
    const int ch = 4 * (threadIdx.x & 31);
    float mx = -INFINITY;
    const int64_t nf = (int64_t)M.Ln * M.H - M.f0, fl = f - M.f0;
    for (int s = 0; s < M.nsplit; ++s) mx = fmaxf(mx, M.plse[(int64_t)s * nf + fl]);
    float wsum = 0.0f;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int s = 0; s < M.nsplit; ++s) {
        const float ls = M.plse[(int64_t)s * nf + fl];
        const float w = ls == -INFINITY ? 0.0f : exp2f(ls - mx);
        const float4 o = *reinterpret_cast<const float4*>(M.po + ((int64_t)s * nf + fl) * D + ch);
        wsum += w;
        acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
    }
    const float inv = 1.0f / wsum;
    *reinterpret_cast<uint2*>(M.out + pair * D + ch) =
        make_uint2(pack_bf16(acc.x * inv, acc.y * inv), pack_bf16(acc.z * inv, acc.w * inv));
    if (M.lse && ch == 0) M.lse[(int64_t)head * M.Ln + row] = (mx + __log2f(wsum)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------------------
// Launch planning

int device_cu_count() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}

// Packed key regions of a call (see KeyPlan) and each segment's region.
// sel_off == nullptr: one region, the whole cache then every new token.
// Otherwise segment a sees the cache-token ranges sel_ranges[2i], [2i+1] for
// i in [sel_off[a], sel_off[a+1]): sorted, non-overlapping, inside
// [0, Lc).  Segments with identical lists share one region (holding every new
// token); else each segment gets its own (its selection, then the new tokens
// up to its end).  Returns NOMAS_OK, NOMAS_EINVAL or NOMAS_EUNSUPPORTED.
int build_key_plan(const SegTable& segs, int Lc, int Ln, const int32_t* sel_off, const int64_t* sel_ranges,
                   KeyPlan* kp, int32_t* seg_reg) {
    std::memset(kp, 0, sizeof(*kp));
    const int n = segs.n;
    auto seg_end = [&](int a) {
        const SegDev& d = segs.s[a];
        return d.start + d.n_text + d.T * d.Hg * d.Wg;
    };
    auto finish = [&]() {
        int64_t tiles = 0;
        for (int r = 0; r < kp->nreg; ++r) {
            kp->tile0[r] = (int32_t)tiles;
            tiles += ((int64_t)kp->nsel[r] + kp->nnew[r] + BN - 1) / BN;
        }
        if (tiles >= ((int64_t)1 << 24)) return (int)NOMAS_EUNSUPPORTED;
        kp->tile0[kp->nreg] = (int32_t)tiles;
        return (int)NOMAS_OK;
    };
    if (!sel_off) {
        kp->nreg = 1;
        kp->nsel[0] = Lc;
        kp->nnew[0] = Ln;
        kp->rng0[0] = 0;
        kp->rng0[1] = Lc > 0 ? 1 : 0;
        kp->rstart[0] = 0;
        kp->rkey0[0] = 0;
        for (int a = 0; a < n; ++a) seg_reg[a] = 0;
        return finish();
    }
    if (!sel_ranges && sel_off[n] > 0) return NOMAS_EINVAL;
    if (sel_off[0] != 0) return NOMAS_EINVAL;
    for (int a = 0; a < n; ++a)
        if (sel_off[a + 1] < sel_off[a]) return NOMAS_EINVAL;
    if (sel_off[n] > NOMAS_MAX_SEL_RANGES) return NOMAS_EUNSUPPORTED;
    for (int a = 0; a < n; ++a) {
        int64_t prev_end = 0;
        for (int i = sel_off[a]; i < sel_off[a + 1]; ++i) {
            const int64_t lo = sel_ranges[2 * i], hi = sel_ranges[2 * i + 1];
            if (lo < prev_end || hi <= lo || hi > Lc) return NOMAS_EINVAL;
            prev_end = hi;
        }
    }
    bool same = true;
    for (int a = 1; a < n && same; ++a) {
        const int na = sel_off[a + 1] - sel_off[a];
        if (na != sel_off[1] - sel_off[0]) { same = false; break; }
        for (int i = 0; i < 2 * na; ++i)
            if (sel_ranges[2 * sel_off[a] + i] != sel_ranges[2 * sel_off[0] + i]) { same = false; break; }
    }
    kp->nreg = same ? 1 : n;
    int nr = 0;
    for (int r = 0; r < kp->nreg; ++r) {
        kp->rng0[r] = nr;
        int32_t key = 0;
        for (int i = sel_off[r]; i < sel_off[r + 1]; ++i) {
            kp->rstart[nr] = (int32_t)sel_ranges[2 * i];
            kp->rkey0[nr] = key;
            key += (int32_t)(sel_ranges[2 * i + 1] - sel_ranges[2 * i]);
            ++nr;
        }
        kp->nsel[r] = key;
        kp->nnew[r] = same ? Ln : seg_end(r);
    }
    kp->rng0[kp->nreg] = nr;
    for (int a = 0; a < n; ++a) seg_reg[a] = same ? 0 : a;
    return finish();
}

// How the query tiles are split into key-range parts: the first `main`
// units (head-major, launch order) run whole, the others in `parts` parts.
struct SplitPlan {
    int parts;
    int64_t main;
};

// First (head, row) pair f = head * Ln + row of the split units: with
// main > 0 there is one segment (starting at row 0) and the split units are
// its last query tiles in head-major order, so their rows are the suffix
// from query tile main % ntq of head main / ntq on.
static int64_t split_f0(const SplitPlan& sp, int ntq, int Ln) {
    return sp.main > 0 ? sp.main / ntq * Ln + sp.main % ntq * BM : 0;
}
static int query_tiles(const SegTable& segs) {
    int nt = 0;
    for (int i = 0; i < segs.n; ++i) {
        const SegDev& s = segs.s[i];
        nt += (s.n_text + s.T * s.Hg * s.Wg + BM - 1) / BM;
    }
    return nt;
}

// Forced when n_split > 0: every unit in n_split parts.  Otherwise, with
// one workgroup per CU, a grid of u equal units takes ceil(u / CUs) rounds
// and its last round may run mostly empty.  Two remedies are priced, in
// units of one workgroup's whole key range:
//  - every unit in p = 2..4 parts: ceil(p u / CUs) / p rounds;
//  - for one segment (units of equal work), only the r = u mod CUs units of
//    the last round, in s = 2..8 parts: floor(u / CUs) + ceil(r s / CUs) / s.
// Split units pay the merge pass, which moves s * 516 + 260 bytes per
// (query, head) at HBM speed while the attention spends 512 FLOP per
// (query, key, head) on MFMA (about 250 FLOP per byte apart, as measured),
// and 2% per extra part for the parts' own prologues and fp32 partial
// outputs.  Every part keeps 16 key tiles or more.
SplitPlan plan_splits(const SegTable& segs, const KeyPlan& kp, const int32_t* seg_reg, int H, int n_split) {
    if (n_split > 0) return {n_split, 0};
    int nq = 0, nt_min = 1 << 30, nseg = 0;
    double keys = 0.0;              // sum over query tiles of their key count
    for (int i = 0; i < segs.n; ++i) {
        const SegDev& s = segs.s[i];
        const int ntok = s.n_text + s.T * s.Hg * s.Wg;
        if (ntok == 0) continue;
        const int tiles = (ntok + BM - 1) / BM;
        const int nk = kp.nsel[seg_reg[i]] + s.start + ntok;
        nq += tiles;
        nt_min = std::min(nt_min, (nk + BN - 1) / BN);
        keys += (double)tiles * nk;
        ++nseg;
    }
    const int cus = device_cu_count();
    if (nq == 0 || cus <= 0) return {1, 0};
    const int64_t units = (int64_t)nq * H;
    const double keys_avg = keys / nq;
    auto overhead = [&](int p) { return (p * 516.0 + 260.0) * 250.0 / (512.0 * keys_avg) + 0.02 * (p - 1); };
    SplitPlan best{1, 0};
    double best_cost = (double)((units + cus - 1) / cus);
    for (int p = 2; p <= 4 && nt_min / p >= 16; ++p) {
        const double cost = (double)((units * p + cus - 1) / cus) / p * (1.0 + overhead(p));
        if (cost < best_cost - 1e-9) { best = {p, 0}; best_cost = cost; }
    }
    const int64_t r = units % cus;
    // one segment: its tiles all see the same keys, and the units past
    // `main` are the last rows of the last heads (the merge relies on it)
    if (segs.n == 1 && nseg == 1 && r > 0 && segs.s[0].start == 0) {
        for (int p = 2; p <= 8 && nt_min / p >= 16; ++p) {
            const double cost = (double)(units / cus) + (double)((r * p + cus - 1) / cus) / p +
                                (double)r / cus * overhead(p);
            if (cost < best_cost - 1e-9) { best = {p, units - r}; best_cost = cost; }
        }
    }
    return best;
}

// per-tile key norms follow the images, padded to 256 bytes
static int64_t knorm_bytes(int64_t tiles) { return (tiles * 4 + 255) / 256 * 256; }

// Workspace bytes, or a negative error code for an invalid selection.  H
// query heads, Hkv key/value heads (tile images are per KV head).
int64_t seg_attn_workspace_bytes(const SegTable& segs, int Lc, int Ln, int H, int Hkv, int n_split,
                                 const int32_t* sel_off, const int64_t* sel_ranges) {
    KeyPlan kp;
    int32_t seg_reg[NOMAS_MAX_SEGS];
    const int rc = build_key_plan(segs, Lc, Ln, sel_off, sel_ranges, &kp, seg_reg);
    if (rc != NOMAS_OK) return rc;
    const SplitPlan sp = plan_splits(segs, kp, seg_reg, H, n_split);
    const int64_t tiles = (int64_t)Hkv * kp.tile0[kp.nreg];
    int64_t b = tiles * TILE_BYTES + knorm_bytes(tiles);
    if (sp.parts > 1) b += (int64_t)sp.parts * ((int64_t)Ln * H - split_f0(sp, query_tiles(segs), Ln)) * (D + 1) * 4;
    return b;
}

int launch_seg_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const SegTable& segs,
                    int Ln, const int8_t* kc, const int8_t* vc, const float* ks, const float* vs,
                    int64_t cap, int Lc, const int32_t* sel_off, const int64_t* sel_ranges, int H, int Hkv,
                    float sm_scale, uint16_t* out, float* lse, int n_split, void* workspace, const RopeTables& rt,
                    hipStream_t stream) {
    PackArgs P{};
    int32_t seg_reg[NOMAS_MAX_SEGS];
    const int rc = build_key_plan(segs, Lc, Ln, sel_off, sel_ranges, &P.kp, seg_reg);
    if (rc != NOMAS_OK) return rc;
    const SplitPlan sp = plan_splits(segs, P.kp, seg_reg, H, n_split);
    const int nsplit = sp.parts;
    const int ntk = P.kp.tile0[P.kp.nreg];
    P.kc = kc; P.vc = vc; P.ks = ks; P.vs = vs;
    P.k = k; P.v = v;
    P.img = static_cast<uint8_t*>(workspace);
    P.knorm = reinterpret_cast<float*>(P.img + (int64_t)Hkv * ntk * TILE_BYTES);
    P.cap = cap; P.H = Hkv; P.ntk = ntk;
    P.segs = segs;
    P.rt = rt;

    AttnArgs A{};
    A.q = q; A.img = P.img; A.knorm = P.knorm;
    A.out = out; A.lse = lse;
    A.Ln = Ln; A.H = H; A.ntk = ntk;
    A.grp = H / Hkv;
    A.nsplit = nsplit;
    A.nmain = (int32_t)sp.main;
    A.xcd_runs = segs.n == 1 ? 1 : 0;       // one segment: every query tile sees the same keys
    A.f0 = split_f0(sp, query_tiles(segs), Ln);
    A.nf = (int64_t)Ln * H - A.f0;
    if (nsplit > 1) {
        A.po = reinterpret_cast<float*>(P.img + (int64_t)Hkv * ntk * TILE_BYTES + knorm_bytes((int64_t)Hkv * ntk));
        A.plse = A.po + (int64_t)nsplit * A.nf * D;
    }
    A.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
    int nt = 0;
    for (int i = 0; i < segs.n; ++i) {
        A.tile0[i] = nt;
        A.ktile0[i] = P.kp.tile0[seg_reg[i]];
        A.nsel[i] = P.kp.nsel[seg_reg[i]];
        const SegDev& s = segs.s[i];
        const int ntok = s.n_text + s.T * s.Hg * s.Wg;
        nt += (ntok + BM - 1) / BM;
    }
    A.tile0[segs.n] = nt;
    A.ntq = nt;
    // launch order: segments by descending key count (stable)
    {
        int nk[NOMAS_MAX_SEGS];
        for (int i = 0; i < segs.n; ++i) {
            const SegDev& s = segs.s[i];
            nk[i] = A.nsel[i] + s.start + s.n_text + s.T * s.Hg * s.Wg;
            A.order[i] = i;
        }
        std::stable_sort(A.order, A.order + segs.n, [&](int x, int y) { return nk[x] > nk[y]; });
        int t = 0;
        for (int i = 0; i < segs.n; ++i) {
            A.lt0[i] = t;
            t += A.tile0[A.order[i] + 1] - A.tile0[A.order[i]];
        }
        A.lt0[segs.n] = t;
    }
    A.segs = segs;
    A.rt = rt;
    if (nt == 0) return NOMAS_OK;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)ntk, (unsigned)Hkv), dim3(PACK_NT), 0, stream, P);
    const int64_t units = (int64_t)nt * H;
    const int64_t blocks = sp.main + (units - sp.main) * nsplit;
    hipLaunchKernelGGL(seg_attn_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, A);
    if (nsplit > 1) {
        const MergeArgs M{A.po, A.plse, out, lse, A.f0, Ln, H, nsplit};
        const int64_t mb = (A.nf + 7) / 8;
        hipLaunchKernelGGL(merge_kernel, dim3((unsigned)mb), dim3(256), 0, stream, M);
    }
    return hipGetLastError() == hipSuccess ? NOMAS_OK : NOMAS_EHIP;
}

}  // namespace nomas
