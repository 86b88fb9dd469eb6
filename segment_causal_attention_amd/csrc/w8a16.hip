// Linear layer with INT8-stored weights and BF16 math: y = x . W^T.
//
// The DiT weights are stored INT8 while the linear layers compute in BF16
// (comfyui-wiki news page on Hy-Nomas, section 单张 4090 配置; huaweicloud blog,
// section 3.5 table).  Each weight enters the product as
// bf16(fl32(code * scale)) with one fp32 scale per output channel, as a
// cached key does; products accumulate in fp32 and y is rounded once to bf16.
//
// Two kernels.  The dequantisation kernel writes the BF16 weights once per
// call into the caller's workspace (N x K x 2 bytes, HBM-bound).  The GEMM
// kernel is then a plain BF16 MFMA loop with no conversion in it: on gfx950
// matrix and vector instructions of a SIMD largely serialise, so weights
// converted inside the loop would cost MFMA time.
//
// GEMM shape.  A workgroup (8 waves, 2 per SIMD) computes a 256 x 256 tile of
// y; wave w owns rows 64 (w % 4) .. +64 and columns 128 (w / 4) .. +128 as
// 2 x 4 accumulators of v_mfma_f32_32x32x16_bf16 (A = x rows, B = W rows, both
// k-contiguous).  K advances in steps of 64: the step's x tile (256 rows) and
// W tile (256 rows), 128 bytes per row, are copied into LDS by buffer-to-LDS
// DMA, 16-byte chunk c of row r landing at chunk c ^ ((r / 2) % 8) of the
// row.  A row is 128 bytes, half of the 64 four-byte banks, so rows 2i and
// 2i+1 cover the two halves; the swizzle by r / 2 spreads the 16 rows that a
// ds_read_b128 serves per cycle over all 16 groups of 4 banks, free of
// conflicts.  Two stages: step t+1
// is copied into the stage step t-1 left while step t computes.  Reads of
// x past row M come back as zeros (buffer range checking); stores stop at M.
#include "common.hpp"

namespace nomas {

typedef __bf16 gbf16x8 __attribute__((ext_vector_type(8)));
typedef float gf32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t gu32x4 __attribute__((ext_vector_type(4)));

constexpr int GT = 256;             // tile rows (x) and columns (W rows) per workgroup
constexpr int GK = 64;              // K per step
constexpr int GNT = 512;            // threads (8 waves)
constexpr int GTILE = GT * GK * 2;  // bytes of one operand tile (32 KB)
constexpr int GSTAGE = 2 * GTILE;   // x tile then W tile

// ---------------------------------------------------------------------------
// dequantisation: one thread = 16 weights of one output channel

__global__ __launch_bounds__(256) void w8_dequant_kernel(const int8_t* __restrict__ codes,
                                                         const float* __restrict__ scale, uint16_t* __restrict__ wb,
                                                         int64_t N, int K) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;      // 16-weight group
    const int64_t groups_per_row = K / 16;
    if (idx >= N * groups_per_row) return;
    const int64_t n = idx / groups_per_row;
    const float s = scale[n];
    const uint4 c = reinterpret_cast<const uint4*>(codes)[idx];
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float q0 = (float)(int8_t)(cw[i] & 0xff), q1 = (float)(int8_t)((cw[i] >> 8) & 0xff);
        const float q2 = (float)(int8_t)((cw[i] >> 16) & 0xff), q3 = (float)(int8_t)(cw[i] >> 24);
        o[2 * i] = pack_bf16(q0 * s, q1 * s);
        o[2 * i + 1] = pack_bf16(q2 * s, q3 * s);
    }
    uint4* dst = reinterpret_cast<uint4*>(wb) + 2 * idx;
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// ---------------------------------------------------------------------------
// GEMM

struct GemmArgs {
    const uint16_t* x;      // [M][K] bf16
    const uint16_t* w;      // [N][K] bf16 (dequantised)
    uint16_t* y;            // [M][N] bf16
    int32_t M, N, K;
    int32_t ntm, ntn;       // row and column tiles
};

__device__ __forceinline__ void g_dma(uint32_t m0, uint32_t voff, gu32x4 rs, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(m0), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void g_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// fragment of row `row` (tile-local), k chunk `ch` (8 bf16) from a swizzled tile
__device__ __forceinline__ gbf16x8 g_frag(const uint8_t* tile, int row, int ch) {
    return *reinterpret_cast<const gbf16x8*>(tile + row * (GK * 2) + 16 * (ch ^ ((row >> 1) & 7)));
}

__global__ __launch_bounds__(GNT) void w8a16_gemm_kernel(const GemmArgs G) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * GSTAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    // Workgroups are dealt to the 8 XCDs in turn (block b to XCD b % 8).  Tile
    // t = (b % 8) * ceil(nb / 8) + b / 8 gives each XCD a contiguous run of
    // tiles, row panel by row panel, so an x panel is read into one XCD's L2.
    const int nb = G.ntm * G.ntn;
    const int per = (nb + 7) / 8;
    const int b = blockIdx.x;
    int tile = (b % 8) * per + b / 8;
    if ((b % 8) >= nb % 8 && nb % 8 != 0) tile -= (b % 8) - nb % 8;     // XCDs past the remainder hold one fewer
    const int tm = __builtin_amdgcn_readfirstlane(tile / G.ntn);
    const int tn = __builtin_amdgcn_readfirstlane(tile - tm * G.ntn);
    const int m0 = tm * GT, n0 = tn * GT;
    const int wm = 64 * (wave & 3), wn = 128 * (wave >> 2);
    const int nsteps = G.K / GK;
    const uint32_t rowb = (uint32_t)G.K * 2;                    // bytes per row of x and of W

    // buffer descriptors: x (its whole extent, so rows past M read as zero) and W
    const uint64_t xb = (uint64_t)(uintptr_t)G.x, wbp = (uint64_t)(uintptr_t)G.w;
    const gu32x4 rx = {(uint32_t)xb, (uint32_t)(xb >> 32) & 0xffffu, (uint32_t)G.M * rowb, 0x00020000u};
    const gu32x4 rw = {(uint32_t)wbp, (uint32_t)(wbp >> 32) & 0xffffu, (uint32_t)G.N * rowb, 0x00020000u};
    // wave w copies 8-row groups w, w+8, w+16, w+24 of the x tile and of the W tile
    const int wv = __builtin_amdgcn_readfirstlane(wave);       // wave-uniform, for scalar DMA operands
    // lane l of a 1 KB copy lands at row 8 grp + l/8, position l%8 of the row,
    // which holds chunk (l%8) ^ ((row / 2) % 8) = (l%8) ^ (l/16 + 4 (grp % 2));
    // grp % 2 = w % 2 for every group the wave copies
    const uint32_t voff = (uint32_t)(lane >> 3) * rowb + 16u * (uint32_t)((lane & 7) ^ ((lane >> 4) + 4 * (wv & 1)));
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
    auto copy_step = [&](int t, int st) {
        const uint32_t kb = (uint32_t)t * (GK * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int grp = wv + 8 * i;
            g_dma(lds0 + st * GSTAGE + 1024 * grp, voff, rx, (uint32_t)(m0 + 8 * grp) * rowb + kb);
            g_dma(lds0 + st * GSTAGE + GTILE + 1024 * grp, voff, rw, (uint32_t)(n0 + 8 * grp) * rowb + kb);
        }
    };

    gf32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    copy_step(0, 0);
    for (int t = 0; t < nsteps; ++t) {
        // this wave's copies of step t are in; after the barrier every wave's
        // are, and every wave is past its reads of step t-1, whose stage step
        // t+1 now fills while step t computes
        g_wait<0>();
        lds_barrier();
        if (t + 1 < nsteps) copy_step(t + 1, (t + 1) & 1);
        const uint8_t* xt = lds + (t & 1) * GSTAGE;
        const uint8_t* wt = xt + GTILE;
#pragma unroll
        for (int kk = 0; kk < GK / 16; ++kk) {
            // raised wave priority over the first half of the step's products
            // (-1 to -3% on the model shapes)
            if (kk == 0) __builtin_amdgcn_s_setprio(2);
            if (kk == 2) __builtin_amdgcn_s_setprio(0);
            gbf16x8 a[2], b[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = g_frag(xt, wm + 32 * i + l32, 2 * kk + g);
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = g_frag(wt, wn + 32 * j + l32, 2 * kk + g);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // acc[i][j] lane: column n0 + wn + 32 j + l32, rows m0 + wm + 32 i + 8 r4 + 4 g + r%4
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn + 32 * j + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
                if (m < G.M) G.y[(int64_t)m * G.N + n] = (uint16_t)(pack_bf16(acc[i][j][r], 0.0f) & 0xffffu);
            }
        }
}

int64_t w8a16_workspace_bytes(int64_t N, int64_t K) { return N * K * 2; }

int launch_w8a16(const uint16_t* x, int64_t M, int64_t K, const int8_t* codes, const float* scale, int64_t N,
                 uint16_t* y, void* workspace, hipStream_t stream) {
    uint16_t* wb = static_cast<uint16_t*>(workspace);
    const int64_t groups = N * (K / 16);
    hipLaunchKernelGGL(w8_dequant_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream, codes, scale,
                       wb, N, (int)K);
    if (M > 0) {
        GemmArgs G{x, wb, y, (int32_t)M, (int32_t)N, (int32_t)K, (int32_t)((M + GT - 1) / GT), (int32_t)(N / GT)};
        const int64_t blocks = ((M + GT - 1) / GT) * (N / GT);
        hipLaunchKernelGGL(w8a16_gemm_kernel, dim3((unsigned)blocks), dim3(GNT), 0, stream, G);
    }
    return hipGetLastError() == hipSuccess ? NOMAS_OK : NOMAS_EHIP;
}

}  // namespace nomas
