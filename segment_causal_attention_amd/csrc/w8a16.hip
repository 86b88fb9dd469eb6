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
// GEMM shape.  A workgroup (8 waves, 2 per SIMD) computes a 384 x 256 tile of
// y; wave w owns rows 96 (w % 4) .. +96 and columns 128 (w / 4) .. +128 as
// 3 x 4 accumulators of v_mfma_f32_32x32x16_bf16 (A = x rows, B = W rows, both
// k-contiguous; 234 VGPRs).  Seven 16-byte fragment reads from LDS feed twelve
// products, against six for eight with 64 x 128 wave tiles: the LDS bytes per
// FLOP that bound a power-limited clock fall by a fifth.  K advances in steps
// of 64: the step's x tile (384 rows) and W tile (256 rows), 128 bytes per
// row, are copied into LDS (2 stages x 80 KB) by buffer-to-LDS
// DMA, 16-byte chunk c of row r landing at chunk c ^ ((r / 2) % 8) of the
// row.  A row is 128 bytes, half of the 64 four-byte banks, so rows 2i and
// 2i+1 cover the two halves; the swizzle by r / 2 spreads the 16 rows that a
// ds_read_b128 serves per cycle over all 16 groups of 4 banks, free of
// conflicts.  With NS stages, step t+NS-1 is copied into the stage step t-1
// left while step t computes (2 stages for the big tiles).  Reads of
// x past row M come back as zeros (buffer range checking); stores stop at M.
// Rows that would fill only a quarter or less of a last round of big tiles
// (and calls too small to fill one) take 128 x 128 tiles from the same code.
#include <mutex>

#include "common.hpp"

namespace nomas {

typedef __bf16 gbf16x8 __attribute__((ext_vector_type(8)));
typedef float gf32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t gu32x4 __attribute__((ext_vector_type(4)));

constexpr int GK = 64;              // K per step
constexpr int GNT = 512;            // threads (8 waves: 4 along the tile's rows, 2 along its columns)
constexpr int GGROUP = 8;           // row panels walked together by the tile order

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

// TM x TN tile per workgroup with NS LDS stages: 384 x 256 (96 x 128 per
// wave, 2 stages) for the bulk of a call, 128 x 128 (32 x 64 per wave) for
// rows that would leave the last round of big tiles mostly idle; a small
// tile's step computes too briefly to hide one copy's latency, so it keeps
// 4 stages (3 steps in flight).
template <int TM, int TN, int NS>
__global__ __launch_bounds__(GNT) void w8a16_gemm_kernel(const GemmArgs G) {
    constexpr int XB = TM * GK * 2;                 // bytes of the x tile of a step
    constexpr int STAGE = (TM + TN) * GK * 2;       // x tile then W tile
    constexpr int WMB = TM / 128, WNB = TN / 64;    // 32 x 32 accumulator blocks per wave
    constexpr int PER = TM / 64 + TN / 64;          // DMA instructions per wave and step
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    // Workgroups are dealt to the 8 XCDs in turn (block b to XCD b % 8).  Index
    // t = (b % 8) * ceil(nb / 8) + b / 8 gives each XCD a contiguous run of
    // the tile order, which walks groups of GGROUP row panels column by column:
    // the ~32 tiles an XCD holds at once span 8 row panels and 4 column panels,
    // so each K step's x and W slices are fetched into its L2 once for 4 or 8
    // tiles (8 x and 4 W panels per round, against 1 x and 32 W panels when an
    // XCD walks one row panel at a time).
    const int nb = G.ntm * G.ntn;
    const int per = (nb + 7) / 8;
    const int b = blockIdx.x;
    int tile = (b % 8) * per + b / 8;
    if ((b % 8) >= nb % 8 && nb % 8 != 0) tile -= (b % 8) - nb % 8;     // XCDs past the remainder hold one fewer
    const int span = GGROUP * G.ntn, grp = tile / span, fm = grp * GGROUP;
    const int gm = min(G.ntm - fm, GGROUP), rr = tile - grp * span;     // the last group may hold fewer rows
    const int tm = __builtin_amdgcn_readfirstlane(fm + rr % gm);
    const int tn = __builtin_amdgcn_readfirstlane(rr / gm);
    const int m0 = tm * TM, n0 = tn * TN;
    const int wm = (TM / 4) * (wave & 3), wn = (TN / 2) * (wave >> 2);
    const int nsteps = G.K / GK;
    const uint32_t rowb = (uint32_t)G.K * 2;                    // bytes per row of x and of W

    // buffer descriptors: x (its whole extent, so rows past M read as zero) and W
    const uint64_t xb = (uint64_t)(uintptr_t)G.x, wbp = (uint64_t)(uintptr_t)G.w;
    const gu32x4 rx = {(uint32_t)xb, (uint32_t)(xb >> 32) & 0xffffu, (uint32_t)G.M * rowb, 0x00020000u};
    const gu32x4 rw = {(uint32_t)wbp, (uint32_t)(wbp >> 32) & 0xffffu, (uint32_t)G.N * rowb, 0x00020000u};
    // wave w copies 8-row groups w, w+8, ... of the x tile and of the W tile
    const int wv = __builtin_amdgcn_readfirstlane(wave);       // wave-uniform, for scalar DMA operands
    // lane l of a 1 KB copy lands at row 8 grp + l/8, position l%8 of the row,
    // which holds chunk (l%8) ^ ((row / 2) % 8) = (l%8) ^ (l/16 + 4 (grp % 2));
    // grp % 2 = w % 2 for every group the wave copies
    const uint32_t voff = (uint32_t)(lane >> 3) * rowb + 16u * (uint32_t)((lane & 7) ^ ((lane >> 4) + 4 * (wv & 1)));
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
    auto copy_step = [&](int t, int st) {
        const uint32_t kb = (uint32_t)t * (GK * 2);
#pragma unroll
        for (int i = 0; i < TM / 64; ++i) {
            const int grp = wv + 8 * i;
            g_dma(lds0 + st * STAGE + 1024 * grp, voff, rx, (uint32_t)(m0 + 8 * grp) * rowb + kb);
        }
#pragma unroll
        for (int i = 0; i < TN / 64; ++i) {
            const int grp = wv + 8 * i;
            g_dma(lds0 + st * STAGE + XB + 1024 * grp, voff, rw, (uint32_t)(n0 + 8 * grp) * rowb + kb);
        }
    };

    gf32x16 acc[WMB][WNB];
#pragma unroll
    for (int i = 0; i < WMB; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < nsteps) copy_step(p, p);
    for (int t = 0; t < nsteps; ++t) {
        // this wave's copies of step t are in once at most the NS - 2 later
        // steps' copies are outstanding (near the end: none, conservatively);
        // after the barrier every wave's are, and every wave is past its reads
        // of step t-1, whose stage step t+NS-1 now fills
        if (t + NS - 2 < nsteps) g_wait<(NS - 2) * PER>();
        else g_wait<0>();
        lds_barrier();
        if (t + NS - 1 < nsteps) copy_step(t + NS - 1, (t + NS - 1) % NS);
        const uint8_t* xt = lds + (t % NS) * STAGE;
        const uint8_t* wt = xt + XB;
#pragma unroll
        for (int kk = 0; kk < GK / 16; ++kk) {
            // raised wave priority over the first half of the step's products
            // (-1 to -3% on the model shapes)
            if (kk == 0) __builtin_amdgcn_s_setprio(2);
            if (kk == 2) __builtin_amdgcn_s_setprio(0);
            gbf16x8 a[WMB], b[WNB];
#pragma unroll
            for (int i = 0; i < WMB; ++i) a[i] = g_frag(xt, wm + 32 * i + l32, 2 * kk + g);
#pragma unroll
            for (int j = 0; j < WNB; ++j) b[j] = g_frag(wt, wn + 32 * j + l32, 2 * kk + g);
#pragma unroll
            for (int i = 0; i < WMB; ++i)
#pragma unroll
                for (int j = 0; j < WNB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // acc[i][j] lane: column n0 + wn + 32 j + l32, rows m0 + wm + 32 i + 8 r4 + 4 g + r%4
#pragma unroll
    for (int i = 0; i < WMB; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j) {
            const int n = n0 + wn + 32 * j + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
                if (m < G.M) G.y[(int64_t)m * G.N + n] = (uint16_t)(pack_bf16(acc[i][j][r], 0.0f) & 0xffffu);
            }
        }
}

int64_t w8a16_workspace_bytes(int64_t N, int64_t K) { return N * K * 2; }

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: the dequantised weights of one
// call go into this static array of the code object instead of a caller
// workspace.  Each device that loads the library holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, so kernels
// are given the device address that hipGetSymbolAddress returns, looked up
// once per device with that device current.

static __device__ __align__(256) uint8_t scratch[NOMAS_W8A16_NOALLOC_MAX_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];
}  // namespace

void w8a16_scratch_forget() {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    for (int d = 0; d < kScratchDevices; ++d) g_scratch_ptr[d] = nullptr;
}

int w8a16_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return NOMAS_EHIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NOMAS_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return NOMAS_OK;
}

namespace {
int dev_current() {
    int d = 0;
    return hipGetDevice(&d) == hipSuccess ? d : 0;
}

template <int TM, int TN, int NS>
void gemm_launch(const uint16_t* x, const uint16_t* wb, uint16_t* y, int64_t M, int64_t N, int64_t K,
                 hipStream_t stream) {
    const int64_t ntm = (M + TM - 1) / TM, ntn = N / TN;
    const GemmArgs G{x, wb, y, (int32_t)M, (int32_t)N, (int32_t)K, (int32_t)ntm, (int32_t)ntn};
    hipLaunchKernelGGL((w8a16_gemm_kernel<TM, TN, NS>), dim3((unsigned)(ntm * ntn)), dim3(GNT), 0, stream, G);
}
}  // namespace

int launch_w8a16(const uint16_t* x, int64_t M, int64_t K, const int8_t* codes, const float* scale, int64_t N,
                 uint16_t* y, void* workspace, hipStream_t stream) {
    uint16_t* wb = static_cast<uint16_t*>(workspace);
    const int64_t groups = N * (K / 16);
    hipLaunchKernelGGL(w8_dequant_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream, codes, scale,
                       wb, N, (int)K);
    if (M > 0) {
        // Big tiles for the whole row panels that fill complete rounds of the
        // device's CUs (one workgroup per CU); when the last round would be at
        // most a quarter full, the rows after those panels go to 128 x 128
        // tiles instead, about a sixth of a big tile's time each.  Every
        // output is still summed over K in one workgroup, in the same order.
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev_current()) != hipSuccess || cus < 1)
            return NOMAS_EHIP;
        const int64_t ntn = N / 256, nb = ((M + 383) / 384) * ntn, tail = nb % cus;
        const int64_t mmain = (tail > 0 && 4 * tail <= cus) ? ((nb - tail) / ntn) * 384 : M;
        if (mmain > 0) gemm_launch<384, 256, 2>(x, wb, y, mmain, N, K, stream);
        if (mmain < M) gemm_launch<128, 128, 4>(x + mmain * K, wb, y + mmain * N, M - mmain, N, K, stream);
    }
    return hipGetLastError() == hipSuccess ? NOMAS_OK : NOMAS_EHIP;
}

}  // namespace nomas
