// Camera cross-attention (comfyui-wiki news page on Hy-Nomas, section
// 相机控制作为一等输入: 64-d camera tokens queried by the video tokens through
// cross-attention in every dual-stream block; section 模型内部: extrinsic
// embedding).  Linear layers and attention run in BF16 (same page, 单张 4090
// 配置), so the camera tokens are rounded to bf16, projected by the bf16
// weights with fp32 accumulation, and the projections rounded to bf16:
//   Kc = bf16(bf16(cam) . Wk_h),  Vc = bf16(bf16(cam) . Wv_h)       per head h
//   out_i = softmax_n(sm_scale <q_i, Kc_n>) . Vc_n                   (all n < Nc)
//
// HBM-bound: every query row is read once and its output written once; the
// scores need only Nc <= 128 keys.  A workgroup (8 waves) owns one head and
// 2048 query rows.  Its prologue builds Kc ([key][d]) and Vc^T ([d][key],
// keys permuted per 16 as in the attention kernel) in LDS with MFMA:
//   Kc^T (d x keys) = Wk_h^T (d x 64) . bf16(cam)^T (64 x keys).
// Each wave then streams 32-query blocks: S^T = Kc . Q^T and O^T = Vc^T . P^T
// on v_mfma_f32_32x32x16_bf16 with the query as the accumulator lane, an
// online softmax over 32-key blocks of camera tokens (so registers do not grow
// with Nc), and the next block's Q already in flight while the current one is
// computed.
#include "common.hpp"

namespace nomas {

typedef __bf16 cbf16x8 __attribute__((ext_vector_type(8)));
typedef float cf32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t cu32x4 __attribute__((ext_vector_type(4)));

constexpr int CAM_WAVES = 8;
constexpr int CAM_ROWS = 2048;              // query rows per workgroup
constexpr int CAM_MAXK = NOMAS_MAX_CAM;     // 128 keys at most
constexpr int CKSTR = D + 8;                // Kc row stride (bf16)
constexpr int CVSTR = CAM_MAXK + 8;         // Vc^T row stride (bf16)
constexpr int CWSTR = 64 + 8;               // W^T row stride (bf16)

__device__ __forceinline__ int cvperm(int k) {
    int w = k & 15;
    int p = (w >= 4 && w < 8) ? w + 4 : (w >= 8 && w < 12) ? w - 4 : w;
    return (k & ~15) + p;
}

template <int NKB>
__global__ __launch_bounds__(512) void cam_xattn_kernel(const uint16_t* __restrict__ q, int64_t Lq, int H,
                                                        const float* __restrict__ cam, int Nc,
                                                        const uint16_t* __restrict__ wk,
                                                        const uint16_t* __restrict__ wv, float scale_log2,
                                                        uint16_t* __restrict__ out, int nblk) {
    __shared__ __attribute__((aligned(16))) uint16_t Kc[CAM_MAXK * CKSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * CVSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Wt[D * CWSTR];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int head = blockIdx.x / nblk;
    const int64_t rbeg = (int64_t)(blockIdx.x - head * nblk) * CAM_ROWS;
    const int64_t rend = min(rbeg + CAM_ROWS, Lq);

    // ---- projections: K first, then V, through the transposed weight tile
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const uint16_t* W = which ? wv : wk;
        // W_h [64][128] -> Wt [128][64]: thread reads 8 channels of one input row
        for (int e = tid; e < 64 * 16; e += 512) {
            const int in = e >> 4, dg = e & 15;
            uint4 x = *reinterpret_cast<const uint4*>(W + (int64_t)in * H * D + head * D + 8 * dg);
            uint32_t xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Wt[(8 * dg + 2 * i) * CWSTR + in] = (uint16_t)(xv[i] & 0xffffu);
                Wt[(8 * dg + 2 * i + 1) * CWSTR + in] = (uint16_t)(xv[i] >> 16);
            }
        }
        __syncthreads();
        // 4 d-blocks x NKB key blocks, spread over the 8 waves
        for (int job = wave; job < 4 * NKB; job += CAM_WAVES) {
            const int db = job & 3, kb = job >> 2;
            const int key = 32 * kb + l32;
            cf32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                // camera token as the B operand (keys on N, inputs on K), rounded to bf16
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                if (key < Nc) {
                    const float4* src = reinterpret_cast<const float4*>(cam + (int64_t)key * 64 + 16 * kk + 8 * g);
                    const float4 x0 = src[0], x1 = src[1];
                    w[0] = pack_bf16(x0.x, x0.y); w[1] = pack_bf16(x0.z, x0.w);
                    w[2] = pack_bf16(x1.x, x1.y); w[3] = pack_bf16(x1.z, x1.w);
                }
                const cbf16x8 cb = __builtin_bit_cast(cbf16x8, cu32x4{w[0], w[1], w[2], w[3]});
                const cbf16x8 a = *reinterpret_cast<const cbf16x8*>(Wt + (32 * db + l32) * CWSTR + 16 * kk + 8 * g);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, cb, acc, 0, 0, 0);
            }
            // acc: lane = key 32kb + l32, regs = d 32db + 8i + 4g + j
            if (which == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<uint2*>(Kc + key * CKSTR + 32 * db + 8 * i + 4 * g) =
                        make_uint2(pack_bf16(acc[4 * i], acc[4 * i + 1]), pack_bf16(acc[4 * i + 2], acc[4 * i + 3]));
            } else {
                const int col = cvperm(key);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int d = 32 * db + 8 * (r >> 2) + 4 * g + (r & 3);
                    Vt[d * CVSTR + col] = (uint16_t)(pack_bf16(acc[r], 0.0f) & 0xffffu);
                }
            }
        }
        __syncthreads();
    }

    // ---- stream 32-query blocks
    const int64_t nrows = rend - rbeg;
    const int nqb = (int)((nrows + 31) / 32);
    uint4 qn[8];
    auto load_q = [&](int b, uint4 (&dst)[8]) {
        const int64_t row = rbeg + 32 * b + l32;
        const uint4* src = reinterpret_cast<const uint4*>(q + (row * H + head) * D);
        const bool ok = row < rend;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) dst[kk] = ok ? src[2 * kk + g] : make_uint4(0, 0, 0, 0);
    };
    int b = wave;
    if (b < nqb) load_q(b, qn);
    for (; b < nqb; b += CAM_WAVES) {
        // keep the Kc / Vc^T operand reads inside the loop (re-read from LDS
        // per block) instead of letting them be hoisted into registers
        __asm__ volatile("" ::: "memory");
        cbf16x8 qf[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qf[kk] = __builtin_bit_cast(cbf16x8, cu32x4{qn[kk].x, qn[kk].y, qn[kk].z, qn[kk].w});
        if (b + CAM_WAVES < nqb) load_q(b + CAM_WAVES, qn);

        // online softmax over the 32-key blocks of the camera tokens
        cf32x16 o[4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
        float m = -INFINITY, lsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            cf32x16 s;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const cbf16x8 ka = *reinterpret_cast<const cbf16x8*>(Kc + (32 * kb + l32) * CKSTR + 16 * kk + 8 * g);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s, 0, 0, 0);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
                if (key >= Nc) s[r] = -INFINITY;
                mx = fmaxf(mx, s[r]);
            }
            mx = half_max(mx);
            const float mn = mx * scale_log2;
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
            uint32_t pk[8];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, nm));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], scale_log2, nm));
                lsum += p0 + p1;
                pk[r >> 1] = pack_bf16(p0, p1);
            }
            const cbf16x8 p0 = __builtin_bit_cast(cbf16x8, cu32x4{pk[0], pk[1], pk[2], pk[3]});
            const cbf16x8 p1 = __builtin_bit_cast(cbf16x8, cu32x4{pk[4], pk[5], pk[6], pk[7]});
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const uint16_t* vrow = Vt + (32 * db + l32) * CVSTR + 32 * kb + 8 * g;
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const cbf16x8*>(vrow), p0, o[db], 0, 0, 0);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const cbf16x8*>(vrow + 16), p1, o[db], 0, 0, 0);
            }
        }
        lsum = half_sum(lsum);
        const float inv = 1.0f / lsum;
        const int64_t row = rbeg + 32 * b + l32;
        if (row < rend) {
            uint16_t* dst = out + (row * H + head) * D;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<uint2*>(dst + 32 * db + 8 * i + 4 * g) =
                        make_uint2(pack_bf16(o[db][4 * i] * inv, o[db][4 * i + 1] * inv),
                                   pack_bf16(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv));
        }
    }
}

int launch_cam_xattn(const uint16_t* q, int64_t Lq, int H, const float* cam, int Nc, const uint16_t* wk,
                     const uint16_t* wv, float sm_scale, uint16_t* out, hipStream_t stream) {
    const int nblk = (int)((Lq + CAM_ROWS - 1) / CAM_ROWS);
    const dim3 grid((unsigned)((int64_t)nblk * H)), block(512);
    const float c = (float)((double)sm_scale * 1.4426950408889634);
    const int nkb = (Nc + 31) / 32;
    switch (nkb) {
        case 1: hipLaunchKernelGGL(cam_xattn_kernel<1>, grid, block, 0, stream, q, Lq, H, cam, Nc, wk, wv, c, out, nblk); break;
        case 2: hipLaunchKernelGGL(cam_xattn_kernel<2>, grid, block, 0, stream, q, Lq, H, cam, Nc, wk, wv, c, out, nblk); break;
        case 3: hipLaunchKernelGGL(cam_xattn_kernel<3>, grid, block, 0, stream, q, Lq, H, cam, Nc, wk, wv, c, out, nblk); break;
        case 4: hipLaunchKernelGGL(cam_xattn_kernel<4>, grid, block, 0, stream, q, Lq, H, cam, Nc, wk, wv, c, out, nblk); break;
        default: return NOMAS_EUNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? NOMAS_OK : NOMAS_EHIP;
}

}  // namespace nomas
