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
// scores need only Nc <= 128 keys.  Two kernels.
//  - cam_proj_kernel, one workgroup per head, builds the head's image in the
//    caller's workspace: Kc ([key][d]) then Vc^T ([d][key], keys permuted
//    per 16 as in the attention kernel), laid out byte for byte as the
//    stream kernel keeps them in LDS, keys past Nc zero.  The projections run
//    on MFMA, Kc^T (d x keys) = Wk_h^T (d x 64) . bf16(cam)^T (64 x keys),
//    through a transposed copy of the head's weights in LDS.
//  - cam_xattn_kernel streams the queries: a workgroup (8 waves) owns 256
//    rows of one head, one 32-row block per wave, and the grid takes the
//    heads of a row range next to one another, so the workgroups in flight
//    read whole 4 KB token rows ([L][H][128]) rather than one head's 256 B
//    slices 4 KB apart.  Each wave issues its query loads before the head's
//    image is copied from L2 into LDS, then S^T = Kc . Q^T and
//    O^T = Vc^T . P^T on v_mfma_f32_32x32x16_bf16 with the query as the
//    accumulator lane.  All Nc scores of a row fit in registers, so the
//    softmax takes the exact row maximum first (no running rescale); O^T is
//    formed and stored in two halves of 64 channels (86 VGPRs at 72 camera
//    tokens, five waves per SIMD).
#include "common.hpp"

namespace nomas {

typedef __bf16 cbf16x8 __attribute__((ext_vector_type(8)));
typedef float cf32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t cu32x4 __attribute__((ext_vector_type(4)));

constexpr int CAM_WAVES = 8;
constexpr int CAM_ROWS = 32 * CAM_WAVES;    // query rows per stream workgroup: one 32-row block per wave
constexpr int CAM_MAXK = NOMAS_MAX_CAM;     // 128 keys at most
constexpr int CKSTR = D + 8;                // Kc row stride (bf16)
constexpr int CWSTR = 64 + 8;               // W^T row stride (bf16)

// Vc^T row stride (bf16) for nkb 32-key blocks, and the bf16 elements of one
// head's image: Kc rows, then Vc^T rows
__host__ __device__ constexpr int cam_vstr(int nkb) { return 32 * nkb + 8; }
__host__ __device__ constexpr int cam_img_elems(int nkb) { return 32 * nkb * CKSTR + D * cam_vstr(nkb); }

__device__ __forceinline__ int cvperm(int k) {
    int w = k & 15;
    int p = (w >= 4 && w < 8) ? w + 4 : (w >= 8 && w < 12) ? w - 4 : w;
    return (k & ~15) + p;
}

// ---------------------------------------------------------------------------
// projections: one workgroup per head

template <int NKB>
__global__ __launch_bounds__(512) void cam_proj_kernel(int H, const float* __restrict__ cam, int Nc,
                                                       const uint16_t* __restrict__ wk,
                                                       const uint16_t* __restrict__ wv, uint16_t* __restrict__ imgs) {
    constexpr int IMG = cam_img_elems(NKB);
    constexpr int CVSTR = cam_vstr(NKB);
    __shared__ __attribute__((aligned(16))) uint16_t img[IMG];
    __shared__ __attribute__((aligned(16))) uint16_t Wt[D * CWSTR];
    uint16_t* Kc = img;
    uint16_t* Vt = img + 32 * NKB * CKSTR;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int head = blockIdx.x;
    for (int i = tid; i < IMG / 8; i += 512) reinterpret_cast<uint4*>(img)[i] = make_uint4(0, 0, 0, 0);

    // K first, then V, through the transposed weight tile
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
    uint4* dst = reinterpret_cast<uint4*>(imgs + (int64_t)head * IMG);
    for (int i = tid; i < IMG / 8; i += 512) dst[i] = reinterpret_cast<const uint4*>(img)[i];
}

// ---------------------------------------------------------------------------
// query stream: one workgroup = 256 rows of one head, one 32-row block per wave

// One 32-query block against the image in LDS: S^T for every 32-key block
// (lane = query l32, register r of block kb = key 32kb + 8(r/4) + 4g + r%4),
// the exact row maximum, probabilities, O^T = Vc^T . P^T in two halves of 64
// channels, each normalised and stored as soon as it is done.
template <int NKB>
__device__ __forceinline__ void cam_block(const uint4 (&qn)[8], const uint16_t* Kc, const uint16_t* Vt, int Nc,
                                          float scale_log2, int g, int l32, uint16_t* dst, bool ok) {
    constexpr int CVSTR = cam_vstr(NKB);
    cf32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const cbf16x8 qf = __builtin_bit_cast(cbf16x8, cu32x4{qn[kk].x, qn[kk].y, qn[kk].z, qn[kk].w});
            const cbf16x8 ka = *reinterpret_cast<const cbf16x8*>(Kc + (32 * kb + l32) * CKSTR + 16 * kk + 8 * g);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf, s[kb], 0, 0, 0);
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= Nc) s[kb][r] = -INFINITY;
            mx = fmaxf(mx, s[kb][r]);
        }
    const float nm = -half_max(mx) * scale_log2;
    // probabilities as bf16 pairs; row sum of the fp32 values
    uint32_t pk[NKB][8];
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], scale_log2, nm));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], scale_log2, nm));
            lsum += p0 + p1;
            pk[kb][r >> 1] = pack_bf16(p0, p1);
        }
    const float inv = 1.0f / half_sum(lsum);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        cf32x16 o[2];
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[d2][r] = 0.0f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const cbf16x8 p0 = __builtin_bit_cast(cbf16x8, cu32x4{pk[kb][0], pk[kb][1], pk[kb][2], pk[kb][3]});
            const cbf16x8 p1 = __builtin_bit_cast(cbf16x8, cu32x4{pk[kb][4], pk[kb][5], pk[kb][6], pk[kb][7]});
#pragma unroll
            for (int d2 = 0; d2 < 2; ++d2) {
                const uint16_t* vrow = Vt + (32 * (2 * half + d2) + l32) * CVSTR + 32 * kb + 8 * g;
                o[d2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const cbf16x8*>(vrow), p0, o[d2], 0, 0, 0);
                o[d2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const cbf16x8*>(vrow + 16), p1, o[d2], 0, 0, 0);
            }
        }
        if (ok) {
#pragma unroll
            for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<uint2*>(dst + 32 * (2 * half + d2) + 8 * i + 4 * g) =
                        make_uint2(pack_bf16(o[d2][4 * i] * inv, o[d2][4 * i + 1] * inv),
                                   pack_bf16(o[d2][4 * i + 2] * inv, o[d2][4 * i + 3] * inv));
        }
    }
}

template <int NKB>
__global__ __launch_bounds__(512) void cam_xattn_kernel(const uint16_t* __restrict__ q, int64_t Lq, int H,
                                                        int Nc, const uint16_t* __restrict__ imgs,
                                                        float scale_log2, uint16_t* __restrict__ out) {
    constexpr int IMG = cam_img_elems(NKB);
    constexpr int CHUNKS = IMG / 8;                       // 16-byte chunks of the image
    constexpr int CPT = (CHUNKS + 511) / 512;             // chunks per thread
    __shared__ __attribute__((aligned(16))) uint16_t img[IMG];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    // row range first, head fastest
    const int rblk = blockIdx.x / H;
    const int head = blockIdx.x - rblk * H;
    // this lane's query row (channels 16kk + 8g .. +8), in flight first
    const int64_t row = (int64_t)rblk * CAM_ROWS + 32 * wave + l32;
    const bool ok = row < Lq;
    uint4 qn[8];
    {
        const uint4* src = reinterpret_cast<const uint4*>(q + (row * H + head) * D);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qn[kk] = ok ? src[2 * kk + g] : make_uint4(0, 0, 0, 0);
    }
    // the head's image, from L2 into LDS
    {
        const uint4* src = reinterpret_cast<const uint4*>(imgs + (int64_t)head * IMG);
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int i = tid + 512 * k;
            if (i < CHUNKS) reinterpret_cast<uint4*>(img)[i] = src[i];
        }
    }
    __syncthreads();
    cam_block<NKB>(qn, img, img + 32 * NKB * CKSTR, Nc, scale_log2, g, l32, out + (row * H + head) * D, ok);
}

int64_t cam_xattn_workspace_bytes(int H, int Nc) {
    const int nkb = (Nc + 31) / 32;
    return (int64_t)H * cam_img_elems(nkb) * 2;
}

template <int NKB>
static void launch_cam(const uint16_t* q, int64_t Lq, int H, const float* cam, int Nc, const uint16_t* wk,
                       const uint16_t* wv, float c, uint16_t* out, uint16_t* imgs, hipStream_t stream) {
    hipLaunchKernelGGL(cam_proj_kernel<NKB>, dim3((unsigned)H), dim3(512), 0, stream, H, cam, Nc, wk, wv, imgs);
    const int64_t nrb = (Lq + CAM_ROWS - 1) / CAM_ROWS;
    hipLaunchKernelGGL(cam_xattn_kernel<NKB>, dim3((unsigned)(nrb * H)), dim3(512), 0, stream, q, Lq, H, Nc, imgs, c,
                       out);
}

int launch_cam_xattn(const uint16_t* q, int64_t Lq, int H, const float* cam, int Nc, const uint16_t* wk,
                     const uint16_t* wv, float sm_scale, uint16_t* out, void* workspace, hipStream_t stream) {
    const float c = (float)((double)sm_scale * 1.4426950408889634);
    uint16_t* imgs = static_cast<uint16_t*>(workspace);
    switch ((Nc + 31) / 32) {
        case 1: launch_cam<1>(q, Lq, H, cam, Nc, wk, wv, c, out, imgs, stream); break;
        case 2: launch_cam<2>(q, Lq, H, cam, Nc, wk, wv, c, out, imgs, stream); break;
        case 3: launch_cam<3>(q, Lq, H, cam, Nc, wk, wv, c, out, imgs, stream); break;
        case 4: launch_cam<4>(q, Lq, H, cam, Nc, wk, wv, c, out, imgs, stream); break;
        default: return NOMAS_EUNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? NOMAS_OK : NOMAS_EHIP;
}

}  // namespace nomas
