// INT8 quantise-and-append of a segment's K/V into the lifelong cache.
//
// Cached keys and values are stored as INT8 while attention runs in BF16
// (comfyui-wiki news page on Hy-Nomas, section 单张 4090 配置; huaweicloud blog,
// section 3.5 table).  Per (token, head) row of 128 values:
//   a = max|x|, s = fl32(a/127), q = clamp(rne(x/s), -127, 127), a = 0 -> s = q = 0.
//
// HBM-bound: each row is read once (256 B) and written once (128 B + 4 B).
// 16 lanes own one row, 8 channels (16 B) each; the row max is a 16-lane
// butterfly.  rne(x/s) is exact: an fp32 quotient picks a candidate q0, the
// residual r = x - q0*s is exact in one fma (|r| is at most about s/2
// and r is a multiple of ulp(s), so it fits 24 bits), and comparing 2|r| with s fixes
// the at most one-off candidate, ties to even.
#include "common.hpp"

namespace nomas {

__device__ __forceinline__ float quant_code(float x, float s) {
    float q = rintf(x / s);
    float r = fmaf(-q, s, x);
    float r2 = 2.0f * fabsf(r);
    float step = copysignf(1.0f, r);
    if (r2 > s) {
        q += step;
    } else if (r2 == s) {
        float q2 = q + step;
        if (fmodf(q2, 2.0f) == 0.0f) q = q2;
    }
    return fminf(fmaxf(q, -127.0f), 127.0f);
}

constexpr int QT_PASSES = 4;        // 16-token passes per block

// Block = 64 consecutive tokens of one head of K or of V, in passes of 16
// whose loads are all issued first: each pass's codes land as 2 KB of
// contiguous cache rows and its scales as 64 contiguous bytes.  Blocks are
// ordered token range first, then head, then K / V, so the blocks in flight
// together read whole 4 KB token rows ([L][H][128] bf16: every head's 256 B
// slice of a token) rather than one head's slices 4 KB apart.
__global__ __launch_bounds__(256) void kv_quant_append_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, int64_t L, int H, int64_t ntb,
    int8_t* __restrict__ kc, int8_t* __restrict__ vc, float* __restrict__ ks, float* __restrict__ vs,
    int64_t cap, int64_t len) {
    const bool is_v = (blockIdx.x & 1) != 0;
    const int64_t b = blockIdx.x >> 1;
    const int64_t tb = b / H;                  // token range
    const int head = (int)(b - tb * H);
    const int lane = threadIdx.x & 15;
    const int64_t tok0 = tb * QT_PASSES * 16 + (threadIdx.x >> 4);
    const uint4* src = is_v ? v : k;
    uint4 w[QT_PASSES];
#pragma unroll
    for (int p = 0; p < QT_PASSES; ++p) {
        const int64_t tok = tok0 + 16 * p;
        w[p] = tok < L ? src[(tok * H + head) * 16 + lane] : make_uint4(0, 0, 0, 0);
    }
    int8_t* codes = is_v ? vc : kc;
    float* scales = is_v ? vs : ks;
#pragma unroll
    for (int p = 0; p < QT_PASSES; ++p) {
        const int64_t tok = tok0 + 16 * p;
        if (tok >= L) break;    // uniform across the 16 lanes of a row, and later passes are further on
        float x[8] = {bf16lo(w[p].x), bf16hi(w[p].x), bf16lo(w[p].y), bf16hi(w[p].y),
                      bf16lo(w[p].z), bf16hi(w[p].z), bf16lo(w[p].w), bf16hi(w[p].w)};
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) a = fmaxf(a, __shfl_xor(a, m, 16));
        const float s = a / 127.0f;
        uint32_t packed[2] = {0u, 0u};
        if (a > 0.0f) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                int q = (int)quant_code(x[i], s);
                packed[i >> 2] |= ((uint32_t)(q & 0xff)) << (8 * (i & 3));
            }
        }
        const int64_t dst = (int64_t)head * cap + len + tok;
        *reinterpret_cast<uint2*>(codes + dst * D + lane * 8) = make_uint2(packed[0], packed[1]);
        if (lane == 0) scales[dst] = (a > 0.0f) ? s : 0.0f;
    }
}

int launch_kv_quant_append(const uint16_t* k_rot, const uint16_t* v, int64_t L, int H,
                           int8_t* k_codes, int8_t* v_codes, float* k_scale, float* v_scale,
                           int64_t cap, int64_t len, hipStream_t stream) {
    const int64_t ntb = (L + 16 * QT_PASSES - 1) / (16 * QT_PASSES);    // blocks per head
    const int64_t blocks = 2 * (int64_t)H * ntb;
    hipLaunchKernelGGL(kv_quant_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(k_rot), reinterpret_cast<const uint4*>(v), L, H, ntb,
                       k_codes, v_codes, k_scale, v_scale, cap, len);
    return hipGetLastError() == hipSuccess ? NOMAS_OK : NOMAS_EHIP;
}

}  // namespace nomas
