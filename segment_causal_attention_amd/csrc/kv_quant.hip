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

__global__ __launch_bounds__(256) void kv_quant_append_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, int64_t rows_per_tensor, int H,
    int8_t* __restrict__ kc, int8_t* __restrict__ vc, float* __restrict__ ks, float* __restrict__ vs,
    int64_t cap, int64_t len) {
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int lane = threadIdx.x & 15;
    if (row >= 2 * rows_per_tensor) return;     // uniform across the 16 lanes of a row
    const bool is_v = row >= rows_per_tensor;
    const int64_t r = is_v ? row - rows_per_tensor : row;   // token * H + head
    const int64_t tok = r / H;
    const int head = (int)(r - tok * H);

    uint4 w = (is_v ? v : k)[r * 16 + lane];
    float x[8] = {bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y),
                  bf16lo(w.z), bf16hi(w.z), bf16lo(w.w), bf16hi(w.w)};
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
    int8_t* codes = is_v ? vc : kc;
    *reinterpret_cast<uint2*>(codes + dst * D + lane * 8) = make_uint2(packed[0], packed[1]);
    if (lane == 0) (is_v ? vs : ks)[dst] = (a > 0.0f) ? s : 0.0f;
}

int launch_kv_quant_append(const uint16_t* k_rot, const uint16_t* v, int64_t L, int H,
                           int8_t* k_codes, int8_t* v_codes, float* k_scale, float* v_scale,
                           int64_t cap, int64_t len, hipStream_t stream) {
    const int64_t rows = L * H;
    const int64_t blocks = (2 * rows + 15) / 16;
    hipLaunchKernelGGL(kv_quant_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(k_rot), reinterpret_cast<const uint4*>(v), rows, H,
                       k_codes, v_codes, k_scale, v_scale, cap, len);
    return hipGetLastError() == hipSuccess ? NOMAS_OK : NOMAS_EHIP;
}

}  // namespace nomas
