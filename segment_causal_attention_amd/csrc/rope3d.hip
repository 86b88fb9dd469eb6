// Standalone 3D RoPE (comfyui-wiki news page on Hy-Nomas, section 模型内部:
// 3D RoPE, axis sizes [16, 56, 56], theta 256), used on a segment's keys
// before they are quantised into the cache.
//
// HBM-bound (4 B per element moved).  16 lanes own one (token, head) row,
// 8 channels (4 pairs) each.  The rotation is evaluated in float64 from the
// float64 table with separately rounded products (no fma contraction), and
// the float64 result is rounded once to bf16: truncating to float32 and
// setting the sticky bit when inexact (round-to-odd) keeps the final
// round-to-nearest-even to bf16 exact.
#include "common.hpp"

namespace nomas {

__device__ __forceinline__ uint32_t f64_to_bf16(double d) {
    float f = __double2float_rz(d);
    uint32_t b = __float_as_uint(f);
    if ((double)f != d) b |= 1u;
    b += 0x7fffu + ((b >> 16) & 1u);
    return b >> 16;
}

__device__ __forceinline__ uint32_t rot_pair_f64(uint32_t in, double2 cs) {
#pragma clang fp contract(off)
    double x0 = (double)bf16lo(in), x1 = (double)bf16hi(in);
    double y0 = x0 * cs.x - x1 * cs.y;
    double y1 = x0 * cs.y + x1 * cs.x;
    return f64_to_bf16(y0) | (f64_to_bf16(y1) << 16);
}

__global__ __launch_bounds__(256) void rope3d_kernel(const uint4* __restrict__ x, uint4* __restrict__ y,
                                                     int64_t rows, int H, const SegTable st,
                                                     const RopeTables rt) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = idx >> 4;
    if (row >= rows) return;
    const int grp = (int)(idx & 15);
    const int tok = (int)(row / H);
    uint4 w = x[idx];
    int t, h, ww;
    if (token_pos(st, tok, t, h, ww)) {
        const double2* tab = rt.f64 + rope_entry(grp, t, h, ww);
        w.x = rot_pair_f64(w.x, tab[0]);
        w.y = rot_pair_f64(w.y, tab[1]);
        w.z = rot_pair_f64(w.z, tab[2]);
        w.w = rot_pair_f64(w.w, tab[3]);
    }
    y[idx] = w;
}

int launch_rope3d(const uint16_t* x, uint16_t* y, int64_t L, int H, const SegTable& st,
                  const RopeTables& rt, hipStream_t stream) {
    const int64_t rows = L * H;
    const int64_t blocks = (rows * 16 + 255) / 256;
    hipLaunchKernelGGL(rope3d_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(x), reinterpret_cast<uint4*>(y), rows, H, st, rt);
    return hipGetLastError() == hipSuccess ? NOMAS_OK : NOMAS_EHIP;
}

}  // namespace nomas
