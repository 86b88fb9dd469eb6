// Standalone 3D RoPE (comfyui-wiki news page on Hy-Nomas, section 模型内部:
// 3D RoPE, axis sizes [16, 56, 56], theta 256), used on a segment's keys
// before they are quantised into the cache.
//
// HBM-bound (4 B per element moved).  16 lanes own one (token, head) row,
// 8 channels (4 pairs) each, rotated by rope_chunk_f64 (float64, rounded
// once to bf16).
#include "common.hpp"

namespace nomas {

__global__ __launch_bounds__(256) void rope3d_kernel(const uint4* __restrict__ x, uint4* __restrict__ y,
                                                     int64_t rows, int H, const SegTable st,
                                                     const RopeTables rt) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = idx >> 4;
    if (row >= rows) return;
    const int grp = (int)(idx & 15);
    const int tok = (int)(row / H);
    y[idx] = rope_chunk_f64(x[idx], grp, tok, st, rt);
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
