// Standalone 3D RoPE (comfyui-wiki news page on Hy-Nomas, section 模型内部:
// 3D RoPE, axis sizes [16, 56, 56], theta 256), used on a segment's keys
// before they are quantised into the cache.
//
// HBM-bound (4 B per element moved).  One wave per token: lane = (8-channel
// group, head block), so the token's position and each group's float64
// cos/sin entries are looked up once and applied to every head (lanes
// 16b .. 16b+15 take heads b, b+4, ...); each head pass moves 1 KB of
// contiguous rows, and the loads of four passes (16 heads, the whole 4 KB
// token) are issued before any of them is rotated, so a wave keeps 4 KB in
// flight.  The rotation is rope_chunk_f64's (float64, rounded once to bf16).
#include "common.hpp"

namespace nomas {

constexpr int ROPE_NT = 256;        // 4 waves = 4 tokens per block

__global__ __launch_bounds__(ROPE_NT) void rope3d_kernel(const uint4* __restrict__ x, uint4* __restrict__ y,
                                                         int64_t L, int H, const SegTable st, const RopeTables rt) {
    const int64_t tok = (int64_t)blockIdx.x * (ROPE_NT / 64) + (threadIdx.x >> 6);
    if (tok >= L) return;
    const int lane = threadIdx.x & 63, grp = lane & 15;
    int t, h, w;
    const bool video = token_pos(st, (int)tok, t, h, w);
    double2 cs[4] = {};
    if (video) {
        const double2* tab = rt.f64 + rope_entry(grp, t, h, w);
#pragma unroll
        for (int i = 0; i < 4; ++i) cs[i] = tab[i];
    }
    for (int hd0 = lane >> 4; hd0 < H; hd0 += 16) {
        uint4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int hd = hd0 + 4 * j;
            if (hd < H) v[j] = x[(tok * H + hd) * 16 + grp];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int hd = hd0 + 4 * j;
            if (hd >= H) break;
            if (video) {
                v[j].x = rot_pair_f64(v[j].x, cs[0]);
                v[j].y = rot_pair_f64(v[j].y, cs[1]);
                v[j].z = rot_pair_f64(v[j].z, cs[2]);
                v[j].w = rot_pair_f64(v[j].w, cs[3]);
            }
            y[(tok * H + hd) * 16 + grp] = v[j];
        }
    }
}

int launch_rope3d(const uint16_t* x, uint16_t* y, int64_t L, int H, const SegTable& st,
                  const RopeTables& rt, hipStream_t stream) {
    const int64_t blocks = (L + ROPE_NT / 64 - 1) / (ROPE_NT / 64);
    hipLaunchKernelGGL(rope3d_kernel, dim3((unsigned)blocks), dim3(ROPE_NT), 0, stream,
                       reinterpret_cast<const uint4*>(x), reinterpret_cast<uint4*>(y), L, H, st, rt);
    return hipGetLastError() == hipSuccess ? NOMAS_OK : NOMAS_EHIP;
}

}  // namespace nomas
