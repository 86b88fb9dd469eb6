// Per-device RoPE cos/sin tables (3D RoPE, axes [16, 56, 56], theta 256:
// comfyui-wiki news page on Hy-Nomas, section 模型内部).
//
// The tables live in static device arrays of this code object, so building
// them allocates nothing: the first call on a device computes them on the host
// in float64 (libm cos/sin of p * 256^(-2i/d)) and copies them in; float32
// entries are the float64 values rounded once.
#include <cmath>
#include <mutex>
#include <vector>

#include "common.hpp"

namespace nomas {

__device__ __attribute__((aligned(16))) float2 g_rope32[ROPE_N];
__device__ __attribute__((aligned(16))) double2 g_rope64[ROPE_N];

double rope_angle(int p, int i, int d) {
    double omega = std::pow(256.0, -2.0 * (double)i / (double)d);
    return (double)p * omega;
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
bool g_ready[kMaxDevices];
RopeTables g_tabs[kMaxDevices];

template <typename V2, typename S>
std::vector<V2> host_table(int npos, int npair, int d) {
    std::vector<V2> v((size_t)npos * npair);
    for (int p = 0; p < npos; ++p)
        for (int i = 0; i < npair; ++i) {
            double a = rope_angle(p, i, d);
            v[(size_t)p * npair + i].x = (S)std::cos(a);
            v[(size_t)p * npair + i].y = (S)std::sin(a);
        }
    return v;
}

template <typename T>
bool upload(const T& sym, const void* src, size_t bytes, const void** addr) {
    if (hipMemcpyToSymbol(HIP_SYMBOL(sym), src, bytes, 0, hipMemcpyHostToDevice) != hipSuccess) return false;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(sym)) != hipSuccess) return false;
    *addr = p;
    return true;
}

}  // namespace

void rope_tables_forget() {
    std::lock_guard<std::mutex> lk(g_mu);
    for (int d = 0; d < kMaxDevices; ++d) g_ready[d] = false;
}

int rope_tables(RopeTables* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NOMAS_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ready[dev]) {
        auto t32 = host_table<float2, float>(NOMAS_MAX_T, NPAIR_T, 16);
        auto h32 = host_table<float2, float>(NOMAS_MAX_HW, NPAIR_HW, 56);
        auto t64 = host_table<double2, double>(NOMAS_MAX_T, NPAIR_T, 16);
        auto h64 = host_table<double2, double>(NOMAS_MAX_HW, NPAIR_HW, 56);
        std::vector<float2> all32;
        std::vector<double2> all64;
        all32.reserve(ROPE_N);
        all64.reserve(ROPE_N);
        all32.insert(all32.end(), t32.begin(), t32.end());
        all32.insert(all32.end(), h32.begin(), h32.end());   // h
        all32.insert(all32.end(), h32.begin(), h32.end());   // w (same widths and frequencies)
        all64.insert(all64.end(), t64.begin(), t64.end());
        all64.insert(all64.end(), h64.begin(), h64.end());
        all64.insert(all64.end(), h64.begin(), h64.end());
        const void* a[2];
        if (!upload(g_rope32, all32.data(), all32.size() * sizeof(float2), &a[0]) ||
            !upload(g_rope64, all64.data(), all64.size() * sizeof(double2), &a[1]))
            return NOMAS_EHIP;
        RopeTables r{};
        r.f32 = (const float2*)a[0];
        r.f64 = (const double2*)a[1];
        g_tabs[dev] = r;
        g_ready[dev] = true;
    }
    *out = g_tabs[dev];
    return NOMAS_OK;
}

}  // namespace nomas
