// Host-side checks of the libnomas C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of the ABI layer (api.hip,
// rope_tables.hip).  Every call here either needs no GPU (table, camera
// tokens, workspace sizes) or is rejected by the argument checks before
// anything reaches a device, so the program runs on a machine without one.
//
// Inputs are heap arrays of exactly the documented length, so a read past
// their end is an ASan report; outputs carry a canary tail after the
// documented length, so a write past it shows even where ASan's redzone
// would not.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <memory>
#include <vector>

#include "nomas.h"

namespace {

int g_fail = 0;
#define EXPECT(c)                                                                  \
    do {                                                                           \
        if (!(c)) {                                                                \
            std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);      \
            ++g_fail;                                                              \
        }                                                                          \
    } while (0)

void* const FAKE = reinterpret_cast<void*>(0x10000);     // aligned, never dereferenced
void* const MISAL = reinterpret_cast<void*>(0x10002);

template <class T>
std::unique_ptr<T[]> exact(size_t n) { return std::unique_ptr<T[]>(new T[n == 0 ? 1 : n]()); }

// n elements followed by a canary tail
template <class T>
struct Guarded {
    static constexpr size_t kPad = 64;
    std::vector<unsigned char> raw;
    size_t n;
    explicit Guarded(size_t n_) : raw((n_ + kPad) * sizeof(T), 0xA5), n(n_) {}
    T* data() { return reinterpret_cast<T*>(raw.data()); }
    bool intact() const {
        for (size_t i = n * sizeof(T); i < raw.size(); ++i)
            if (raw[i] != 0xA5) return false;
        return true;
    }
};

std::unique_ptr<nomas_seg[]> segs_of(const std::vector<nomas_seg>& v) {
    auto a = exact<nomas_seg>(v.size());
    for (size_t i = 0; i < v.size(); ++i) a[i] = v[i];
    return a;
}

void check_messages() {
    for (int c = -8; c <= 4; ++c) {
        const char* s = nomas_strerror(c);
        EXPECT(s != nullptr && std::strlen(s) > 0);
    }
    EXPECT(std::strstr(nomas_version(), "gfx950") != nullptr);
    EXPECT(nomas_shutdown() == NOMAS_OK && nomas_shutdown() == NOMAS_OK);
}

void check_rope_table() {
    const int npos_max[3] = {NOMAS_MAX_T, NOMAS_MAX_HW, NOMAS_MAX_HW};
    for (int axis = 0; axis < 3; ++axis) {
        const int half = axis == 0 ? 8 : 28;
        for (int npos : {0, 1, 7, npos_max[axis]}) {
            Guarded<float> c((size_t)npos * half), s((size_t)npos * half);
            EXPECT(nomas_rope_table(axis, npos, c.data(), s.data()) == NOMAS_OK);
            EXPECT(c.intact() && s.intact());
            for (size_t i = 0; i < c.n; i += 97) {
                const double r = (double)c.data()[i] * c.data()[i] + (double)s.data()[i] * s.data()[i];
                EXPECT(std::fabs(r - 1.0) < 1e-6);
            }
        }
        Guarded<float> c(8), s(8);
        EXPECT(nomas_rope_table(axis, npos_max[axis] + 1, c.data(), s.data()) == NOMAS_EUNSUPPORTED);
        EXPECT(nomas_rope_table(axis, -1, c.data(), s.data()) == NOMAS_EINVAL);
        EXPECT(nomas_rope_table(axis, 1, nullptr, s.data()) == NOMAS_EINVAL);
        EXPECT(c.intact() && s.intact());
    }
    float c[8], s[8];
    EXPECT(nomas_rope_table(3, 1, c, s) == NOMAS_EINVAL);
    EXPECT(nomas_rope_table(-1, 1, c, s) == NOMAS_EINVAL);
}

// c2w of a rotation by `ang` about a unit axis, translated by t
void pose(double* m, const double a[3], double ang, const double t[3]) {
    const double x = a[0], y = a[1], z = a[2], c = std::cos(ang), s = std::sin(ang), k = 1.0 - c;
    const double R[9] = {c + k * x * x, k * x * y - s * z, k * x * z + s * y,
                         k * x * y + s * z, c + k * y * y, k * y * z - s * x,
                         k * x * z - s * y, k * y * z + s * x, c + k * z * z};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 3; ++j) m[4 * i + j] = R[3 * i + j];
        m[4 * i + 3] = t[i];
    }
    m[12] = m[13] = m[14] = 0.0;
    m[15] = 1.0;
}

void check_cam_tokens() {
    const double axis[3] = {0.3 / 1.0488088481701516, -0.8 / 1.0488088481701516, 0.5 / 1.0488088481701516};
    for (int n : {4, 8, 288}) {
        auto c2w = exact<double>((size_t)n * 16);
        for (int k = 0; k < n; ++k) {
            const double t[3] = {0.1 * k, -0.2 * k, 0.05 * k * k};
            // angles through a right angle up to just short of a half turn
            pose(c2w.get() + 16 * k, axis, 3.14159265358979 * k / n, t);
        }
        Guarded<float> tok((size_t)n / 4 * 64);
        EXPECT(nomas_cam_tokens(c2w.get(), n, 1.0, 2.5, tok.data()) == NOMAS_OK);
        EXPECT(tok.intact());
        for (int k = 0; k < n; ++k) {
            const float* o = tok.data() + 16 * k;
            EXPECT(o[12] == 0.0f && o[13] == 0.0f && o[14] == 0.0f && o[15] == 1.0f);
            for (int i = 0; i < 12; ++i) EXPECT(std::isfinite(o[i]));
        }
    }
    auto c2w = exact<double>(6 * 16);
    Guarded<float> tok(64);
    EXPECT(nomas_cam_tokens(c2w.get(), 6, 1.0, 2.5, tok.data()) == NOMAS_EINVAL);
    EXPECT(nomas_cam_tokens(c2w.get(), 0, 1.0, 2.5, tok.data()) == NOMAS_EINVAL);
    EXPECT(nomas_cam_tokens(c2w.get(), 4, NAN, 2.5, tok.data()) == NOMAS_EINVAL);
    EXPECT(nomas_cam_tokens(c2w.get(), 4, 1.0, INFINITY, tok.data()) == NOMAS_EINVAL);
    EXPECT(nomas_cam_tokens(nullptr, 4, 1.0, 2.5, tok.data()) == NOMAS_EINVAL);
    EXPECT(tok.intact());
}

void check_workspace_sizes() {
    // 1..64 segments read from an array of exactly that length
    for (int n : {1, 2, 17, NOMAS_MAX_SEGS}) {
        std::vector<nomas_seg> v;
        for (int i = 0; i < n; ++i) v.push_back({i % 3, i, i % 2 ? 1 : 0, 3, 5});
        auto a = segs_of(v);
        for (int split : {0, 1, 4}) {
            const int64_t b = nomas_seg_attn_workspace(a.get(), n, 1000, 3, split);
            EXPECT(b > 0 && b % 16 == 0);
        }
        // segment 0 is empty (no tokens, no tiles); any other segment adds tiles
        EXPECT(n == 1 ? nomas_seg_attn_bwd_workspace(a.get(), n, 2) == 0 : nomas_seg_attn_bwd_workspace(a.get(), n, 2) > 0);
        // a selection: one range per segment, arrays of exactly n + 1 offsets and 2n bounds
        auto off = exact<int32_t>(n + 1);
        auto rng = exact<int64_t>(2 * (size_t)n);
        for (int i = 0; i <= n; ++i) off[i] = i;
        for (int i = 0; i < n; ++i) { rng[2 * i] = 10 * i; rng[2 * i + 1] = 10 * i + 5; }
        EXPECT(nomas_seg_attn_sel_workspace(a.get(), n, 1000, off.get(), rng.get(), 3, 1) > 0);
        rng[2 * (n - 1) + 1] = 1001;      // past the cache
        EXPECT(nomas_seg_attn_sel_workspace(a.get(), n, 1000, off.get(), rng.get(), 3, 1) == NOMAS_EINVAL);
    }
    std::vector<nomas_seg> many(NOMAS_MAX_SEGS + 1, nomas_seg{1, 0, 0, 0, 0});
    auto m = segs_of(many);
    EXPECT(nomas_seg_attn_workspace(m.get(), NOMAS_MAX_SEGS + 1, 0, 1, 1) == NOMAS_EUNSUPPORTED);
    auto one = segs_of({{16, 0, 2, 4, 6}});
    EXPECT(nomas_seg_attn_workspace(one.get(), 1, -1, 3, 1) == NOMAS_EINVAL);
    EXPECT(nomas_seg_attn_workspace(one.get(), 1, 0, 0, 1) == NOMAS_EINVAL);
    EXPECT(nomas_seg_attn_workspace(one.get(), 1, 0, 2, NOMAS_MAX_SPLIT + 1) == NOMAS_EUNSUPPORTED);
    EXPECT(nomas_seg_attn_workspace(nullptr, 1, 0, 2, 1) == NOMAS_EINVAL);
    auto bad = segs_of({{-1, 0, 0, 0, 0}});
    EXPECT(nomas_seg_attn_workspace(bad.get(), 1, 0, 2, 1) == NOMAS_EINVAL);
    auto late = segs_of({{0, NOMAS_MAX_T - 1, 2, 4, 4}});
    EXPECT(nomas_seg_attn_workspace(late.get(), 1, 0, 2, 1) == NOMAS_EUNSUPPORTED);
    EXPECT(nomas_gqa_attn_workspace(100, 4, 2) > 0);
    EXPECT(nomas_gqa_attn_workspace(100, 4, 3) == NOMAS_EINVAL);
    EXPECT(nomas_w8a16_linear_workspace(2048, 8192) == (int64_t)2048 * 8192 * 2);
    EXPECT(nomas_w8a16_linear_workspace(2000, 8192) == NOMAS_EUNSUPPORTED);
}

void check_rejected_calls() {
    auto seg = segs_of({{16, 0, 2, 4, 6}});     // 64 tokens
    nomas_bf16* const F = static_cast<nomas_bf16*>(FAKE);
    nomas_bf16* const M = static_cast<nomas_bf16*>(MISAL);
    // rope3d
    EXPECT(nomas_rope3d(nullptr, F, seg.get(), 1, 2, nullptr) == NOMAS_EINVAL);
    EXPECT(nomas_rope3d(F, M, seg.get(), 1, 2, nullptr) == NOMAS_EINVAL);
    EXPECT(nomas_rope3d(F, F, seg.get(), 1, 0, nullptr) == NOMAS_EINVAL);
    EXPECT(nomas_rope3d(F, F, nullptr, 1, 2, nullptr) == NOMAS_EINVAL);
    // kv_quant_append: capacity, length and pointers; len is left as it was
    int8_t* const C = static_cast<int8_t*>(FAKE);
    float* const S = static_cast<float*>(FAKE);
    int64_t len = 90;
    EXPECT(nomas_kv_quant_append(F, F, 11, 2, C, C, S, S, 100, &len, nullptr) == NOMAS_ECAPACITY);
    EXPECT(len == 90);
    EXPECT(nomas_kv_quant_append(F, F, 0, 2, C, C, S, S, 100, &len, nullptr) == NOMAS_OK && len == 90);
    EXPECT(nomas_kv_quant_append(F, F, -1, 2, C, C, S, S, 100, &len, nullptr) == NOMAS_EINVAL);
    EXPECT(nomas_kv_quant_append(F, F, 5, 2, C, C, S, S, 100, nullptr, nullptr) == NOMAS_EINVAL);
    EXPECT(nomas_kv_quant_append(M, F, 5, 2, C, C, S, S, 100, &len, nullptr) == NOMAS_EINVAL);
    EXPECT(nomas_kv_quant_append(F, F, 5, 2, C, C, static_cast<float*>(MISAL), S, 100, &len, nullptr) == NOMAS_EINVAL);
    EXPECT(len == 90);
    // seg_attn: workspace, scale, cache pointers, sizes
    const int64_t need = nomas_seg_attn_workspace(seg.get(), 1, 0, 2, 1);
    EXPECT(need > 0);
    auto call = [&](int64_t clen, int64_t cap, float sm, void* ws, int64_t wsb, int H = 2, int split = 1) {
        return nomas_seg_attn(F, F, F, seg.get(), 1, clen ? C : nullptr, clen ? C : nullptr, clen ? S : nullptr,
                              clen ? S : nullptr, cap, clen, H, sm, F, nullptr, split, ws, wsb, nullptr);
    };
    EXPECT(call(0, 0, 0.088f, FAKE, need - 1) == NOMAS_EINVAL);
    EXPECT(call(0, 0, 0.088f, nullptr, need) == NOMAS_EINVAL);
    EXPECT(call(0, 0, 0.088f, MISAL, need) == NOMAS_EINVAL);
    EXPECT(call(0, 0, 0.0f, FAKE, need) == NOMAS_EINVAL);
    EXPECT(call(0, 0, NAN, FAKE, need) == NOMAS_EINVAL);
    EXPECT(call(5, 4, 0.088f, FAKE, 1 << 30) == NOMAS_EINVAL);                 // cache_len > cap
    EXPECT(call(0, (int64_t)NOMAS_MAX_CACHE + 1, 0.088f, FAKE, need) == NOMAS_EUNSUPPORTED);
    EXPECT(call(0, 0, 0.088f, FAKE, need, 2, NOMAS_MAX_SPLIT + 1) == NOMAS_EUNSUPPORTED);
    // seg_attn_sel: an unsorted selection
    auto off = exact<int32_t>(2);
    auto rng = exact<int64_t>(4);
    off[0] = 0; off[1] = 2;
    rng[0] = 20; rng[1] = 30; rng[2] = 0; rng[3] = 10;
    EXPECT(nomas_seg_attn_sel(F, F, F, seg.get(), 1, C, C, S, S, 100, 100, off.get(), rng.get(), 2, 0.088f, F,
                              nullptr, 1, FAKE, 1 << 30, nullptr) == NOMAS_EINVAL);
    // seg_attn_bwd, gqa_attn, w8a16_linear, cam_xattn
    float* const G = static_cast<float*>(FAKE);
    EXPECT(nomas_seg_attn_bwd(F, F, F, F, nullptr, F, seg.get(), 1, 2, 0.088f, G, G, G, FAKE, 1 << 30, nullptr) ==
           NOMAS_EINVAL);
    EXPECT(nomas_seg_attn_bwd(F, F, F, F, G, F, seg.get(), 1, 2, 0.088f, G, G, G, FAKE, 16, nullptr) == NOMAS_EINVAL);
    EXPECT(nomas_gqa_attn(F, F, F, 100, 4, 3, 0.088f, F, nullptr, FAKE, 1 << 30, nullptr) == NOMAS_EINVAL);
    EXPECT(nomas_w8a16_linear(F, 10, 96, C, S, 256, F, FAKE, 1 << 20, nullptr) == NOMAS_EUNSUPPORTED);
    EXPECT(nomas_w8a16_linear(F, 10, 128, C, S, 256, F, FAKE, 128 * 256 * 2 - 1, nullptr) == NOMAS_EINVAL);
    const int64_t cw = nomas_cam_xattn_workspace(2, 72);
    EXPECT(cw > 0 && nomas_cam_xattn_workspace(2, NOMAS_MAX_CAM + 1) == NOMAS_EUNSUPPORTED);
    EXPECT(nomas_cam_xattn(F, 10, 2, S, NOMAS_MAX_CAM + 1, F, F, 0.088f, F, FAKE, cw, nullptr) == NOMAS_EUNSUPPORTED);
    EXPECT(nomas_cam_xattn(F, 10, 2, S, 0, F, F, 0.088f, F, FAKE, cw, nullptr) == NOMAS_EINVAL);
    EXPECT(nomas_cam_xattn(F, 10, 2, S, 72, F, F, 0.088f, F, FAKE, cw - 1, nullptr) == NOMAS_EINVAL);
    EXPECT(nomas_cam_xattn(F, 10, 2, S, 72, F, F, 0.088f, F, nullptr, cw, nullptr) == NOMAS_EINVAL);
    EXPECT(nomas_cam_xattn(F, 0, 2, S, 4, F, F, 0.088f, F, nullptr, 0, nullptr) == NOMAS_OK);     // nothing to do
}

}  // namespace

int main() {
    check_messages();
    check_rope_table();
    check_cam_tokens();
    check_workspace_sizes();
    check_rejected_calls();
    if (g_fail) {
        std::fprintf(stderr, "%d check(s) failed\n", g_fail);
        return 1;
    }
    std::printf("abi host checks passed\n");
    return 0;
}
