// extern "C" entry points of libnomas: argument checks, launch planning and
// the host-side camera-token normalisation.  Every check runs before anything
// is enqueued; no entry point allocates device memory per call.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "common.hpp"

namespace nomas {
int launch_kv_quant_append(const uint16_t* k_rot, const uint16_t* v, int64_t L, int H, int8_t* k_codes,
                           int8_t* v_codes, float* k_scale, float* v_scale, int64_t cap, int64_t len,
                           hipStream_t stream);
int launch_rope3d(const uint16_t* x, uint16_t* y, int64_t L, int H, const SegTable& st, const RopeTables& rt,
                  hipStream_t stream);
int launch_seg_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const SegTable& segs, int Ln,
                    const int8_t* kc, const int8_t* vc, const float* ks, const float* vs, int64_t cap, int Lc,
                    const int32_t* sel_off, const int64_t* sel_ranges, int H, int Hkv, float sm_scale,
                    uint16_t* out, float* lse, int n_split, void* workspace, const RopeTables& rt,
                    hipStream_t stream);
int64_t seg_attn_workspace_bytes(const SegTable& segs, int Lc, int Ln, int H, int Hkv, int n_split,
                                 const int32_t* sel_off, const int64_t* sel_ranges);
int launch_w8a16(const uint16_t* x, int64_t M, int64_t K, const int8_t* codes, const float* scale, int64_t N,
                 uint16_t* y, void* workspace, hipStream_t stream);
int64_t w8a16_workspace_bytes(int64_t N, int64_t K);
int w8a16_scratch(void** out);
void w8a16_scratch_forget();
void rope_tables_forget();
int launch_seg_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                        const float* lse, const uint16_t* dout, const SegTable& st, int Ln, int H, float sm_scale,
                        float* dq, float* dk, float* dv, void* workspace, const RopeTables& rt, hipStream_t stream);
int64_t seg_attn_bwd_workspace_bytes(const SegTable& st, int H);
int launch_cam_xattn(const uint16_t* q, int64_t Lq, int H, const float* cam, int Nc, const uint16_t* wk,
                     const uint16_t* wv, float sm_scale, uint16_t* out, void* workspace, hipStream_t stream);
int64_t cam_xattn_workspace_bytes(int H, int Nc);
}  // namespace nomas

using namespace nomas;

namespace {

constexpr int64_t kMaxTokens = (int64_t)1 << 30;   // token counts stay far inside int32 indexing
constexpr int kMaxHeads = 256;

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Descriptor list -> device table.  Returns the total token count in *total.
int build_segs(const nomas_seg* segs, int n, SegTable* st, int64_t* total) {
    if (!segs || n < 1) return NOMAS_EINVAL;
    if (n > NOMAS_MAX_SEGS) return NOMAS_EUNSUPPORTED;
    std::memset(st, 0, sizeof(*st));
    st->n = n;
    int64_t start = 0;
    for (int i = 0; i < n; ++i) {
        const nomas_seg& s = segs[i];
        if (s.n_text < 0 || s.t0 < 0 || s.T < 0 || s.Hg < 0 || s.Wg < 0) return NOMAS_EINVAL;
        if (s.T > 0 && (s.Hg < 1 || s.Wg < 1)) return NOMAS_EINVAL;
        if (s.T > 0 && ((int64_t)s.t0 + s.T > NOMAS_MAX_T || s.Hg > NOMAS_MAX_HW || s.Wg > NOMAS_MAX_HW))
            return NOMAS_EUNSUPPORTED;
        if ((int64_t)s.T * s.Hg * s.Wg >= ((int64_t)1 << 24)) return NOMAS_EUNSUPPORTED;   // float-estimated divisions
        const int64_t ntok = (int64_t)s.n_text + (int64_t)s.T * s.Hg * s.Wg;
        SegDev& d = st->s[i];
        d.start = (int32_t)start;
        d.n_text = s.n_text;
        d.t0 = s.t0;
        d.T = s.T;
        d.Hg = s.T > 0 ? s.Hg : 1;
        d.Wg = s.T > 0 ? s.Wg : 1;
        d.inv_hw = 1.0f / (float)(d.Hg * d.Wg);
        d.inv_w = 1.0f / (float)d.Wg;
        start += ntok;
        if (start > kMaxTokens) return NOMAS_EUNSUPPORTED;
    }
    *total = start;
    return NOMAS_OK;
}

bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }

// --- rotations for the camera tokens (float64, host) -------------------------

void mat3_mul(const double A[9], const double B[9], double C[9]) {
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) C[3 * i + j] = A[3 * i] * B[j] + A[3 * i + 1] * B[3 + j] + A[3 * i + 2] * B[6 + j];
}

// Axis (unit) and angle in [0, pi] of a rotation matrix R = exp(ang [a]x).
// The skew part of R is sin(ang) a; its symmetric part minus cos(ang) I is
// (1 - cos(ang)) a a^T.  Up to a right angle the axis is the normalised skew
// part.  Beyond it the skew part shrinks towards zero at pi, so the axis is
// read from the symmetric part (column of its largest diagonal entry) and
// only its sign from the skew part.  At a half turn +a and -a are the same
// rotation and the skew part is zero up to rounding: where its component
// along the chosen column is no larger than 1e-12 (far above the rounding of
// products of orthonormal double matrices) the largest axis component is
// taken positive.
void rot_log(const double R[9], double axis[3], double* ang) {
    const double v[3] = {0.5 * (R[7] - R[5]), 0.5 * (R[2] - R[6]), 0.5 * (R[3] - R[1])};
    const double s = std::sqrt(v[0] * v[0] + v[1] * v[1] + v[2] * v[2]);
    const double c = 0.5 * (R[0] + R[4] + R[8] - 1.0);
    *ang = std::atan2(s, c);
    if (c >= 0.0) {
        if (s == 0.0) {
            axis[0] = 1.0; axis[1] = 0.0; axis[2] = 0.0;
            *ang = 0.0;
        } else {
            for (int i = 0; i < 3; ++i) axis[i] = v[i] / s;
        }
        return;
    }
    // A = (sym(R) - c I) / (1 - c) = a a^T
    double A[9];
    for (int r = 0; r < 3; ++r)
        for (int k = 0; k < 3; ++k)
            A[3 * r + k] = (0.5 * (R[3 * r + k] + R[3 * k + r]) - (r == k ? c : 0.0)) / (1.0 - c);
    int j = 0;
    if (A[4] > A[0]) j = 1;
    if (A[8] > A[4 * j]) j = 2;
    const double d = std::sqrt(A[4 * j]);           // >= 1/sqrt(3) for a unit axis
    double a[3] = {A[j] / d, A[3 + j] / d, A[6 + j] / d};
    if (v[j] < -1e-12)
        for (int i = 0; i < 3; ++i) a[i] = -a[i];
    const double n = std::sqrt(a[0] * a[0] + a[1] * a[1] + a[2] * a[2]);
    for (int i = 0; i < 3; ++i) axis[i] = a[i] / n;
}

void rot_exp(const double axis[3], double ang, double R[9]) {
    const double x = axis[0], y = axis[1], z = axis[2];
    const double K[9] = {0, -z, y, z, 0, -x, -y, x, 0};
    double K2[9];
    mat3_mul(K, K, K2);
    const double s = std::sin(ang), c1 = 1.0 - std::cos(ang);
    for (int i = 0; i < 9; ++i) R[i] = ((i % 4) == 0 ? 1.0 : 0.0) + s * K[i] + c1 * K2[i];
}

}  // namespace

extern "C" {

const char* nomas_strerror(int code) {
    switch (code) {
        case NOMAS_OK: return "ok";
        case NOMAS_EINVAL: return "invalid argument (null or misaligned pointer, bad size or segment descriptor)";
        case NOMAS_ECAPACITY: return "cache capacity exceeded (len + L > cap)";
        case NOMAS_EHIP: return "HIP runtime error (launch or runtime call failed)";
        case NOMAS_EUNSUPPORTED: return "size outside the library's limits";
        default: return "unknown error code";
    }
}

const char* nomas_version(void) { return "nomas 0.1 (gfx950)"; }

int nomas_shutdown(void) {
    rope_tables_forget();
    w8a16_scratch_forget();
    return NOMAS_OK;
}

int nomas_rope_table(int axis, int npos, float* cos_out, float* sin_out) {
    if (axis < 0 || axis > 2 || npos < 0 || !cos_out || !sin_out) return NOMAS_EINVAL;
    if (npos > (axis == 0 ? NOMAS_MAX_T : NOMAS_MAX_HW)) return NOMAS_EUNSUPPORTED;
    const int d = axis == 0 ? 16 : 56;
    for (int p = 0; p < npos; ++p)
        for (int i = 0; i < d / 2; ++i) {
            const double a = rope_angle(p, i, d);
            cos_out[p * (d / 2) + i] = (float)std::cos(a);
            sin_out[p * (d / 2) + i] = (float)std::sin(a);
        }
    return NOMAS_OK;
}

int nomas_rope3d(const nomas_bf16* x, nomas_bf16* y, const nomas_seg* segs, int n_segs, int H, void* stream) {
    if (!x || !y || H < 1 || !al16(x) || !al16(y)) return NOMAS_EINVAL;
    if (H > kMaxHeads) return NOMAS_EUNSUPPORTED;
    SegTable st;
    int64_t L = 0;
    int rc = build_segs(segs, n_segs, &st, &L);
    if (rc != NOMAS_OK) return rc;
    if (L == 0) return NOMAS_OK;
    RopeTables rt;
    if ((rc = rope_tables(&rt)) != NOMAS_OK) return rc;
    return launch_rope3d(x, y, L, H, st, rt, (hipStream_t)stream);
}

int nomas_kv_quant_append(const nomas_bf16* k_rot, const nomas_bf16* v, int64_t L, int H, int8_t* k_codes,
                          int8_t* v_codes, float* k_scale, float* v_scale, int64_t cap, int64_t* len,
                          void* stream) {
    if (!len || L < 0 || H < 1 || cap < 0 || *len < 0 || *len > cap) return NOMAS_EINVAL;
    if (H > kMaxHeads || L > kMaxTokens || cap > kMaxTokens) return NOMAS_EUNSUPPORTED;
    if (L == 0) return NOMAS_OK;
    if (!k_rot || !v || !k_codes || !v_codes || !k_scale || !v_scale) return NOMAS_EINVAL;
    if (!al16(k_rot) || !al16(v) || !al16(k_codes) || !al16(v_codes) || !al4(k_scale) || !al4(v_scale))
        return NOMAS_EINVAL;
    if (*len + L > cap) return NOMAS_ECAPACITY;
    int rc = launch_kv_quant_append(k_rot, v, L, H, k_codes, v_codes, k_scale, v_scale, cap, *len,
                                    (hipStream_t)stream);
    if (rc == NOMAS_OK) *len += L;
    return rc;
}

int64_t nomas_seg_attn_sel_workspace(const nomas_seg* new_segs, int n_new_segs, int64_t cache_len,
                                     const int32_t* sel_off, const int64_t* sel_ranges, int H, int n_split) {
    if (H < 1 || cache_len < 0 || n_split < 0) return NOMAS_EINVAL;
    if (n_split > NOMAS_MAX_SPLIT) return NOMAS_EUNSUPPORTED;
    if (H > kMaxHeads || cache_len > NOMAS_MAX_CACHE) return NOMAS_EUNSUPPORTED;
    SegTable st;
    int64_t Ln = 0;
    int rc = build_segs(new_segs, n_new_segs, &st, &Ln);
    if (rc != NOMAS_OK) return rc;
    if (Ln * H > NOMAS_MAX_TOKEN_HEADS) return NOMAS_EUNSUPPORTED;
    return seg_attn_workspace_bytes(st, (int)cache_len, (int)Ln, H, H, n_split, sel_off, sel_ranges);
}

int64_t nomas_seg_attn_workspace(const nomas_seg* new_segs, int n_new_segs, int64_t cache_len, int H,
                                 int n_split) {
    return nomas_seg_attn_sel_workspace(new_segs, n_new_segs, cache_len, nullptr, nullptr, H, n_split);
}

int nomas_seg_attn_sel(const nomas_bf16* q, const nomas_bf16* k_new, const nomas_bf16* v_new,
                       const nomas_seg* new_segs, int n_new_segs, const int8_t* k_codes, const int8_t* v_codes,
                       const float* k_scale, const float* v_scale, int64_t cap, int64_t cache_len,
                       const int32_t* sel_off, const int64_t* sel_ranges, int H, float sm_scale, nomas_bf16* out,
                       float* lse, int n_split, void* workspace, int64_t workspace_bytes, void* stream) {
    if (!q || !k_new || !v_new || !out || H < 1 || !finite_pos(sm_scale) || n_split < 0) return NOMAS_EINVAL;
    if (n_split > NOMAS_MAX_SPLIT) return NOMAS_EUNSUPPORTED;
    if (!al16(q) || !al16(k_new) || !al16(v_new) || !al16(out) || (lse && !al4(lse))) return NOMAS_EINVAL;
    if (cap < 0 || cache_len < 0 || cache_len > cap) return NOMAS_EINVAL;
    if (H > kMaxHeads || cap > kMaxTokens) return NOMAS_EUNSUPPORTED;
    if (cache_len > 0) {
        if (!k_codes || !v_codes || !k_scale || !v_scale) return NOMAS_EINVAL;
        if (!al16(k_codes) || !al16(v_codes) || !al4(k_scale) || !al4(v_scale)) return NOMAS_EINVAL;
    }
    SegTable st;
    int64_t Ln = 0;
    int rc = build_segs(new_segs, n_new_segs, &st, &Ln);
    if (rc != NOMAS_OK) return rc;
    if (cap > NOMAS_MAX_CACHE || Ln * H > NOMAS_MAX_TOKEN_HEADS) return NOMAS_EUNSUPPORTED;
    // the selection is checked (and the workspace sized) before anything else is looked at on the device
    const int64_t need = seg_attn_workspace_bytes(st, (int)cache_len, (int)Ln, H, H, n_split, sel_off, sel_ranges);
    if (need < 0) return (int)need;
    if (Ln == 0) return NOMAS_OK;
    if (!workspace || !al16(workspace) || workspace_bytes < need) return NOMAS_EINVAL;
    RopeTables rt;
    if ((rc = rope_tables(&rt)) != NOMAS_OK) return rc;
    return launch_seg_attn(q, k_new, v_new, st, (int)Ln, k_codes, v_codes, k_scale, v_scale, cap, (int)cache_len,
                           sel_off, sel_ranges, H, H, sm_scale, out, lse, n_split, workspace, rt,
                           (hipStream_t)stream);
}

int64_t nomas_seg_attn_bwd_workspace(const nomas_seg* segs, int n_segs, int H) {
    if (H < 1) return NOMAS_EINVAL;
    if (H > kMaxHeads) return NOMAS_EUNSUPPORTED;
    SegTable st;
    int64_t Ln = 0;
    const int rc = build_segs(segs, n_segs, &st, &Ln);
    if (rc != NOMAS_OK) return rc;
    if (Ln * H > NOMAS_MAX_TOKEN_HEADS) return NOMAS_EUNSUPPORTED;
    return seg_attn_bwd_workspace_bytes(st, H);
}

int nomas_seg_attn_bwd(const nomas_bf16* q, const nomas_bf16* k, const nomas_bf16* v, const nomas_bf16* out,
                       const float* lse, const nomas_bf16* d_out, const nomas_seg* segs, int n_segs, int H,
                       float sm_scale, float* dq, float* dk, float* dv, void* workspace, int64_t workspace_bytes,
                       void* stream) {
    if (!q || !k || !v || !out || !lse || !d_out || !dq || !dk || !dv) return NOMAS_EINVAL;
    if (H < 1 || !finite_pos(sm_scale)) return NOMAS_EINVAL;
    if (!al16(q) || !al16(k) || !al16(v) || !al16(out) || !al16(d_out) || !al4(lse)) return NOMAS_EINVAL;
    if (!al16(dq) || !al16(dk) || !al16(dv)) return NOMAS_EINVAL;
    const int64_t need = nomas_seg_attn_bwd_workspace(segs, n_segs, H);
    if (need < 0) return (int)need;
    SegTable st;
    int64_t Ln = 0;
    build_segs(segs, n_segs, &st, &Ln);
    if (Ln == 0) return NOMAS_OK;
    if (!workspace || !al16(workspace) || workspace_bytes < need) return NOMAS_EINVAL;
    RopeTables rt;
    const int rc = rope_tables(&rt);
    if (rc != NOMAS_OK) return rc;
    return launch_seg_attn_bwd(q, k, v, out, lse, d_out, st, (int)Ln, H, sm_scale, dq, dk, dv, workspace, rt,
                               (hipStream_t)stream);
}

// decoder window attention: one all-text segment (no rotation), no cache,
// KV heads shared by groups of query heads
static int gqa_plan(int64_t L, int Hq, int Hkv, SegTable* st) {
    if (L < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return NOMAS_EINVAL;
    if (Hq > kMaxHeads || L > kMaxTokens || L * Hq > NOMAS_MAX_TOKEN_HEADS) return NOMAS_EUNSUPPORTED;
    const nomas_seg s = {(int32_t)L, 0, 0, 0, 0};
    int64_t Ln = 0;
    return build_segs(&s, 1, st, &Ln);
}

int64_t nomas_gqa_attn_workspace(int64_t L, int Hq, int Hkv) {
    SegTable st;
    const int rc = gqa_plan(L, Hq, Hkv, &st);
    if (rc != NOMAS_OK) return rc;
    return seg_attn_workspace_bytes(st, 0, (int)L, Hq, Hkv, 0, nullptr, nullptr);
}

int nomas_gqa_attn(const nomas_bf16* q, const nomas_bf16* k, const nomas_bf16* v, int64_t L, int Hq, int Hkv,
                   float sm_scale, nomas_bf16* out, float* lse, void* workspace, int64_t workspace_bytes,
                   void* stream) {
    if (!q || !k || !v || !out || !finite_pos(sm_scale)) return NOMAS_EINVAL;
    if (!al16(q) || !al16(k) || !al16(v) || !al16(out) || (lse && !al4(lse))) return NOMAS_EINVAL;
    SegTable st;
    int rc = gqa_plan(L, Hq, Hkv, &st);
    if (rc != NOMAS_OK) return rc;
    if (L == 0) return NOMAS_OK;
    const int64_t need = seg_attn_workspace_bytes(st, 0, (int)L, Hq, Hkv, 0, nullptr, nullptr);
    if (need < 0) return (int)need;
    if (!workspace || !al16(workspace) || workspace_bytes < need) return NOMAS_EINVAL;
    RopeTables rt;
    if ((rc = rope_tables(&rt)) != NOMAS_OK) return rc;
    return launch_seg_attn(q, k, v, st, (int)L, nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr, nullptr, Hq, Hkv,
                           sm_scale, out, lse, 0, workspace, rt, (hipStream_t)stream);
}

int nomas_seg_attn(const nomas_bf16* q, const nomas_bf16* k_new, const nomas_bf16* v_new,
                   const nomas_seg* new_segs, int n_new_segs, const int8_t* k_codes, const int8_t* v_codes,
                   const float* k_scale, const float* v_scale, int64_t cap, int64_t cache_len, int H,
                   float sm_scale, nomas_bf16* out, float* lse, int n_split, void* workspace,
                   int64_t workspace_bytes, void* stream) {
    return nomas_seg_attn_sel(q, k_new, v_new, new_segs, n_new_segs, k_codes, v_codes, k_scale, v_scale, cap,
                              cache_len, nullptr, nullptr, H, sm_scale, out, lse, n_split, workspace,
                              workspace_bytes, stream);
}

namespace {
int w8a16_shape(int64_t M, int64_t K, int64_t N) {
    if (M < 0 || K < 1 || N < 1) return NOMAS_EINVAL;
    if (K % 64 != 0 || N % 256 != 0) return NOMAS_EUNSUPPORTED;
    if (M * K * 2 >= ((int64_t)1 << 31) || N * K * 2 >= ((int64_t)1 << 31) || M * N >= ((int64_t)1 << 40))
        return NOMAS_EUNSUPPORTED;
    return NOMAS_OK;
}
}  // namespace

int64_t nomas_w8a16_linear_workspace(int64_t K, int64_t N) {
    const int rc = w8a16_shape(0, K, N);
    return rc != NOMAS_OK ? rc : w8a16_workspace_bytes(N, K);
}

int nomas_w8a16_linear(const nomas_bf16* x, int64_t M, int64_t K, const int8_t* w_codes, const float* w_scale,
                       int64_t N, nomas_bf16* y, void* workspace, int64_t workspace_bytes, void* stream) {
    int rc = w8a16_shape(M, K, N);
    if (rc != NOMAS_OK) return rc;
    if (!w_codes || !w_scale || !workspace) return NOMAS_EINVAL;
    if (M > 0 && (!x || !y)) return NOMAS_EINVAL;
    if ((x && !al16(x)) || (y && !al16(y)) || !al16(w_codes) || !al4(w_scale) || !al16(workspace))
        return NOMAS_EINVAL;
    if (workspace_bytes < w8a16_workspace_bytes(N, K)) return NOMAS_EINVAL;
    return launch_w8a16(x, M, K, w_codes, w_scale, N, y, workspace, (hipStream_t)stream);
}

int nomas_w8a16_linear_noalloc(const nomas_bf16* x, int64_t M, int64_t K, const int8_t* w_codes,
                               const float* w_scale, int64_t N, nomas_bf16* y, void* stream) {
    int rc = w8a16_shape(M, K, N);
    if (rc != NOMAS_OK) return rc;
    if (!w_codes || !w_scale) return NOMAS_EINVAL;
    if (M > 0 && (!x || !y)) return NOMAS_EINVAL;
    if ((x && !al16(x)) || (y && !al16(y)) || !al16(w_codes) || !al4(w_scale)) return NOMAS_EINVAL;
    if (w8a16_workspace_bytes(N, K) > NOMAS_W8A16_NOALLOC_MAX_BYTES) return NOMAS_EUNSUPPORTED;
    void* ws = nullptr;
    if ((rc = w8a16_scratch(&ws)) != NOMAS_OK) return rc;
    return launch_w8a16(x, M, K, w_codes, w_scale, N, y, ws, (hipStream_t)stream);
}

int nomas_cam_tokens(const double* c2w, int n_frames, double translation_scale, double rotation_scale,
                     float* tokens) {
    if (!c2w || !tokens || n_frames < 4 || (n_frames % 4) != 0) return NOMAS_EINVAL;
    if (!std::isfinite(translation_scale) || !std::isfinite(rotation_scale)) return NOMAS_EINVAL;
    const double* M0 = c2w;
    double R0t[9], t0[3];
    for (int i = 0; i < 3; ++i) {
        t0[i] = M0[4 * i + 3];
        for (int j = 0; j < 3; ++j) R0t[3 * i + j] = M0[4 * j + i];   // R0^T
    }
    for (int k = 0; k < n_frames; ++k) {
        const double* M = c2w + 16 * k;
        double Rk[9], Rr[9], dt[3], tr[3], axis[3], ang, Rs[9];
        for (int i = 0; i < 3; ++i) {
            dt[i] = M[4 * i + 3] - t0[i];
            for (int j = 0; j < 3; ++j) Rk[3 * i + j] = M[4 * i + j];
        }
        mat3_mul(R0t, Rk, Rr);
        for (int i = 0; i < 3; ++i) tr[i] = R0t[3 * i] * dt[0] + R0t[3 * i + 1] * dt[1] + R0t[3 * i + 2] * dt[2];
        rot_log(Rr, axis, &ang);
        rot_exp(axis, rotation_scale * ang, Rs);
        float* o = tokens + 16 * k;
        for (int i = 0; i < 3; ++i) {
            for (int j = 0; j < 3; ++j) o[4 * i + j] = (float)Rs[3 * i + j];
            o[4 * i + 3] = (float)(translation_scale * tr[i]);
        }
        o[12] = 0.0f; o[13] = 0.0f; o[14] = 0.0f; o[15] = 1.0f;
    }
    return NOMAS_OK;
}

int64_t nomas_cam_xattn_workspace(int H, int Nc) {
    if (H < 1 || Nc < 1) return NOMAS_EINVAL;
    if (H > kMaxHeads || Nc > NOMAS_MAX_CAM) return NOMAS_EUNSUPPORTED;
    return cam_xattn_workspace_bytes(H, Nc);
}

int nomas_cam_xattn(const nomas_bf16* q, int64_t Lq, int H, const float* cam, int Nc, const nomas_bf16* w_k,
                    const nomas_bf16* w_v, float sm_scale, nomas_bf16* out, void* workspace, int64_t workspace_bytes,
                    void* stream) {
    if (Lq < 0 || H < 1 || Nc < 1 || !finite_pos(sm_scale)) return NOMAS_EINVAL;
    if (H > kMaxHeads || Lq > kMaxTokens || Nc > NOMAS_MAX_CAM) return NOMAS_EUNSUPPORTED;
    if (Lq == 0) return NOMAS_OK;
    if (!q || !cam || !w_k || !w_v || !out) return NOMAS_EINVAL;
    if (!al16(q) || !al16(cam) || !al16(w_k) || !al16(w_v) || !al16(out)) return NOMAS_EINVAL;
    if (!workspace || !al16(workspace) || workspace_bytes < cam_xattn_workspace_bytes(H, Nc)) return NOMAS_EINVAL;
    return launch_cam_xattn(q, Lq, H, cam, Nc, w_k, w_v, sm_scale, out, workspace, (hipStream_t)stream);
}

}  // extern "C"
