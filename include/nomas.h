/*
 * nomas.h -- C ABI of libnomas: segment-causal attention over a lifelong INT8
 * KV cache, for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (Hy-Nomas pages, cited by title and section):
 *  - "Hy-Nomas：腾讯混元交互式世界模型，8 步生成 720p 可控视频" (comfyui-wiki news),
 *    section 一个世界，分段生成: video is generated segment by segment; each
 *    segment attends to the key/value cache of every earlier segment, and
 *    attention is causal between segments (a segment never needs a later one).
 *  - same page, section 模型内部: 16 heads x 128, 3D RoPE with axis sizes
 *    [16, 56, 56] and theta 256, latent patch 1x1x1 (880 tokens per 1280x704
 *    latent frame); camera extrinsics injected by cross-attention.
 *  - same page, section 单张 4090 配置, and "Hy-Nomas:8B 参数、单张 4090 跑 60 秒
 *    可控世界" (huaweicloud blog), section 3.5 table: cached keys and values are
 *    stored as INT8 while attention is computed in BF16.
 *  - huaweicloud blog, section 2.1: the text and video K,V of each segment are
 *    cached and handed to the next segment.
 *  - comfyui-wiki news, section 相机控制作为一等输入: c2w [N,4,4], normalised,
 *    grouped per 4 video frames into 64-d inputs that video tokens query by
 *    cross-attention; translation scale 1.0 and rotation scale 2.5.
 *
 * Conventions for every entry point
 *  - Tensor pointers marked "device" are caller-owned device memory (HBM) on
 *    the current HIP device; pointers marked "host" are ordinary host memory.
 *    The library never frees or keeps caller pointers.
 *  - bf16 tensors hold raw bfloat16 bit patterns (nomas_bf16).  Token-major
 *    tensors are [L][H][128] (token, head, channel), 16-byte aligned.
 *  - The INT8 cache is head-major: codes [H][cap][128] (int8), scales
 *    [H][cap] (float32), one scale per (token, head).  Keys are cached after
 *    RoPE, so cached entries carry no position.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work on it; they never synchronise.
 *  - Arguments are checked on the host before anything is enqueued.  A
 *    non-zero return means nothing was launched and no output was written:
 *      NOMAS_EINVAL       null pointer, bad size, misaligned pointer, token
 *                         counts that disagree with the segment descriptors
 *      NOMAS_ECAPACITY    the cache cannot hold the appended tokens
 *      NOMAS_EUNSUPPORTED a size outside the library's fixed limits
 *      NOMAS_EHIP         a HIP runtime call or launch failed
 *    A fault inside a kernel surfaces at the caller's next synchronisation.
 *  - The only device memory the library owns is static: a RoPE cos/sin table
 *    per device (uploaded on first use) and the scratch array of
 *    nomas_w8a16_linear_noalloc.  Both belong to the loaded code object and
 *    are released with it when the process ends; nomas_shutdown() drops the
 *    host state that refers to them.
 *  - Token layout of a segment: its n_text text tokens first, then its
 *    T*Hg*Wg video tokens in (t, h, w) row-major order, t in [t0, t0+T).
 *    Text tokens are not rotated; video token (t, h, w) uses t as the
 *    absolute latent-frame index and h, w counted from 0.
 */
#ifndef NOMAS_H
#define NOMAS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t nomas_bf16;

/* One segment of tokens: [n_text text | T*Hg*Wg video, (t,h,w) row-major]. */
typedef struct {
    int32_t n_text, t0, T, Hg, Wg;
} nomas_seg;

enum {
    NOMAS_OK = 0,
    NOMAS_EINVAL = -1,
    NOMAS_ECAPACITY = -2,
    NOMAS_EHIP = -3,
    NOMAS_EUNSUPPORTED = -4
};

#define NOMAS_HEAD_DIM 128
#define NOMAS_MAX_SEGS 64          /* segments per call (new or packed)        */
#define NOMAS_MAX_T 16384          /* latent-frame positions t < NOMAS_MAX_T   */
#define NOMAS_MAX_HW 1024          /* grid positions h, w < NOMAS_MAX_HW       */
#define NOMAS_MAX_CAM 128          /* camera tokens per call                   */
#define NOMAS_MAX_CACHE (1 << 24)  /* nomas_seg_attn: cache capacity (tokens)  */
#define NOMAS_MAX_TOKEN_HEADS (1 << 23)  /* nomas_seg_attn: new tokens x heads */
#define NOMAS_MAX_SPLIT 4          /* nomas_seg_attn: key-range parts per query tile */
#define NOMAS_MAX_SEL_RANGES 64    /* nomas_seg_attn_sel: cache-token ranges per call */

/*
 * 3D RoPE (comfyui-wiki news, 模型内部: axes [16, 56, 56], theta 256).
 * Channels [0,16) turn with t, [16,72) with h, [72,128) with w.  In a chunk
 * of width d, pair (2i, 2i+1) turns by phi = p * 256^(-2i/d):
 *   (x0, x1) -> (x0 cos phi - x1 sin phi, x0 sin phi + x1 cos phi).
 * x, y: device, [L][H][128] bf16 with L = sum of the segments' token counts;
 * y may equal x (in place).  The rotation is evaluated in double precision
 * and rounded once to bf16 (nearest even).  Text tokens are copied unchanged.
 */
int nomas_rope3d(const nomas_bf16* x, nomas_bf16* y, const nomas_seg* segs, int n_segs,
                 int H, void* stream);

/*
 * INT8 quantise-and-append of a segment's K and V into the lifelong cache
 * (cached K/V stored as INT8: comfyui-wiki news, 单张 4090 配置; huaweicloud
 * blog, section 3.5).  For every (token i, head h) row of 128 values:
 *   a = max |x|,  s = fl32(a / 127),  q = clamp(rne(x / s), -127, 127)
 * with the exact quotient x/s (a = 0 gives s = 0 and q = 0).  Row (i, h) of
 * k_rot goes to k_codes[h][len+i][:] / k_scale[h][len+i]; likewise v.
 * k_rot, v: device, [L][H][128] bf16 (keys already rotated).
 * k_codes, v_codes: device, [H][cap][128] int8.  k_scale, v_scale: device,
 * [H][cap] float32.  len: host, in = tokens already cached, out = len + L.
 * L = 0 is a no-op.  ECAPACITY if len + L > cap (nothing written, len kept).
 */
int nomas_kv_quant_append(const nomas_bf16* k_rot, const nomas_bf16* v, int64_t L, int H,
                          int8_t* k_codes, int8_t* v_codes, float* k_scale, float* v_scale,
                          int64_t cap, int64_t* len, void* stream);

/*
 * Segment-causal joint attention of the current segment(s) (comfyui-wiki
 * news, 一个世界，分段生成; huaweicloud blog, section 2.1).
 * Query i of new segment a attends to every cached token and to the new
 * tokens of segments 0..a: bidirectional inside its own segment, never to a
 * later segment.  With one new segment this is inference; several new
 * segments pack a training sequence (block-causal).
 *   s_ij = sm_scale * <RoPE(q_i), K_j>,  o_i = softmax_j(s_ij) . V_j
 * over the allowed j; lse_i = ln sum_j exp(s_ij).
 * BF16 compute: RoPE(q), RoPE(k_new) are rounded to bf16; cached entries
 * enter as bf16(fl32(code * scale)); products accumulate in fp32.
 * q, k_new, v_new: device, [Ln][H][128] bf16, q and k_new BEFORE RoPE
 *   (rotated inside: q in float32, k_new in float64 exactly as
 *   nomas_rope3d), Ln = sum of the new segments' token counts.
 * k_codes, v_codes, k_scale, v_scale: device cache as for
 *   nomas_kv_quant_append; its first cache_len entries are used (may be 0,
 *   then the cache pointers may be NULL).
 * sm_scale > 0 (1/sqrt(128) for the model).
 * out: device, [Ln][H][128] bf16.  lse: device [H][Ln] float32 or NULL.
 * n_split: 0 lets the library split query tiles' keys into contiguous
 *   parts so that the grid fills the GPU's last round of workgroups: every
 *   tile into 1..4 parts, or, with one new segment, only the tiles of the
 *   last round into up to 8 (partial results are merged by the log-sum-exp
 *   identity); 1..NOMAS_MAX_SPLIT forces that many parts for every tile.
 *   Results agree to rounding.
 * workspace: device scratch of at least nomas_seg_attn_workspace(...)
 *   bytes (same segments, cache_len, H and n_split, on the current device),
 *   16-byte aligned, owned by the caller; the call overwrites it, so two
 *   calls in flight must not share one.  It holds the keys the call may see
 *   laid out as bf16 64-key tile images, 35,840 bytes per tile and head
 *   (560 bytes per cached or new token and head: 2.84 GB for 253,440 cached
 *   + 63,360 new tokens at 16 heads), each tile's largest squared key norm,
 *   and fp32 partial results when the keys are split.  Too small or NULL:
 *   NOMAS_EINVAL.
 * n_new_segs in [1, NOMAS_MAX_SEGS]; cap <= NOMAS_MAX_CACHE and
 * Ln * H <= NOMAS_MAX_TOKEN_HEADS, else NOMAS_EUNSUPPORTED.
 */
int nomas_seg_attn(const nomas_bf16* q, const nomas_bf16* k_new, const nomas_bf16* v_new,
                   const nomas_seg* new_segs, int n_new_segs,
                   const int8_t* k_codes, const int8_t* v_codes,
                   const float* k_scale, const float* v_scale,
                   int64_t cap, int64_t cache_len, int H, float sm_scale,
                   nomas_bf16* out, float* lse, int n_split, void* workspace, int64_t workspace_bytes,
                   void* stream);

/*
 * nomas_seg_attn with a history selection: each new segment attends to a
 * chosen subset of the cached tokens instead of the whole cache.  The pages
 * let a segment look at a subset of the earlier frames: the most recent latent
 * frames or frames sampled by temporal_context (huaweicloud blog, section 3.5
 * table; comfyui-wiki news, 单张 4090 配置), chosen by the kind of action
 * (huaweicloud blog, section 2.2).  The caller names the cache tokens:
 * sel_off: host, n_new_segs + 1 non-decreasing int32 offsets, sel_off[0] = 0;
 *   segment a uses ranges sel_off[a] .. sel_off[a+1]-1.
 * sel_ranges: host, int64 pairs (start, end) of cache tokens, 0 <= start <
 *   end <= cache_len, sorted and non-overlapping within a segment (NULL
 *   allowed when there are no ranges).  A segment with no ranges sees no
 *   cached token.  sel_off == NULL: every segment sees the whole cache, i.e.
 *   nomas_seg_attn.
 * Query i of segment a then attends to its selected cache tokens and to the
 * new tokens of segments 0..a.  Segments with identical lists share packed
 * key tiles; otherwise each segment's keys are packed separately, which the
 * workspace size accounts for.  Other arguments, the workspace and the errors
 * are those of nomas_seg_attn; an invalid selection gives NOMAS_EINVAL, more
 * than NOMAS_MAX_SEL_RANGES ranges NOMAS_EUNSUPPORTED.
 */
int nomas_seg_attn_sel(const nomas_bf16* q, const nomas_bf16* k_new, const nomas_bf16* v_new,
                       const nomas_seg* new_segs, int n_new_segs,
                       const int8_t* k_codes, const int8_t* v_codes,
                       const float* k_scale, const float* v_scale,
                       int64_t cap, int64_t cache_len,
                       const int32_t* sel_off, const int64_t* sel_ranges,
                       int H, float sm_scale,
                       nomas_bf16* out, float* lse, int n_split, void* workspace, int64_t workspace_bytes,
                       void* stream);

/*
 * Workspace bytes nomas_seg_attn_sel needs (same selection arguments), or a
 * negative error code.  Host only.
 */
int64_t nomas_seg_attn_sel_workspace(const nomas_seg* new_segs, int n_new_segs, int64_t cache_len,
                                     const int32_t* sel_off, const int64_t* sel_ranges, int H, int n_split);

/*
 * Workspace bytes nomas_seg_attn needs for these new segments, cache length,
 * head count and n_split on the current device: with T = H * ceil((cache_len
 * + Ln) / 64) tiles, T * 35840 + (4T rounded up to a multiple of 256), plus
 * parts * 516 per (query, head) of the split query tiles when keys are
 * split into parts > 1 (all Ln * H pairs when every tile is split); or a negative
 * error code (NOMAS_EINVAL / NOMAS_EUNSUPPORTED as for nomas_seg_attn).
 * Host only.
 */
int64_t nomas_seg_attn_workspace(const nomas_seg* new_segs, int n_new_segs, int64_t cache_len, int H,
                                 int n_split);

/*
 * Backward pass of packed segment-causal attention, for segment-forcing
 * training on packed sequences (huaweicloud blog, section 2.3: sequences
 * packed up to 360,000 tokens; the block-causal mask of comfyui-wiki news,
 * 一个世界，分段生成): the gradients with respect to q, k and v of
 * nomas_seg_attn in packed mode (several segments, no cache), given dO, the
 * gradient with respect to its output.  Per head, over the allowed pairs:
 *   P = exp(s - lse),  dV = P^T dO,  dP = dO V^T,  D_i = <dO_i, out_i>,
 *   dS = P * (dP - D),  dq = R^T sm_scale dS Kr,  dk = R^T sm_scale dS^T Qr
 * where Qr, Kr are the rotated bf16 operands of the forward call (rebuilt
 * bit for bit) and R^T undoes the 3D RoPE rotation; the bf16 rounding of the
 * rotated q and k is taken as a cast with identity derivative.  P and dS
 * enter their products as bf16, sums are fp32.
 * q, k, v: device [L][H][128] bf16, exactly as given to nomas_seg_attn
 *   (q and k before RoPE).  out, lse: device, the forward's output [L][H][128]
 *   bf16 and log-sum-exp [H][L] float32 (natural log) for the same
 *   arguments and sm_scale.  d_out: device [L][H][128] bf16.
 * dq, dk, dv: device [L][H][128] float32, overwritten (never accumulated).
 * segs: the packed segments (the forward's new_segs), L = their token count.
 * workspace: device scratch of at least nomas_seg_attn_bwd_workspace(...)
 *   bytes, 16-byte aligned, owned by the caller (each segment's tokens laid
 *   out as 64-token tiles: 70,656 bytes per tile and head); two calls in
 *   flight must not share one.  Pointers 16-byte aligned (lse 4).
 * Errors as nomas_seg_attn; L * H <= NOMAS_MAX_TOKEN_HEADS.
 */
int nomas_seg_attn_bwd(const nomas_bf16* q, const nomas_bf16* k, const nomas_bf16* v,
                       const nomas_bf16* out, const float* lse, const nomas_bf16* d_out,
                       const nomas_seg* segs, int n_segs, int H, float sm_scale,
                       float* dq, float* dk, float* dv, void* workspace, int64_t workspace_bytes,
                       void* stream);

/*
 * Workspace bytes nomas_seg_attn_bwd needs: H * 70,656 * (sum over the
 * segments of ceil(tokens / 64)); or a negative error code.  Host only.
 */
int64_t nomas_seg_attn_bwd_workspace(const nomas_seg* segs, int n_segs, int H);

/*
 * Attention of one decoder window with grouped key/value heads.  The
 * PixelUMM decoder has 32 query heads and 8 KV heads over a 4096-wide hidden
 * state and reconstructs RGB from 4 x 16 x 16 tubelets on 10-latent-frame
 * windows overlapping by 5 frames (comfyui-wiki news, 模型内部).  Every token
 * of the window attends to every token of it; query head h uses KV head
 * h / (Hq / Hkv); no positions are applied here (rotate q and k first with
 * nomas_rope3d if the caller's model uses them):
 *   s_ij = sm_scale * <q_i, k_j>,  o_i = softmax_j(s_ij) . v_j,  lse_i = ln sum_j exp(s_ij)
 * q: device [L][Hq][128] bf16; k, v: device [L][Hkv][128] bf16; out: device
 * [L][Hq][128] bf16; lse: device [Hq][L] float32 or NULL.  Hq a multiple of
 * Hkv, sm_scale > 0.  workspace: device scratch of at least
 * nomas_gqa_attn_workspace(L, Hq, Hkv) bytes, 16-byte aligned, owned by the
 * caller (the keys laid out as 64-key tiles per KV head).  Errors as
 * nomas_seg_attn; L * Hq <= NOMAS_MAX_TOKEN_HEADS.
 */
int nomas_gqa_attn(const nomas_bf16* q, const nomas_bf16* k, const nomas_bf16* v, int64_t L, int Hq, int Hkv,
                   float sm_scale, nomas_bf16* out, float* lse, void* workspace, int64_t workspace_bytes,
                   void* stream);

/* Workspace bytes nomas_gqa_attn needs, or a negative error code.  Host only. */
int64_t nomas_gqa_attn_workspace(int64_t L, int Hq, int Hkv);

/*
 * Linear layer with INT8-stored weights and BF16 math: y = x . W^T.  The DiT
 * weights are stored INT8 while the linear layers compute in BF16
 * (comfyui-wiki news, 单张 4090 配置; huaweicloud blog, section 3.5 table).
 * Each weight enters as bf16(fl32(code * scale)) with one fp32 scale per
 * output channel; products accumulate in fp32 and y is rounded to bf16.
 * x: device [M][K] bf16; w_codes: device [N][K] int8; w_scale: device [N]
 * float32; y: device [M][N] bf16.  K a multiple of 64 and N of 256 (the
 * model's 2048 / 6144 / 8192), else NOMAS_EUNSUPPORTED; M >= 0 any.
 * workspace: device scratch of at least nomas_w8a16_linear_workspace(K, N)
 * bytes (the weights dequantised to bf16 for this call), 16-byte aligned,
 * owned by the caller.  Pointers 16-byte aligned (scales 4).
 */
int nomas_w8a16_linear(const nomas_bf16* x, int64_t M, int64_t K, const int8_t* w_codes, const float* w_scale,
                       int64_t N, nomas_bf16* y, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes nomas_w8a16_linear needs (N * K * 2), or a negative error code.  Host only. */
int64_t nomas_w8a16_linear_workspace(int64_t K, int64_t N);

/* Largest N * K * 2 (dequantised weight bytes) nomas_w8a16_linear_noalloc
 * takes: 32 MiB, every linear shape of the DiT (2048 -> 6144 / 8192,
 * 8192 -> 2048). */
#define NOMAS_W8A16_NOALLOC_MAX_BYTES ((int64_t)32 << 20)

/*
 * nomas_w8a16_linear for callers that cannot allocate device memory: code
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, result and kernels as nomas_w8a16_linear,
 * without the workspace: the dequantised weights go into a static scratch
 * array of the library (NOMAS_W8A16_NOALLOC_MAX_BYTES per device, held from
 * the library's load until the process ends).  No memory is allocated or
 * freed and no allocating routine is called.  The first call on a device
 * looks up the scratch array's device address (hipGetSymbolAddress) and
 * keeps it.  N * K * 2 > NOMAS_W8A16_NOALLOC_MAX_BYTES: NOMAS_EUNSUPPORTED,
 * checked before anything touches the device.  Every call on one device
 * shares that device's array, and each call overwrites the part it uses
 * before reading it (nothing needs clearing), so calls that overlap in time
 * on one device (other streams, other threads) race: serialise them.
 */
int nomas_w8a16_linear_noalloc(const nomas_bf16* x, int64_t M, int64_t K, const int8_t* w_codes,
                               const float* w_scale, int64_t N, nomas_bf16* y, void* stream);

/*
 * Camera tokens of one turn (comfyui-wiki news, 相机控制作为一等输入).
 * Poses are made relative to the first frame (R0^T R_k, R0^T (t_k - t0)),
 * translations are multiplied by translation_scale and rotation angles
 * (axis-angle) by rotation_scale; 4 consecutive 4x4 matrices, row-major,
 * form one 64-value token.  Host-side: c2w host [n_frames][4][4] float64,
 * n_frames a positive multiple of 4; tokens host [n_frames/4][64] float32.
 */
int nomas_cam_tokens(const double* c2w, int n_frames, double translation_scale,
                     double rotation_scale, float* tokens);

/*
 * Camera cross-attention (comfyui-wiki news, 相机控制作为一等输入 and 模型内部:
 * extrinsic embedding injected by cross-attention).  Kc = bf16(cam . w_k),
 * Vc = bf16(cam . w_v) per head; every query attends to all Nc camera tokens:
 *   out_i = softmax_n(sm_scale <q_i, Kc_n>) . Vc_n    (no RoPE)
 * q: device [Lq][H][128] bf16 (video-token queries).  cam: device [Nc][64]
 * float32.  w_k, w_v: device [64][H*128] bf16.  out: device [Lq][H][128]
 * bf16.  1 <= Nc <= NOMAS_MAX_CAM.
 * workspace: device scratch of at least nomas_cam_xattn_workspace(H, Nc)
 * bytes, 16-byte aligned, owned by the caller: each head's projected camera
 * keys and values (Kc, then Vc transposed) as the query stream keeps them
 * in LDS, written by the call and read by its second kernel (52,736 bytes
 * per head for 65..96 camera tokens); two calls in flight must not share one.
 * Too small or NULL: NOMAS_EINVAL (Lq = 0 needs none).
 */
int nomas_cam_xattn(const nomas_bf16* q, int64_t Lq, int H, const float* cam, int Nc,
                    const nomas_bf16* w_k, const nomas_bf16* w_v, float sm_scale,
                    nomas_bf16* out, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes nomas_cam_xattn needs for H heads and Nc camera tokens, or
 * a negative error code.  Host only. */
int64_t nomas_cam_xattn_workspace(int H, int Nc);

/*
 * Host copy of the library's float32 RoPE table for one axis (0 = t, 1 = h,
 * 2 = w): cos_out/sin_out host [npos][d/2] with entry (p, i) =
 * fl32(cos(p * 256^(-2i/d))).  Needs no GPU.
 */
int nomas_rope_table(int axis, int npos, float* cos_out, float* sin_out);

/*
 * Drops the library's per-device host state: the "RoPE table uploaded" flag
 * and the cached device addresses of its static arrays, for every device.
 * The next call on a device uploads the table and looks the addresses up
 * again.  Call it after resetting a device (hipDeviceReset reloads the code
 * object, whose static arrays then start empty) or when the library should
 * hold no state; no device memory is freed (there is none to free) and
 * work already enqueued is unaffected.  It must not run concurrently with
 * other calls of the library.  Host only; returns NOMAS_OK.
 */
int nomas_shutdown(void);

/* Static description of an error code; never NULL. */
const char* nomas_strerror(int code);

/* Library version string. */
const char* nomas_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NOMAS_H */
