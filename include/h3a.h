/*
 * h3a -- packed varlen attention head for AMD Instinct MI355X (gfx950).
 *
 * The per-step attention of the MiniMax H3 video+audio DiT over one packed
 * multi-segment sequence:
 *   1. a step-invariant 3D (t, h, w) rotary table for the packed segments,
 *   2. per-head RMSNorm of Q and K fused with NeoX rotary on the first R dims,
 *   3. bidirectional attention restricted to each cu_seqlens segment.
 * Variants of the same path (the *_ex and suffixed calls below): other rotary
 * table modes (fp64 linspace grid, the ViT3D's length-normalised ids,
 * interleaved M-RoPE), grouped K/V heads and a causal mask (the encoder text
 * tower), the Q norm + rotary folded into the attention, and low-precision
 * attention: FP8 E4M3 operands with per-block power-of-two scales, INT8
 * scores with per-token q and per-64-key-block k scales (with a bf16 or FP8
 * PV product), and norm + rotary passes writing the quantised operands.
 *
 * Sources (the pages this library was built from):
 *   - vllm.cpp PR #26 "feat(minimax-h3): port the MiniMax-H3 omni-modal
 *     video+audio DiT", opening commit: the DiT runs once per step over the
 *     whole packed sequence, and its packed non-causal attention is exactly a
 *     cu_seqlens varlen flash-attention call with a per-document bidirectional
 *     contract; the fp64 position grid feeds the rotary.
 *   - same PR, description, "The device-resident forward (W2b)": the H3 3D
 *     rotary is plain NeoX rotate-half fed by a per-row cos/sin cache whose
 *     angles come from three axes; RmsNorm reduces in f32.
 *   - same PR, commit on the attention fast path: f32 accumulation and an
 *     online-softmax recurrence.
 *   - h3-spark model card, "What this config does": Q RMSNorm followed by the
 *     rotary on the first 96 dims, byte-exact on default and non-default
 *     streams; rope/cond/mask tables are step-invariant caches.
 *
 * Conventions for every call:
 *   - Device pointers are owned by the caller.  The library owns only its
 *     attention tile plans (small device buffers keyed by the cu_seqlens
 *     content; see h3a_release_caches).
 *   - Every argument is validated before anything is launched.  On error the
 *     call returns a non-zero status, records a message naming the offending
 *     argument (h3a_last_error), and writes nothing.  No C++ exception crosses
 *     the boundary: a failed host allocation inside the library returns
 *     EUNSUPPORTED.  Attention calls (and h3a_plan_tiles) refuse, with
 *     EUNSUPPORTED and before building anything, a packing whose tile plan
 *     would exceed 2^26 work items (far beyond any packing whose tensors fit
 *     in one GPU's memory).
 *   - Work is enqueued on `stream` (0 = the null stream); no call
 *     synchronises the stream.  Results are bitwise deterministic and
 *     independent of the stream used.
 *   - Graph capture: once an attention call has run with a given cu_seqlens,
 *     head count and device (its tile plan is then cached), every call
 *     only launches kernels on `stream`: no allocation, copy, memset or
 *     synchronisation, so such calls (and every non-attention call) can be
 *     captured in a HIP graph and replayed; replays read the buffers'
 *     current contents.  The first call for a new packing allocates and
 *     uploads its plan synchronously (and, with 256 plans cached, frees the
 *     oldest after synchronising its device): made on a capturing stream it
 *     fails with EUNSUPPORTED and enqueues nothing, and it must not run
 *     while another stream captures in hipStreamCaptureModeGlobal.
 *   - Plan lifetime: a plan used by a call on a capturing stream is pinned --
 *     the graph keeps its device address -- and is never evicted; only
 *     h3a_release_caches frees it, so destroy graphs holding attention
 *     launches before calling h3a_release_caches.
 *   - Tensors are token-major: element (n, h, d) of a [S, H, D] tensor with
 *     token stride `stride` (in elements) is at base[n * stride + h * D + d].
 *   - Floating point: H3A_BF16 tensors hold bfloat16; arithmetic is fp32 and
 *     each bf16 result is rounded once, to nearest even.  H3A_F32 is fp32
 *     throughout.
 */
#ifndef H3A_H
#define H3A_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum h3a_status {
  H3A_OK = 0,
  H3A_EINVAL = 1,       /* null pointer, negative size, bad cu_seqlens ...   */
  H3A_ESHAPE = 2,       /* sizes that disagree with each other               */
  H3A_EDTYPE = 3,       /* unknown dtype                                     */
  H3A_EUNSUPPORTED = 4, /* valid request outside what the kernels implement  */
  H3A_EHIP = 5          /* the HIP runtime reported an error                 */
} h3a_status;

typedef enum h3a_dtype { H3A_F32 = 0, H3A_BF16 = 1 } h3a_dtype;

/*
 * Step-invariant rotary table for a packed sequence (built once per request).
 *
 * segments       host int32 [nseg][4]: (T, H, W, L) per segment, packed in this
 *                order.  T, H, W >= 1 and 0 <= L <= T*H*W.  Token n < L of a
 *                segment sits at t = n / (H*W), h = (n / W) % H, w = n % W
 *                (row-major, w fastest); positions restart at 0 per segment.
 * axis_dims      host int32 [3]: rotated dims owned by the t, h, w axes; each
 *                even and >= 0; R = sum.  Axis a contributes axis_dims[a]/2
 *                frequencies base^(-2j/axis_dims[a]), j = 0, 1, ...
 * base           rotary base (> 0), e.g. 10000.
 * cos_sin        device fp32 [2][S][R/2]: cos block, then sin block.  Entry
 *                (n, i) is cos/sin of the i-th angle of token n, where the
 *                angle vector is concat(t*f_t, h*f_h, w*f_w), evaluated in
 *                fp64 and rounded once to fp32.  Must be 16-byte aligned.
 * S              total tokens; must equal the sum of L (the size of cos_sin).
 * cu_seqlens_out host int32 [nseg+1] or NULL: prefix sums of L, from 0.
 *
 * Errors: EINVAL (null segments/axis_dims, nseg < 1, T/H/W < 1, L out of
 * range, odd or negative axis dims, base <= 0, S mismatch, S > INT32_MAX,
 * null cos_sin with R > 0), EHIP.
 */
h3a_status h3a_build_rope_table(const int32_t* segments, int32_t nseg, const int32_t* axis_dims,
                                double base, float* cos_sin, int64_t S, int32_t* cu_seqlens_out,
                                hipStream_t stream);

/*
 * Other ways of filling the same rotary table.  Only the angles change; the
 * table layout, the rotate-half that consumes it and every other argument
 * are as for h3a_build_rope_table.
 *
 * For a token with grid index i_a and segment extent n_a on axis a (n_t = T,
 * n_h = H, n_w = W), the fp64 coordinate p_a is
 *   H3A_ROPE_GRID         i_a (exactly h3a_build_rope_table);
 *   H3A_ROPE_LINSPACE     i_a * step_a + start[a], step_a = (stop[a] -
 *                         start[a]) / n_a -- numpy.linspace(start, stop, n_a,
 *                         endpoint=False), whose evaluation order the DiT's
 *                         fp64 grid follows bit for bit (vllm.cpp PR #26
 *                         description, "Correctness gates");
 *   H3A_ROPE_NORMALIZED   2 pi (2 ((i_a + 0.5) / n_a) - 1), the ViT3D
 *                         decoder's length-normalised ids; L may exceed
 *                         T*H*W, and tokens past the grid (its register and
 *                         cls suffix) get angle 0, the identity (video-VAE
 *                         decoder commit, "3D ROPE DETAIL");
 *   H3A_ROPE_INTERLEAVED  i_a, with M-RoPE's interleaved layout (encoder-tower
 *                         commit, "M-RoPE": axes [t h w t h w ...]).
 * GRID, LINSPACE and NORMALIZED use per-axis blocks: angle vector
 * concat(p_t f_t, p_h f_h, p_w f_w) with f_a[j] = base^(-2j/axis_dims[a]).
 * INTERLEAVED uses one ladder F[j] = base^(-2j/R), j < R/2, where angle j
 * takes axis h if j % 3 == 1 and j < 3 n_h, axis w if j % 3 == 2 and
 * j < 3 n_w, else t (n_a = axis_dims[a] / 2); the shares must come out
 * exactly (e.g. equal shares, or Qwen-style (48, 40, 40) for R = 128).
 *
 * spec           host pointer, read during the call only.
 * Errors: as h3a_build_rope_table, plus EINVAL for a null spec, an unknown
 * mode, non-finite start/stop, shares that do not interleave, or T*H*W
 * above INT32_MAX.
 */
typedef enum h3a_rope_mode {
  H3A_ROPE_GRID = 0,
  H3A_ROPE_LINSPACE = 1,
  H3A_ROPE_NORMALIZED = 2,
  H3A_ROPE_INTERLEAVED = 3
} h3a_rope_mode;

typedef struct h3a_rope_spec {
  int32_t mode;          /* h3a_rope_mode */
  int32_t axis_dims[3];  /* rotated dims owned by the t, h, w axes; each even */
  double base;           /* frequency base (> 0) */
  double start[3];       /* H3A_ROPE_LINSPACE only: per-axis start */
  double stop[3];        /* H3A_ROPE_LINSPACE only: per-axis stop (excluded) */
} h3a_rope_spec;

h3a_status h3a_build_rope_table_ex(const int32_t* segments, int32_t nseg, const h3a_rope_spec* spec,
                                   float* cos_sin, int64_t S, int32_t* cu_seqlens_out,
                                   hipStream_t stream);

/*
 * Fused per-head RMSNorm + NeoX rotary of Q and K.
 *
 * For every token n, head h and x in {q, k} (each with its own gain g):
 *   y_d  = x_d / sqrt(mean_d(x_d^2) + eps) * g_d               (d < D)
 *   y'_i       = y_i cos(n,i) - y_{i+R/2} sin(n,i)              (i < R/2)
 *   y'_{i+R/2} = y_{i+R/2} cos(n,i) + y_i sin(n,i)
 *   y'_d = y_d                                                  (d >= R)
 * V is not touched.
 *
 * q, k           device [S, H, D] of `dtype`, token strides stride_q, stride_k.
 * q_out, k_out   device [S, H, D] of `dtype`, token strides stride_qo,
 *                stride_ko.  An output may be its input (same pointer and
 *                stride: in place); any other overlap is rejected.
 * gamma_q/k      device fp32 [D].
 * cos_sin        device fp32 [2][S][R/2] from h3a_build_rope_table; may be
 *                NULL when rot_dim == 0.
 * Supported: D in {64, 128}; rot_dim even, 0 <= rot_dim <= D, and (rot_dim/2)
 * a multiple of 8 (bf16) or 4 (fp32); pointers 16-byte aligned and strides
 * multiples of 16 bytes; strides >= H*D and below 2^31 / 64 bytes.
 *
 * Errors: EINVAL, ESHAPE (stride < H*D), EDTYPE, EUNSUPPORTED, EHIP.
 */
h3a_status h3a_qk_rmsnorm_rope(const void* q, const void* k, void* q_out, void* k_out,
                               h3a_dtype dtype, int64_t S, int32_t H, int32_t D,
                               int64_t stride_q, int64_t stride_k, int64_t stride_qo,
                               int64_t stride_ko, const float* gamma_q, const float* gamma_k,
                               float eps, const float* cos_sin, int32_t rot_dim,
                               hipStream_t stream);

/*
 * h3a_qk_rmsnorm_rope with Hk K heads against Hq Q heads (the grouped K/V
 * heads of causal GQA; encoder-tower commit: per-head q/k RMSNorm, then
 * interleaved M-RoPE, then causal GQA).  q, q_out: [S, Hq, D]; k, k_out:
 * [S, Hk, D]; everything else as for h3a_qk_rmsnorm_rope, which is this call
 * with Hk = Hq.  Errors: as h3a_qk_rmsnorm_rope, plus EINVAL for Hk < 1.
 */
/*
 * RMSNorm + NeoX rotary of one tensor (the K half of h3a_qk_rmsnorm_rope, for
 * use with h3a_varlen_attn_fwd_qnorm, which does the Q half itself).
 * x, x_out: [S, H, D]; in place when x_out == x with the same stride;
 * gamma: fp32 [D].  Same arithmetic, shapes and errors as
 * h3a_qk_rmsnorm_rope.
 */
h3a_status h3a_rmsnorm_rope(const void* x, void* x_out, h3a_dtype dtype, int64_t S, int32_t H, int32_t D,
                            int64_t stride_x, int64_t stride_xo, const float* gamma, float eps,
                            const float* cos_sin, int32_t rot_dim, hipStream_t stream);

h3a_status h3a_qk_rmsnorm_rope_ex(const void* q, const void* k, void* q_out, void* k_out,
                                  h3a_dtype dtype, int64_t S, int32_t Hq, int32_t Hk, int32_t D,
                                  int64_t stride_q, int64_t stride_k, int64_t stride_qo,
                                  int64_t stride_ko, const float* gamma_q, const float* gamma_k,
                                  float eps, const float* cos_sin, int32_t rot_dim,
                                  hipStream_t stream);

/*
 * Bidirectional attention restricted to each packed segment.
 *
 * For segment s = [cu[s], cu[s+1]) and head h, every query row i in s gets
 *   o_i = sum_j softmax_j(scale * <q_i, k_j>) v_j,   j in s.
 * There are no cross-segment terms and no causal mask.  Empty segments are
 * legal and produce nothing.
 *
 * q, k, v        device [S, H, D] of `dtype` with token strides stride_q/k/v.
 * o              device [S, H, D] of `dtype`, token stride stride_o; must not
 *                overlap q, k or v.  Rows of every segment are written; there
 *                are no other rows (cu[nseg] == S).
 * cu_seqlens     HOST int32 [nseg+1]: cu[0] = 0, non-decreasing, cu[nseg] = S.
 *                It is planned on the host (tile work list, longest segments
 *                first, balanced over the chip's XCDs) and the plan is cached
 *                by content, so no device-to-host synchronisation happens.
 * scale          softmax scale (> 0 and finite), typically 1/sqrt(D).
 * Numerics: bf16 -- bf16 MFMA products with fp32 accumulation, fp32 online
 * softmax, probabilities rounded to bf16 for the PV product, output rounded
 * once; fp32 -- fp32 throughout.
 * Supported: D in {64, 128}; pointers 16-byte aligned; strides multiples of
 * 16 bytes, >= H*D and below 2^31 / 64 bytes; S <= INT32_MAX.
 *
 * Errors: EINVAL, ESHAPE, EDTYPE, EUNSUPPORTED, EHIP.
 */
h3a_status h3a_varlen_attn_fwd(const void* q, const void* k, const void* v, void* o,
                               h3a_dtype dtype, int64_t S, int32_t H, int32_t D,
                               int64_t stride_q, int64_t stride_k, int64_t stride_v,
                               int64_t stride_o, const int32_t* cu_seqlens, int32_t nseg,
                               float scale, hipStream_t stream);

/*
 * Bidirectional varlen attention whose Q rows arrive raw: each workgroup
 * RMS-normalises (gain gamma_q, eps) and rotates (cos_sin, rot_dim) its Q
 * tile in registers before the attention, so the Q half of the separate norm
 * + rotary pass disappears (the GB10 build fuses Q RMSNorm + rot96 RoPE into
 * its attention front end: h3-spark model card, "What this config does").
 * k must already be normalised and rotated (h3a_rmsnorm_rope).
 *
 * The result is bit-identical to h3a_qk_rmsnorm_rope followed by
 * h3a_varlen_attn_fwd(_ex): the fused prologue performs the same fp32
 * operations in the same order and rounds q' to bf16 once.
 *
 * q              device bf16 [S, Hq, D], raw (before norm and rotary); not
 *                modified.
 * k, v           device bf16 [S, Hkv, D]; Hkv divides Hq.
 * gamma_q        device fp32 [D], 16-byte aligned.
 * cos_sin        the [2][S][rot_dim/2] table; rot_dim a multiple of 32 and
 *                at most D (e.g. 96 for d = 128).
 * Everything else as for h3a_varlen_attn_fwd_ex with causal = 0.
 *
 * Errors: as h3a_varlen_attn_fwd_ex, plus EUNSUPPORTED for fp32 or a
 * rot_dim not a multiple of 32, EINVAL for a bad eps or null gamma/table.
 */
h3a_status h3a_varlen_attn_fwd_qnorm(const void* q, const void* k, const void* v, void* o, h3a_dtype dtype,
                                     int64_t S, int32_t Hq, int32_t Hkv, int32_t D, int64_t stride_q,
                                     int64_t stride_k, int64_t stride_v, int64_t stride_o,
                                     const int32_t* cu_seqlens, int32_t nseg, float scale, const float* gamma_q,
                                     float eps, const float* cos_sin, int32_t rot_dim, hipStream_t stream);

/*
 * Low-precision attention: FP8 E4M3 codes with per-block scales.
 *
 * The pages' GB10 builds run Q, K and V through low-precision attention
 * kernels quantised per block and calibrated on the activations themselves
 * (SageAttention 2++, Comfy Kitchen's INT8 attention; h3-spark model card,
 * runtime options and "What this config does"), after the Q RMSNorm + rot96
 * rotary.  Here every block of 32 elements along the contraction of a product
 * shares one power-of-two scale 2^X (an E8M0 code X + 127, one byte): 32 head
 * dims of one token and head for q and k, 32 keys of one head dim for v (key
 * blocks aligned at each segment's start).  X is the smallest integer with
 * max|x| * 2^-X <= 448 over the block, so no finite element saturates; X =
 * -127 for an all-zero block.  Each element is stored as the OCP FP8 E4M3
 * ("fn") code of x * 2^-X, round to nearest even; infinities saturate to
 * +-448 * 2^X and a NaN becomes an E4M3 NaN code (0x7f, 0xff), so NaN inputs
 * stay NaN through the FP8 attention as through the bf16 one.  The gfx950
 * scaled FP8 MFMA applies the scales inside the instruction.
 *
 * Scale arrays are caller-owned, packed and 2-byte (D = 64) or 4-byte
 * (D = 128) aligned.  q and k scales are head-major, q_scale [Hq][S][D/32]
 * and k_scale [Hk][S][D/32]: byte (h * S + n) * D/32 + b holds block b of
 * token n, head h, so the scales of a tile of consecutive keys are one
 * contiguous run.  For the transposed V layout vt_scale
 * [Hkv][vt_cols / 64][2][32][D/32] (block j of tile t, dim 32 b + r at
 * [h][t][j][r][b]).
 *
 * h3a_quantize_e4m3: bf16 x [S, H, D] (token stride stride_x elements) to
 *   codes y [S, H, D] (uint8, token stride stride_y bytes, a multiple of 16)
 *   and y_scale [H][S][D/32].  Errors: EINVAL (null, sizes, overlap),
 *   ESHAPE, EUNSUPPORTED, EHIP.
 */
h3a_status h3a_quantize_e4m3(const void* x, void* y, void* y_scale, int64_t S, int32_t H, int32_t D,
                             int64_t stride_x, int64_t stride_y, hipStream_t stream);

/*
 * Norm + rotary and quantisation in one HBM pass: h3a_qk_rmsnorm_rope_ex on
 * bf16 q [S, Hq, D] and k [S, Hk, D] writing codes q8 [S, Hq, D], k8
 * [S, Hk, D] (uint8, token strides stride_q8, stride_k8 in bytes, multiples
 * of 16) and scales q_scale, k_scale instead of bf16: each result is rounded
 * to bf16 first, so codes and scales equal h3a_qk_rmsnorm_rope_ex followed by
 * h3a_quantize_e4m3 (the GB10 build fuses Q RMSNorm + rot96 RoPE into its
 * attention's Q quantisation: h3-spark model card, "What this config does").
 * q and k are not modified.  Errors: as h3a_qk_rmsnorm_rope_ex (bf16 only).
 */
h3a_status h3a_qk_rmsnorm_rope_e4m3(const void* q, const void* k, void* q8, void* k8, void* q_scale, void* k_scale,
                                    int64_t S, int32_t Hq, int32_t Hk, int32_t D, int64_t stride_q, int64_t stride_k,
                                    int64_t stride_q8, int64_t stride_k8, const float* gamma_q, const float* gamma_k,
                                    float eps, const float* cos_sin, int32_t rot_dim, hipStream_t stream);

/*
 * h3a_varlen_attn_fwd_ex with q and k given as scaled E4M3 codes.  The score
 * product q.k runs on the scaled FP8 MFMA (twice the bf16 rate) with fp32
 * accumulation; the softmax, the bf16 probabilities, the PV product with
 * bf16 v and the bf16 output are those of the bf16 path.
 *
 * q8, q_scale    device uint8 [S, Hq, D] codes (token stride stride_q bytes,
 *                a multiple of 16) and their scales.
 * k8, k_scale    device uint8 [S, Hkv, D] codes (token stride stride_k bytes)
 *                and their scales.
 * v, o           device bf16 as for h3a_varlen_attn_fwd_ex.
 * The result equals attention on the block-scaled E4M3 values of q, k up to
 * the bf16 path's rounding.  Errors: as h3a_varlen_attn_fwd_ex, plus EINVAL /
 * EUNSUPPORTED for null or misaligned scale arrays.
 */
h3a_status h3a_varlen_attn_fwd_fp8qk(const void* q8, const void* k8, const void* q_scale, const void* k_scale,
                                     const void* v, void* o, int64_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                     int64_t stride_q, int64_t stride_k, int64_t stride_v, int64_t stride_o,
                                     const int32_t* cu_seqlens, int32_t nseg, float scale, int32_t causal,
                                     hipStream_t stream);

/*
 * Low-precision attention with both products in FP8.  V goes through a
 * layout pass first: vt8 [Hkv][D][vt_cols] holds E4M3 codes of v transposed
 * (rows are head dims), each segment padded to whole 64-key tiles: segment s
 * occupies columns col0(s) .. col0(s) + L_s - 1, col0(s) = sum over earlier
 * segments of ceil(L / 64) * 64, and padding columns hold code 0.
 *
 * h3a_vt_e4m3_columns: vt_cols for cu_seqlens (host only).
 * h3a_prepare_vt_e4m3: bf16 v [S, Hkv, D] (token stride stride_v elements)
 *   -> vt8 (device, Hkv * D * vt_cols bytes, 16-byte aligned) and vt_scale
 *   (Hkv * vt_cols * D / 32 bytes), blocks of 32 keys of each segment.
 * h3a_varlen_attn_fwd_fp8: as h3a_varlen_attn_fwd_fp8qk, with V given as
 *   vt8, vt_scale; the probabilities, offset by 2^4 against the running
 *   reference so the largest weights stay in E4M3's normal range, are rounded
 *   to E4M3 for the PV product (scaled FP8 MFMA, fp32 accumulation) and the
 *   row sum adds exactly those weights.  Against attention on the block-scaled
 *   E4M3 values of q, k, v with exact weights the result carries the E4M3
 *   rounding of the weights.
 * Errors: as h3a_varlen_attn_fwd_fp8qk, plus ESHAPE for a vt_cols that does
 * not match cu_seqlens and EUNSUPPORTED when D * vt_cols exceeds INT32_MAX.
 */
h3a_status h3a_vt_e4m3_columns(const int32_t* cu_seqlens, int32_t nseg, int64_t* columns);
h3a_status h3a_prepare_vt_e4m3(const void* v, void* vt8, void* vt_scale, int64_t S, int32_t Hkv, int32_t D,
                               int64_t stride_v, int64_t vt_cols, const int32_t* cu_seqlens, int32_t nseg,
                               hipStream_t stream);
h3a_status h3a_varlen_attn_fwd_fp8(const void* q8, const void* k8, const void* vt8, const void* q_scale,
                                   const void* k_scale, const void* vt_scale, void* o, int64_t S, int32_t Hq,
                                   int32_t Hkv, int32_t D, int64_t stride_q, int64_t stride_k, int64_t vt_cols,
                                   int64_t stride_o, const int32_t* cu_seqlens, int32_t nseg, float scale,
                                   int32_t causal, hipStream_t stream);


/*
 * INT8 score product, after the pages' INT8 Q/K attention (Comfy Kitchen's
 * INT8 Q/K/V kernel and a Sol-Attn INT8 QK switch among the request-level
 * attention backends: H3 Blackwell Runtime README, "Hot Runtime Service";
 * the "Sage Q-INT8" tail of the fused Q norm + rotary: h3-spark model card,
 * "What this config does").  q has one fp32 scale per token and head, k one
 * per block of 64 keys of a segment and head (blocks aligned at the segment
 * start, a segment's last one possibly shorter, numbered segment by segment:
 * block j of segment s is sum over earlier segments of ceil(L / 64), plus j).
 * With amax a block's largest magnitude: scale = amax / 127 and code =
 * rint(x * (127 / amax)) clamped to [-127, 127], in fp32 with correctly
 * rounded divisions; a zero block has scale 0 and codes 0; a block holding a
 * NaN or an infinity gets a NaN or infinite scale and codes 0, so its scores
 * become NaN.
 *
 * h3a_quantize_i8_rows: bf16 x [S, H, D] (token stride stride_x elements) ->
 *   codes y [S, H, D] (int8, token stride stride_y bytes, a multiple of 16)
 *   and y_scale [H][S] fp32 (4-byte aligned).
 * h3a_i8_key_blocks: the number of 64-key blocks of cu_seqlens (host only).
 * h3a_quantize_i8_keys: as h3a_quantize_i8_rows with y_scale [H][n_blocks]
 *   fp32, one scale per key block of each head; n_blocks must equal
 *   h3a_i8_key_blocks (else ESHAPE).
 * h3a_varlen_attn_fwd_i8qk: h3a_varlen_attn_fwd_ex with q8 / q_scale from
 *   h3a_quantize_i8_rows (Hq heads) and k8 / k_scale from
 *   h3a_quantize_i8_keys (Hkv heads) on the same cu_seqlens.  The score
 *   product runs on the INT8 MFMA (int32 sums, exact), each score is the sum
 *   times q scale * k scale * scale; the softmax, the bf16 probabilities, the
 *   PV product with bf16 v and the bf16 output are those of the bf16 path.
 *   The result equals attention on the values the codes stand for (code *
 *   scale) up to the bf16 path's rounding.  Errors: as
 *   h3a_varlen_attn_fwd_fp8qk, plus EUNSUPPORTED when the segments' padded
 *   64-key blocks cover more than INT32_MAX keys.
 */
h3a_status h3a_quantize_i8_rows(const void* x, void* y, void* y_scale, int64_t S, int32_t H, int32_t D,
                                int64_t stride_x, int64_t stride_y, hipStream_t stream);
h3a_status h3a_i8_key_blocks(const int32_t* cu_seqlens, int32_t nseg, int64_t* n_blocks);

/*
 * Norm + rotary and the q quantisation in one HBM pass (the fused "Sage
 * Q-INT8" tail of the GB10 build's Q RMSNorm + rot96 RoPE: h3-spark model
 * card, "What this config does"): h3a_qk_rmsnorm_rope_ex on bf16 q [S, Hq, D]
 * and k [S, Hk, D], writing q as INT8 codes q8 [S, Hq, D] (token stride
 * stride_q8 bytes, a multiple of 16) with q_scale [Hq][S] fp32, and k as bf16
 * k_out [S, Hk, D] (token stride stride_ko elements; k_out may be k itself)
 * for h3a_quantize_i8_keys.  Each q result is rounded to bf16 first, so codes
 * and scales equal h3a_qk_rmsnorm_rope_ex followed by h3a_quantize_i8_rows,
 * and k_out equals its k result.  q is not modified.  Errors: as
 * h3a_qk_rmsnorm_rope_ex (bf16 only), plus EINVAL when q8 or q_scale overlaps
 * another tensor.
 */
h3a_status h3a_qk_rmsnorm_rope_i8q(const void* q, const void* k, void* q8, void* k_out, void* q_scale,
                                   int64_t S, int32_t Hq, int32_t Hk, int32_t D, int64_t stride_q, int64_t stride_k,
                                   int64_t stride_q8, int64_t stride_ko, const float* gamma_q, const float* gamma_k,
                                   float eps, const float* cos_sin, int32_t rot_dim, hipStream_t stream);
h3a_status h3a_quantize_i8_keys(const void* x, void* y, void* y_scale, int64_t S, int32_t H, int32_t D,
                                int64_t stride_x, int64_t stride_y, int64_t n_blocks, const int32_t* cu_seqlens,
                                int32_t nseg, hipStream_t stream);

/*
 * Centred keys for the INT8 scores (SageAttention's K smoothing, SageAttention
 * being among the GB10 build's attention backends: H3 Blackwell Runtime
 * README, attention backends).  Within one segment every query's scores move
 * by the same q . mean when the segment's mean key is subtracted from k, which
 * the softmax cancels; K's per-channel offsets then no longer set the INT8
 * block scales.
 *
 * h3a_i8_key_mean_chunks: the number of 256-key chunks of cu_seqlens (each
 *   segment's counted from its start; host only).
 * h3a_segment_key_means: mu [nseg][H][D] fp32 = the mean of bf16 k [S, H, D]
 *   (token stride stride_k elements) over each segment's keys, 0 for an empty
 *   segment, through the caller's workspace partial [n_chunks][H][D] fp32
 *   (n_chunks from h3a_i8_key_mean_chunks, else ESHAPE).  Sums are taken in
 *   fp32 in a fixed order (bitwise deterministic), then divided by the
 *   segment length.  mu and partial are 4-byte aligned and overlap nothing.
 * h3a_quantize_i8_keys_centered: h3a_quantize_i8_keys on the fp32
 *   differences x - mu[segment] (mu 16-byte aligned, not overlapping y or
 *   y_scale); the codes and scales stand for the centred keys, and
 *   h3a_varlen_attn_fwd_i8qk / _i8qk_fp8pv take them unchanged.
 */
h3a_status h3a_i8_key_mean_chunks(const int32_t* cu_seqlens, int32_t nseg, int64_t* n_chunks);
h3a_status h3a_segment_key_means(const void* k, void* partial, void* mu, int64_t S, int32_t H, int32_t D,
                                 int64_t stride_k, int64_t n_chunks, const int32_t* cu_seqlens, int32_t nseg,
                                 hipStream_t stream);
h3a_status h3a_quantize_i8_keys_centered(const void* x, const void* mu, void* y, void* y_scale, int64_t S, int32_t H,
                                         int32_t D, int64_t stride_x, int64_t stride_y, int64_t n_blocks,
                                         const int32_t* cu_seqlens, int32_t nseg, hipStream_t stream);
h3a_status h3a_varlen_attn_fwd_i8qk(const void* q8, const void* k8, const void* q_scale, const void* k_scale,
                                    const void* v, void* o, int64_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                    int64_t stride_q, int64_t stride_k, int64_t stride_v, int64_t stride_o,
                                    const int32_t* cu_seqlens, int32_t nseg, float scale, int32_t causal,
                                    hipStream_t stream);

/*
 * INT8 scores with the PV product in FP8 (SageAttention 2's split of the two
 * products, named by the pages among the GB10 build's attention backends:
 * H3 Blackwell Runtime README, attention backends): q8 / q_scale and k8 /
 * k_scale as for h3a_varlen_attn_fwd_i8qk, v as the transposed E4M3 layout
 * vt8 / vt_scale of h3a_prepare_vt_e4m3 (vt_cols from h3a_vt_e4m3_columns,
 * whose 64-key column blocks are also k_scale's key blocks).  The weights are
 * formed and rounded as for h3a_varlen_attn_fwd_fp8.  The result equals
 * attention on the values the codes stand for up to the rounding of the
 * weights to E4M3 and the bf16 output.  Errors: as h3a_varlen_attn_fwd_fp8.
 */
h3a_status h3a_varlen_attn_fwd_i8qk_fp8pv(const void* q8, const void* k8, const void* vt8, const void* q_scale,
                                          const void* k_scale, const void* vt_scale, void* o, int64_t S, int32_t Hq,
                                          int32_t Hkv, int32_t D, int64_t stride_q, int64_t stride_k, int64_t vt_cols,
                                          int64_t stride_o, const int32_t* cu_seqlens, int32_t nseg, float scale,
                                          int32_t causal, hipStream_t stream);

/*
 * Varlen attention with grouped K/V heads and an optional causal mask: the
 * encoder text tower's causal GQA (vllm.cpp PR #26, encoder-tower commit,
 * "Causal GQA attention": K/V heads are broadcast across their query group).
 *
 * q, o           device [S, Hq, D] of `dtype`, token strides stride_q/o.
 * k, v           device [S, Hkv, D] of `dtype`, token strides stride_k/v
 *                (>= Hkv*D).  Hkv >= 1 divides Hq; query head h attends
 *                with K/V head h / (Hq / Hkv).
 * causal         0: bidirectional within each segment (exactly
 *                h3a_varlen_attn_fwd when Hkv == Hq).  1: query row i of a
 *                segment sees the segment's keys 0..i (the mask is aligned at
 *                the segment start).
 * Everything else -- cu_seqlens, scale, numerics, supported shapes, plan
 * cache -- as for h3a_varlen_attn_fwd.
 *
 * Errors: as h3a_varlen_attn_fwd, plus EINVAL (Hkv < 1, causal not 0/1) and
 * ESHAPE (Hkv does not divide Hq).
 */
h3a_status h3a_varlen_attn_fwd_ex(const void* q, const void* k, const void* v, void* o,
                                  h3a_dtype dtype, int64_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                  int64_t stride_q, int64_t stride_k, int64_t stride_v,
                                  int64_t stride_o, const int32_t* cu_seqlens, int32_t nseg,
                                  float scale, int32_t causal, hipStream_t stream);

/*
 * The attention tile plan, on the host only (no GPU needed); for tests and
 * tooling.  Writes up to `cap` items of 4 int32 each -- (segment start,
 * segment length, first query row relative to the segment start, head); an
 * item with length 0 is padding -- in launch order, and sets *n_items to the
 * plan's length (the attention grid size).  block_m is the query rows per
 * item (128 for bf16, 64 for fp32); n_xcd the number of XCDs to balance over
 * (>= 1).  Errors: EINVAL, ESHAPE (cap too small: *n_items still set).
 */
h3a_status h3a_plan_tiles(const int32_t* cu_seqlens, int32_t nseg, int32_t H, int32_t block_m,
                          int32_t n_xcd, int32_t* items, int64_t cap, int64_t* n_items);

/* h3a_plan_tiles for the causal variant (causal = 1: an item costs the keys
 * up to its last row, and each chunk of one segment and head lists its
 * query tiles last to first).  causal = 0 is h3a_plan_tiles. */
h3a_status h3a_plan_tiles_ex(const int32_t* cu_seqlens, int32_t nseg, int32_t H, int32_t block_m,
                             int32_t n_xcd, int32_t causal, int32_t* items, int64_t cap, int64_t* n_items);

/*
 * h3a_varlen_attn_fwd_ex without device allocation, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, validation, kernels and
 * output bytes as h3a_varlen_attn_fwd_ex; the only difference is where the
 * attention's tile plan (its work queue) lives.
 *
 * The plan goes into a fixed array in device memory that the library
 * reserves for this call, 2 MiB on each GPU it runs on, held until the
 * process ends; nothing is allocated, freed or cached per call, and the
 * call never synchronises the host.  The plan is built on `stream` from a
 * per-segment table (segments longest first, query tiles dealt to the XCDs
 * in chunks of 16; no per-XCD balancing as in the cached plan).
 *
 * Limits: at most 256 non-empty segments and 65,536 work items (one item is
 * 128 query rows of one head in bf16, 64 in fp32; the item count is padded up
 * to a multiple of 16 per XCD): e.g. S * H up to ~8.3M rows in bf16.  Beyond
 * them the call fails with EUNSUPPORTED before touching the device.
 *
 * Sharing: every call on one GPU uses that GPU's array; it keeps the last
 * call's plan.  Calls are ordered through it on the GPU (each waits, on its
 * stream, for the previous call's attention kernel, whatever stream that ran
 * on), so overlapping calls on one GPU do not corrupt each other but do not
 * run concurrently either.  The first call on a device resolves the array's
 * address and creates one event (set-up, once per device).
 * Errors: as h3a_varlen_attn_fwd_ex, plus the limits above.
 */
h3a_status h3a_varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, h3a_dtype dtype,
                                       int64_t S, int32_t Hq, int32_t Hkv, int32_t D, int64_t stride_q,
                                       int64_t stride_k, int64_t stride_v, int64_t stride_o,
                                       const int32_t* cu_seqlens, int32_t nseg, float scale, int32_t causal,
                                       hipStream_t stream);

/* Message of the last failed call on this thread ("" if none). */
const char* h3a_last_error(void);

/* Frees every cached attention plan, pinned ones included, after waiting for
 * each device that holds one (attention kernels launched earlier may still
 * read it).  If a device cannot be synchronised, nothing is freed.  Calls on
 * other threads wait.  A graph that captured an attention call must not be
 * replayed after this (its plan is gone); capture it again. */
void h3a_release_caches(void);

/* Key-range splitting of attention plans (the bf16-tile kernels: bf16, fused
 * Q norm, FP8; bidirectional plans only).  When a packing has few, long work
 * items -- fewer (segment, head, query tile) items than the GPU has workgroup
 * slots, or whole rounds of long items that leave slots idle at the end --
 * an item's keys can be cut into ranges of whole 64-key tiles, each range its
 * own work item storing its unnormalised rows with their running max and row
 * sum; a merge kernel then combines the ranges of each item in key order, as
 * the streaming softmax itself combines tiles (each packing's vllm.cpp PR #26
 * cu_seqlens call stays one call: the split is internal).  Results are
 * deterministic run to run; they differ from the unsplit kernel's only by
 * fp32 rounding of the combination.
 *
 * policy: H3A_SPLIT_AUTO (default) splits when a list-scheduling estimate of
 * the kernel time, charging the merge pass for reading every partial result
 * back, improves by more than 10%; H3A_SPLIT_NEVER never; H3A_SPLIT_ALWAYS
 * cuts every item of four or more key tiles into about three ranges (for
 * tests); a plan that would need more than 16,384 partial results (1.1 GB of
 * workspace) stays unsplit.  The policy applies to plans built afterwards; cached plans keep
 * theirs (they are keyed by it).  Calls under stream capture always use the
 * unsplit items of a cached plan, so a graph never holds the shared partial
 * workspace; calls outside capture that use one plan's split items are
 * ordered on the GPU (each waits for the previous one's merge).
 * Errors: EINVAL for an unknown policy. */
typedef enum { H3A_SPLIT_AUTO = 0, H3A_SPLIT_NEVER = 1, H3A_SPLIT_ALWAYS = 2 } h3a_split_policy;
h3a_status h3a_set_split_policy(int32_t policy);

/* Library version, major * 10000 + minor * 100 + patch (0.2.0). */
int32_t h3a_version(void);

#ifdef __cplusplus
}
#endif

#endif /* H3A_H */
