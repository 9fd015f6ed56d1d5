/*
 * convrot.h -- C ABI of the MI355X (gfx950) ConvRot quantized linear.
 *
 * The method (sources: the "SAM 3.1 Multiplex INT8/INT4 ConvRot" release page, section
 * "Quantization recipe"; the "TRELLIS.2 INT8 ConvRot in ComfyUI" guide, section "What ConvRot
 * changes"; the "Explanation of INT8 ConvRot" article, format taxonomy):
 *   offline  W[N,K] --(FP32 upcast, block-Hadamard rotation along K)--> per-row absmax
 *            scale w_scale[N] and INT8 / INT4 codes Wq;
 *   online   X[M,K] --(the matching rotation, dynamic per-token quantization)--> Xq, x_scale;
 *            acc = Xq * Wq^T in int32; Y = fp16/bf16( f32(acc) * (w_scale[n]*x_scale[m]) + bias[n] ).
 *
 * Numerics (exact; every output is reproducible bit for bit on the CPU):
 *   rotation   per 128-wide block of K: unnormalized Walsh-Hadamard transform in fp32 with the
 *              butterfly stages h = 1, 2, 4, ..., 64 in this order (Sylvester order, no signs);
 *              the 1/sqrt(128) normalization is folded into the scale.
 *   scale      a = max |u| over the whole row, inv = fl(q_max / a); q_max = 127 (8-bit) or
 *              7 (4-bit). a == 0, or a so small that inv is +inf (a below about
 *              q_max * 2^-128, reachable from bf16 / f32 inputs only) -> scale 0 and codes 0:
 *              the row is quantized as a zero row. Else scale = fl(fl(a * fl(1/sqrt 128)) /
 *              q_max), code = round_half_even(fl(u * inv)).
 *   storage    8-bit: int8 [rows, K]; 4-bit: uint8 [rows, K/2], two's-complement nibbles,
 *              low nibble = even k.
 *   activation code layouts (rq_qconfig.x_layout):
 *              RQ_X_ROWS   row-major as above, rows * Kb bytes (Kb = K or K/2 bytes per row);
 *              RQ_X_TILED  the GEMM's tile order: 256-row panels, each split into 64-byte
 *                          k steps stored as [panel][step][256 rows][64 B]. Byte b of row m
 *                          sits at ((m / 256 * (Kb / 64) + b / 64) * 256 + m % 256) * 64 + b % 64.
 *                          Rows are padded to a multiple of 256 (pad rows hold no defined value
 *                          and are never used); rq_codes_bytes() gives the size. The GEMM's
 *                          operand loads are then whole contiguous 1 KB blocks.
 *              RQ_X_FP6    4-bit codes as FP6 tiles (below), 256-row panels.
 *   weight code layouts (rq_qconfig.w_layout):
 *              RQ_W_ROWS   row-major int8 [N, K] / packed int4 [N, K/2];
 *              RQ_W_FP6    4-bit codes as FP6 tiles, 128-row panels; rq_weight_bytes() gives
 *                          the size. The GEMM then runs on the FP6 matrix cores (below).
 *   FP6 tiles  Every 4-bit code q in [-7, 7] is exactly an FP6 E2M3 value (sign bit 5, exponent
 *              bits 4..3 with bias 1, mantissa bits 2..0): 0 -> 0, 1 -> 8, 2 -> 16, 3 -> 20,
 *              4 -> 24, 5 -> 26, 6 -> 28, 7 -> 30, plus 32 for negative codes. Products of two
 *              codes and their sums stay exact integers in fp32 (|acc| <= 49 K < 2^24), so the
 *              FP6 MFMA gives the int32 accumulator exactly, at twice the int8 rate. Layout, for
 *              a panel height P: K is split into 64-code slices; slice s of rows
 *              [pP, pP + P) is one block of P * 48 bytes at ((p * K/64) + s) * P * 48. Within a
 *              row, the slice's codes 32h .. 32h + 31 (h = 0, 1) form a 24-byte string (code e
 *              of the half at bits 6e .. 6e+5, little-endian). Bytes 0..15 of half h of tile row
 *              r sit in plane 1 at r * 32 + 16 * (h ^ (r >> 3 & 1)); bytes 16..23 in plane 2,
 *              which starts at P * 32, at r * 16 + 8 * (h ^ (r >> 4 & 1)). Pad rows hold no
 *              defined value and are never used.
 *   epilogue   y = fma(f32(acc), fl(w_scale[n] * x_scale[m]), bias[n] or +0), rounded to
 *              nearest-even fp16 / bf16.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major, owned by the caller. The library
 *     allocates nothing and keeps no state between calls (apart from the static scratch of
 *     rq_rotq_linear_noalloc, below); it is safe to call from several host threads as long as
 *     concurrent calls do not share output buffers or workspaces.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream). Outputs are
 *     valid once the stream has been synchronized. Inputs must stay alive until then.
 *   - Every argument is validated on the host BEFORE any launch; a failed check launches nothing
 *     and returns a status code (never a silent fallback). A launch failure returns RQ_EHIP.
 *     rq_last_error_detail() describes the most recent failure on the calling thread.
 *   - Inputs must be finite; NaN / Inf inputs give unspecified codes.
 *   - Alignment: every tensor pointer must be 16-byte aligned.
 *   - Limits: K % 128 == 0 and 128 <= K <= 131072; N % 16 == 0; M >= 0 (M == 0 is a no-op);
 *     M, N < 2^31. The K bound keeps every int32 accumulator exact: 127^2 * K < 2^31, and the
 *     4-bit path, which accumulates 256 * acc, has 256 * 7^2 * K < 2^31 for the codes the
 *     quantizer emits (rq_gemm_s32 also accepts the nibble -8; a dot product in which all
 *     131072 products are (-8) * (-8) is the one input that does not fit).
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RQ_OK = 0,            /* success (work enqueued on the stream) */
  RQ_EINVAL = 1,        /* NULL / misaligned pointer, negative size, bad dtype, aliasing */
  RQ_EUNSUPPORTED = 2,  /* a shape or configuration outside the limits above */
  RQ_EWORKSPACE = 3,    /* workspace smaller than rq_rotq_linear_workspace_size() */
  RQ_EHIP = 4           /* the HIP runtime reported an error at launch */
} rq_status;

typedef enum { RQ_F32 = 0, RQ_F16 = 1, RQ_BF16 = 2 } rq_dtype;

enum { RQ_ROT_WHT = 1 };   /* normalized Walsh-Hadamard rotation, Sylvester order */

enum { RQ_X_ROWS = 0, RQ_X_TILED = 1, RQ_X_FP6 = 2 };   /* activation code layouts (see above) */
enum { RQ_W_ROWS = 0, RQ_W_FP6 = 1 };                   /* weight code layouts (see above) */

/* Weight-scale rules of rq_quantize_weights. Each picks a clipping threshold t per row and
 * then quantizes exactly as above with a replaced by t: inv = fl(q_max / t),
 * scale = fl(fl(t * fl(1/sqrt 128)) / q_max), code = clamp(round_half_even(fl(u * inv)),
 * -q_max, q_max); t = 0, or a t whose inv is +inf, gives scale 0 and codes 0 (the zero-row
 * rule above; in RQ_W_MSE such a candidate is the all-zero quantization of the row).
 *   RQ_W_ABSMAX   t = a = max |u| of the row (the default; the rule of the activations).
 *   RQ_W_MSE      MSE-optimized clipping ("Quantization recipe", step 3: the converter picks
 *                 the clipping scale with the least squared error). t = fl(a * alpha_i),
 *                 alpha_i = fl((100 - i) / 100), i = 0..50, minimizing
 *                 E_i = sum_k (u_k * fl(1/sqrt 128) - scale_i * code_ik)^2, evaluated in
 *                 binary64 in increasing k (the two products exact, the difference, square and
 *                 running sum each rounded to nearest); ties keep the smaller i (larger alpha).
 *   RQ_W_TENSOR   tensor-wise scale (the int8_tensorwise variant of the HSWQ ConvRot model
 *                 card): t = max |u| over the whole rotated matrix, so every row gets the same
 *                 scale. The GEMM is unchanged: w_scale[n] is simply constant. */
enum { RQ_W_ABSMAX = 0, RQ_W_MSE = 1, RQ_W_TENSOR = 2 };

/* Activation fused into the epilogue, for the first linear of an MLP pair (the "SAM 3.1
 * Multiplex INT8/INT4 ConvRot" page, "Future improvements": larger gains from fusing
 * operations and cutting dispatches; the pages do not name the MLP's activation). With v the
 * binary32 epilogue value fma(f32(acc), fl(s_w * s_x), bias), the stored value is
 * round_to_nearest_even(GELU(v)) in fp16/bf16, GELU evaluated in binary32 with the device math
 * library as
 *   RQ_ACT_GELU_ERF   0.5 v erfc(-v / sqrt 2)                    (= v * Phi(v), the erf form)
 *   RQ_ACT_GELU_TANH  v * logistic(2u), u = sqrt(2/pi) (v + 0.044715 v^3)   (the tanh form,
 *                     0.5 v (1 + tanh u)), the logistic as 1/(1+e) or e/(1+e), e = exp(-2|u|)
 * which is within a few binary32 ulps of the exact value: the output is the correctly rounded
 * GELU except, rarely, one ulp away next to a rounding midpoint. RQ_ACT_NONE stores v itself. */
enum { RQ_ACT_NONE = 0, RQ_ACT_GELU_ERF = 1, RQ_ACT_GELU_TANH = 2 };

typedef struct {
  int32_t bits;       /* 8 (W8A8) or 4 (W4A4) */
  int32_t rot_kind;   /* must be RQ_ROT_WHT */
  int32_t rot_block;  /* must be 128 */
  int32_t x_layout;   /* RQ_X_ROWS or RQ_X_TILED: layout of Xq in rq_rotate_quantize,
                         rq_gemm_dequant and rq_gemm_s32 (rq_quantize_weights ignores it;
                         rq_rotq_linear always uses RQ_X_TILED inside its workspace) */
  int32_t w_scale_mode; /* RQ_W_ABSMAX, RQ_W_MSE or RQ_W_TENSOR: the scale rule of
                           rq_quantize_weights (every other entry point ignores it) */
  int32_t w_layout;     /* RQ_W_ROWS or RQ_W_FP6 (bits 4 only): layout of Wq for
                           rq_quantize_weights, rq_rotq_linear and the GEMM entry points. The
                           GEMM entry points need x_layout == RQ_X_FP6 exactly when w_layout is
                           RQ_W_FP6; rq_rotq_linear picks its workspace layout to match. */
  int32_t act;          /* RQ_ACT_NONE, RQ_ACT_GELU_ERF or RQ_ACT_GELU_TANH: activation applied
                           by the epilogue of rq_rotq_linear and rq_gemm_dequant to each fp32
                           value before its fp16/bf16 rounding (below); ignored by the other
                           entry points. */
} rq_qconfig;

/* Bytes of activation codes for `rows` rows of length K in cfg's bits and x_layout
 * (0 if cfg is invalid or the sizes are out of range). */
size_t rq_codes_bytes(int64_t rows, int64_t K, const rq_qconfig *cfg);

/* Bytes of weight codes for N rows of length K in cfg's bits and w_layout (0 if cfg is invalid
 * or the sizes are out of range). */
size_t rq_weight_bytes(int64_t N, int64_t K, const rq_qconfig *cfg);

/* Offline weight quantizer ("Quantization recipe": upcast to FP32, block-Hadamard transform,
 * per-row scales), with the scale rule cfg->w_scale_mode.
 *   W        [N, K] device, dtype w_dtype (RQ_F32, RQ_F16 or RQ_BF16)
 *   Wq       out: rq_weight_bytes(N, K, cfg) bytes in cfg->w_layout: int8 [N, K] (bits 8) or
 *            uint8 [N, K/2] (bits 4) row-major, or FP6 tiles
 *   w_scale  out: float [N] (RQ_W_TENSOR also uses it as scratch between its kernels)
 * Returns RQ_OK or a status; see the conventions above. */
rq_status rq_quantize_weights(const void *W, int32_t w_dtype, int64_t N, int64_t K,
                              const rq_qconfig *cfg, void *Wq, float *w_scale, void *stream);

/* Online activation rotate + quantize alone (the first kernel of rq_rotq_linear), with the
 * same arithmetic as rq_quantize_weights ("What ConvRot changes": the matching rotation is
 * applied to activations at run time; "Quantization recipe": dynamic activation quantization).
 *   X        [M, K] device, dtype x_dtype (RQ_F32, RQ_F16 or RQ_BF16)
 *   Xq       out: rq_codes_bytes(M, K, cfg) bytes in cfg->x_layout: int8 [M, K] (bits 8) or
 *            uint8 [M, K/2] (bits 4) row-major, or the tiled layout
 *   x_scale  out: float [M] (one scale per token) */
rq_status rq_rotate_quantize(const void *X, int32_t x_dtype, int64_t M, int64_t K,
                             const rq_qconfig *cfg, void *Xq, float *x_scale, void *stream);

/* Bytes of device workspace rq_rotq_linear needs: Xq in RQ_X_TILED layout (RQ_X_FP6 when
 * cfg->w_layout is RQ_W_FP6; rq_codes_bytes(M, K) with that x_layout) followed by x_scale [M],
 * each rounded up to 256 bytes. Returns 0 if cfg is invalid. */
size_t rq_rotq_linear_workspace_size(int64_t M, int64_t K, const rq_qconfig *cfg);

/* The quantized linear ("Quantization recipe": W8A8 / W4A4 operations with online activation
 * quantization; "What ConvRot changes"): rotate + quantize X, int8 MFMA GEMM against Wq,
 * fused dequantize + bias + fp16/bf16 store.
 *   X         [M, K] device, x_dtype RQ_F16 or RQ_BF16
 *   Wq        codes in cfg->w_layout (from rq_quantize_weights with the same cfg)
 *   w_scale   [N] float
 *   bias      [N] float, or NULL (no bias)
 *   Y         out: [M, N], same dtype as X, after cfg->act; must not overlap X, Wq or the
 *             workspace
 *   workspace device buffer of ws_bytes >= rq_rotq_linear_workspace_size(M, K, cfg) */
rq_status rq_rotq_linear(const void *X, int32_t x_dtype, int64_t M, int64_t K,
                         const void *Wq, const float *w_scale, int64_t N, const float *bias,
                         const rq_qconfig *cfg, void *Y, void *workspace, size_t ws_bytes,
                         void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): rq_rotq_linear without a workspace argument. The
 * workspace is a static device array of RQ_NOALLOC_SCRATCH_BYTES inside the library, one per
 * GPU, held until the process ends; its address is looked up (hipGetSymbolAddress) on the first
 * call on each device, with that device current. The call allocates nothing and runs the same
 * kernels as rq_rotq_linear, on the current device (`stream` must belong to it).
 *   Limit: rq_rotq_linear_workspace_size(M, K, cfg) <= RQ_NOALLOC_SCRATCH_BYTES (64 MiB: every
 *   workload shape here, e.g. 41472 x 1024 or 8192 x 6144 8-bit codes); a larger call returns
 *   RQ_EWORKSPACE and launches nothing.
 *   Every call on one GPU shares that GPU's array, which keeps the last call's contents:
 *   calls that overlap in time on one GPU (several host threads or streams) race. Nothing in
 *   it needs to start at zero (each call writes all it reads).
 * Other arguments, layouts, statuses and the output: as rq_rotq_linear. */
#define RQ_NOALLOC_SCRATCH_BYTES (64u << 20)
rq_status rq_rotq_linear_noalloc(const void *X, int32_t x_dtype, int64_t M, int64_t K,
                                 const void *Wq, const float *w_scale, int64_t N,
                                 const float *bias, const rq_qconfig *cfg, void *Y, void *stream);

/* The GEMM + epilogue alone (the second kernel of rq_rotq_linear).
 *   Xq codes of M rows in cfg->x_layout (as rq_rotate_quantize writes them), x_scale [M];
 *   Wq, w_scale, bias as above;
 *   Y  out: [M, N] of y_dtype (RQ_F16 or RQ_BF16), after cfg->act. */
rq_status rq_gemm_dequant(const void *Xq, const float *x_scale, const void *Wq,
                          const float *w_scale, const float *bias, int64_t M, int64_t N,
                          int64_t K, const rq_qconfig *cfg, void *Y, int32_t y_dtype,
                          void *stream);

/* The exact int32 accumulators acc[M, N] = sum_k Xq[m,k] * Wq[n,k] (for bit-exact checks);
 * Xq in cfg->x_layout. For every shape, bits and layout this runs the kernel, launch geometry
 * and mainloop that rq_gemm_dequant runs with cfg->act == RQ_ACT_NONE (and so rq_rotq_linear,
 * whose codes are in RQ_X_TILED or RQ_X_FP6), with the int32 store in place of the epilogue. */
rq_status rq_gemm_s32(const void *Xq, const void *Wq, int64_t M, int64_t N, int64_t K,
                      const rq_qconfig *cfg, int32_t *acc, void *stream);

/* Host-only validation of rq_rotq_linear's arguments (no HIP call, no launch): returns the
 * status rq_rotq_linear would return before launching. Pointers are only compared and
 * checked for NULL / alignment, never dereferenced. */
rq_status rq_check_rotq_linear_args(const void *X, int32_t x_dtype, int64_t M, int64_t K,
                                    const void *Wq, const float *w_scale, int64_t N,
                                    const float *bias, const rq_qconfig *cfg, const void *Y,
                                    const void *workspace, size_t ws_bytes);

/* Static text for a status code. */
const char *rq_status_string(rq_status s);

/* Human-readable detail of the last non-OK status returned on the calling thread. */
const char *rq_last_error_detail(void);

/* Library version, e.g. "0.1.0". */
const char *rq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
