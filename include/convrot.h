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
 *   scale      a = max |u| over the whole row; a == 0 -> scale 0, codes 0;
 *              else inv = fl(q_max / a), scale = fl(fl(a * fl(1/sqrt 128)) / q_max),
 *              code = round_half_even(fl(u * inv)); q_max = 127 (8-bit) or 7 (4-bit).
 *   storage    8-bit: int8 [rows, K]; 4-bit: uint8 [rows, K/2], two's-complement nibbles,
 *              low nibble = even k.
 *   epilogue   y = fma(f32(acc), fl(w_scale[n] * x_scale[m]), bias[n] or +0), rounded to
 *              nearest-even fp16 / bf16.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major, owned by the caller. The library
 *     allocates nothing and keeps no state between calls; it is safe to call from several host
 *     threads as long as concurrent calls do not share output buffers or workspaces.
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

typedef struct {
  int32_t bits;       /* 8 (W8A8) or 4 (W4A4) */
  int32_t rot_kind;   /* must be RQ_ROT_WHT */
  int32_t rot_block;  /* must be 128 */
} rq_qconfig;

/* Offline weight quantizer ("Quantization recipe": upcast to FP32, block-Hadamard transform,
 * per-row scales).
 *   W        [N, K] device, dtype w_dtype (RQ_F32, RQ_F16 or RQ_BF16)
 *   Wq       out: int8 [N, K] (bits 8) or uint8 [N, K/2] (bits 4)
 *   w_scale  out: float [N]
 * Returns RQ_OK or a status; see the conventions above. */
rq_status rq_quantize_weights(const void *W, int32_t w_dtype, int64_t N, int64_t K,
                              const rq_qconfig *cfg, void *Wq, float *w_scale, void *stream);

/* Online activation rotate + quantize alone (the first kernel of rq_rotq_linear), with the
 * same arithmetic as rq_quantize_weights ("What ConvRot changes": the matching rotation is
 * applied to activations at run time; "Quantization recipe": dynamic activation quantization).
 *   X        [M, K] device, dtype x_dtype (RQ_F32, RQ_F16 or RQ_BF16)
 *   Xq       out: int8 [M, K] (bits 8) or uint8 [M, K/2] (bits 4)
 *   x_scale  out: float [M] (one scale per token) */
rq_status rq_rotate_quantize(const void *X, int32_t x_dtype, int64_t M, int64_t K,
                             const rq_qconfig *cfg, void *Xq, float *x_scale, void *stream);

/* Bytes of device workspace rq_rotq_linear needs: Xq followed by x_scale, each rounded up to
 * 256 bytes. Returns 0 if cfg is invalid. */
size_t rq_rotq_linear_workspace_size(int64_t M, int64_t K, const rq_qconfig *cfg);

/* The quantized linear ("Quantization recipe": W8A8 / W4A4 operations with online activation
 * quantization; "What ConvRot changes"): rotate + quantize X, int8 MFMA GEMM against Wq,
 * fused dequantize + bias + fp16/bf16 store.
 *   X         [M, K] device, x_dtype RQ_F16 or RQ_BF16
 *   Wq        [N, K] int8 or [N, K/2] uint8 (from rq_quantize_weights with the same cfg)
 *   w_scale   [N] float
 *   bias      [N] float, or NULL (no bias)
 *   Y         out: [M, N], same dtype as X; must not overlap X, Wq or the workspace
 *   workspace device buffer of ws_bytes >= rq_rotq_linear_workspace_size(M, K, cfg) */
rq_status rq_rotq_linear(const void *X, int32_t x_dtype, int64_t M, int64_t K,
                         const void *Wq, const float *w_scale, int64_t N, const float *bias,
                         const rq_qconfig *cfg, void *Y, void *workspace, size_t ws_bytes,
                         void *stream);

/* The GEMM + epilogue alone (the second kernel of rq_rotq_linear).
 *   Xq [M, K] int8 / [M, K/2] uint8, x_scale [M]; Wq, w_scale, bias as above;
 *   Y  out: [M, N] of y_dtype (RQ_F16 or RQ_BF16). */
rq_status rq_gemm_dequant(const void *Xq, const float *x_scale, const void *Wq,
                          const float *w_scale, const float *bias, int64_t M, int64_t N,
                          int64_t K, const rq_qconfig *cfg, void *Y, int32_t y_dtype,
                          void *stream);

/* Same mainloop, storing the exact int32 accumulators acc[M, N] = sum_k Xq[m,k] * Wq[n,k]
 * (for bit-exact checks). */
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
