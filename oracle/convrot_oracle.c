/*
 * convrot_oracle.c -- plain, slow CPU oracle for the ConvRot quantized linear.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file: only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code, header, table or constant with the HIP library.
 *
 * What it computes (sources are the web pages this method is documented on):
 *   - "SAM 3.1 Multiplex INT8/INT4 ConvRot" release page (civarchive), section
 *     "Quantization recipe": the converter upcasts each eligible weight to FP32, applies a
 *     block-Hadamard ConvRot transform, and stores per-row quantization scales; W8A8 / W4A4
 *     use 8-bit / 4-bit weights with online (dynamic, per-operation) activation quantization.
 *   - "TRELLIS.2 INT8 ConvRot in ComfyUI" guide, section "What ConvRot changes": a grouped,
 *     normalized Hadamard rotation is applied before per-row INT8 weight quantization and
 *     the matching rotation is applied to activations at run time.
 *   - "Explanation of INT8 ConvRot" article, format taxonomy tables: INT8 encoding, row-wise
 *     scaling, ConvRot quantization method.
 * Readings where the pages are silent (each one is listed in the design notes):
 *   block size 128; Sylvester Hadamard in natural order without sign flips; rotation and
 *   quantization arithmetic in fp32 (the recipe's FP32 upcast); butterfly stages in the
 *   order h = 1, 2, 4, ..., 64; one absmax scale per row over all of K; q_max = 127 (int8)
 *   or 7 (int4), symmetric; round half to even; the normalization 1/sqrt(128) folded into
 *   the scale; zero rows get scale 0 and codes 0; int4 two per byte, low nibble = even k;
 *   int32 accumulation; epilogue y = fma(f32(acc), s_w*s_x, bias) rounded to fp16/bf16;
 *   the MLP activation (when fused into the epilogue) GELU in its erf or tanh form.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC (see build.py).
 * -ffp-contract=off matters: every fp32 operation below is one correctly rounded IEEE op.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BLOCK 128

/* ------------------------------------------------------------------------------------ */
/* Exact number-format conversions, written from the IEEE-754 binary16 definition and the  */
/* bfloat16 definition (binary32 with the low 16 bits dropped).                            */
/* ------------------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* binary16 -> binary32 (exact: every binary16 value is a binary32 value). */
float orc_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1f, m = h & 0x3ffu;
  if (e == 0x1f) return bits_f32(sign | 0x7f800000u | (m << 13));        /* inf / NaN */
  if (e == 0) {                                                           /* zero / subnormal */
    float v = (float)m * 0x1p-24f;                                        /* exact: m < 2^10 */
    return sign ? -v : v;
  }
  return bits_f32(sign | ((e - 15 + 127) << 23) | (m << 13));
}

/* bfloat16 -> binary32 (exact: append 16 zero bits). */
float orc_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* binary32 -> binary16, round to nearest, ties to even; overflow -> +-inf; NaN -> qNaN. */
uint16_t orc_f32_to_f16(float f) {
  uint32_t x = f32_bits(f);
  uint16_t s = (uint16_t)((x >> 16) & 0x8000u);
  uint32_t ax = x & 0x7fffffffu;
  if (ax > 0x7f800000u) return s | 0x7e00u;
  if (ax == 0x7f800000u) return s | 0x7c00u;
  int be = (int)(ax >> 23);
  if (be == 0) return s;                         /* |f| < 2^-126: far below half of 2^-24 */
  uint64_t M = (ax & 0x7fffffu) | 0x800000u;     /* |f| = M * 2^(be-150) */
  int E = be - 150;
  int e16 = be - 127;                            /* floor(log2 |f|) */
  int qexp = (e16 < -14) ? -24 : e16 - 10;       /* exponent of one binary16 ulp at |f| */
  int shift = qexp - E;                          /* >= 13 */
  uint64_t n;
  if (shift >= 63) {
    n = 0;
  } else {
    n = M >> shift;
    uint64_t rem = M - (n << shift), half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (n & 1u))) n++;
  }
  if (qexp == -24) return s | (uint16_t)n;       /* subnormal (n == 1024 encodes 2^-14) */
  int e = e16;
  if (n == 2048) { n = 1024; e++; }
  if (e > 15) return s | 0x7c00u;
  return s | (uint16_t)(((e + 15) << 10) | (n - 1024));
}

/* binary32 -> bfloat16, round to nearest, ties to even on the 16 dropped bits. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t x = f32_bits(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u);
  uint32_t lsb = (x >> 16) & 1u;
  x += 0x7fffu + lsb;
  return (uint16_t)(x >> 16);
}

/* ------------------------------------------------------------------------------------ */
/* Hadamard rotation.                                                                    */
/* ------------------------------------------------------------------------------------ */

/* Sylvester Hadamard entry H_128[i][j] = (-1)^popcount(i & j). */
int orc_hadamard_entry(int i, int j) { return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1; }

/* fl(1/sqrt(128)): 1/sqrt(128) = sqrt(2)/16, and sqrtf is correctly rounded, so this is the
 * binary32 value nearest to 1/sqrt(128). */
float orc_inv_sqrt_block(void) { return sqrtf(2.0f) / 16.0f; }

/* Unnormalized fast Walsh-Hadamard transform of one 128-block, in fp32, in place.
 * Stage h = 1, 2, 4, ..., 64 (in this order); in each stage every pair (i, i+h) with
 * (i & h) == 0 becomes (v_i + v_{i+h}, v_i - v_{i+h}). The result is H_128 * v. */
void orc_fwht128(float *v) {
  for (int h = 1; h < ORC_BLOCK; h *= 2)
    for (int i = 0; i < ORC_BLOCK; i++)
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
}

/* fp64 shadow: y = x * R with R = blockdiag(H_128 / sqrt(128)), as an explicit matrix
 * product per block (no fast transform). x, y: [rows, K] row-major doubles. */
void orc_rotate_f64(const double *x, int64_t rows, int64_t K, double *y) {
  const double c = 1.0 / sqrt(128.0);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t b = 0; b < K / ORC_BLOCK; b++)
      for (int j = 0; j < ORC_BLOCK; j++) {
        double acc = 0.0;
        for (int i = 0; i < ORC_BLOCK; i++)
          acc += x[r * K + b * ORC_BLOCK + i] * (double)orc_hadamard_entry(i, j);
        y[r * K + b * ORC_BLOCK + j] = acc * c;
      }
}

/* ------------------------------------------------------------------------------------ */
/* Row quantizer: the step applied offline to weight rows and online to activation rows.  */
/* ------------------------------------------------------------------------------------ */

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

static float load_elem(const void *x, int dtype, int64_t idx) {
  switch (dtype) {
    case ORC_F32: return ((const float *)x)[idx];
    case ORC_F16: return orc_f16_to_f32(((const uint16_t *)x)[idx]);
    default: return orc_bf16_to_f32(((const uint16_t *)x)[idx]);
  }
}

/*
 * For each row r of x [rows, K] (dtype f32 / f16 / bf16 raw bits):
 *   u   = f32(x[r, :]);  if rotate: u <- FWHT_128 of each 128-block (unnormalized)
 *   a   = max_k |u_k|;  inv = fl(q_max / a)
 *   a == 0, or inv = +inf (a too small for its reciprocal to be finite, below about
 *            q_max * 2^-128):  scale = 0, codes = 0 (the row is quantized as a zero row)
 *   else:    scale = fl(fl(a * c) / q_max)  (c = fl(1/sqrt 128), or 1 without rotation);
 *            p_k = fl(u_k * inv);  q_k = round-half-even(p_k)
 * codes: int8 [rows, K] (unpacked, in [-q_max, q_max]); scales: f32 [rows];
 * pre (optional, may be NULL): f32 [rows, K], the pre-rounding values p_k.
 * Returns 0, or -1 if a code fell outside [-q_max, q_max] (cannot happen; checked anyway),
 * or -2 on bad arguments.
 */
int orc_quantize_rows(const void *x, int dtype, int64_t rows, int64_t K, int bits, int rotate,
                      int8_t *codes, float *scales, float *pre) {
  if (K <= 0 || K % ORC_BLOCK != 0 || (bits != 8 && bits != 4) || rows < 0) return -2;
  const float qmax = (bits == 8) ? 127.0f : 7.0f;
  const float c = rotate ? orc_inv_sqrt_block() : 1.0f;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; r++) {
    float *u = (float *)malloc((size_t)K * sizeof(float));
    for (int64_t k = 0; k < K; k++) u[k] = load_elem(x, dtype, r * K + k);
    if (rotate)
      for (int64_t b = 0; b < K / ORC_BLOCK; b++) orc_fwht128(u + b * ORC_BLOCK);
    float a = 0.0f;
    for (int64_t k = 0; k < K; k++) a = fmaxf(a, fabsf(u[k]));
    const float inv = (a > 0.0f) ? qmax / a : 0.0f;
    if (a == 0.0f || isinf(inv)) {
      scales[r] = 0.0f;
      for (int64_t k = 0; k < K; k++) {
        codes[r * K + k] = 0;
        if (pre) pre[r * K + k] = 0.0f;
      }
    } else {
      float ac = a * c;
      scales[r] = ac / qmax;
      for (int64_t k = 0; k < K; k++) {
        float p = u[k] * inv;
        float q = nearbyintf(p); /* default rounding mode: to nearest, ties to even */
        if (q > qmax || q < -qmax) bad = 1;
        codes[r * K + k] = (int8_t)q;
        if (pre) pre[r * K + k] = p;
      }
    }
    free(u);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------------------ */
/* Weight-quantizer variants.                                                           */
/* ------------------------------------------------------------------------------------ */

#define ORC_NCLIP 51   /* clipping candidates alpha = 1.00, 0.99, ..., 0.50 */

/* Candidate i's clipping factor: the binary32 nearest to (100 - i) / 100. */
float orc_clip_alpha(int i) { return (float)(100 - i) / 100.0f; }

/* Quantize the rotated row u[K] against clipping threshold t (> 0): inv = fl(q_max / t),
 * s = fl(fl(t * c) / q_max), q_k = clamp(rne(fl(u_k * inv)), -q_max, q_max); a threshold whose
 * reciprocal overflows (inv = +inf) quantizes the row to zero (s = 0, codes 0), the rule of
 * orc_quantize_rows. Returns s and, in err, sum_k (u_k * c - s * q_k)^2 evaluated in binary64 in
 * increasing k (the products are exact in binary64; the differences, squares and sums are
 * rounded). */
static float quantize_clipped(const float *u, int64_t K, float t, float qmax, float c, int8_t *q,
                              double *err) {
  const float inv0 = qmax / t;
  const int zero = isinf(inv0);
  const float inv = zero ? 0.0f : inv0;
  const float s = zero ? 0.0f : (t * c) / qmax;
  double e = 0.0;
  for (int64_t k = 0; k < K; k++) {
    float v = nearbyintf(u[k] * inv);
    if (v > qmax) v = qmax;
    if (v < -qmax) v = -qmax;
    q[k] = (int8_t)v;
    const double d = (double)u[k] * (double)c - (double)s * (double)v;
    e += d * d;
  }
  *err = e;
  return s;
}

/* MSE-optimized clipping (the release page's "Quantization recipe", step 3, with the reading
 * stated in the design notes): per row, after the rotation, the clipping threshold
 * t = fl(a * alpha_i) is chosen among the ORC_NCLIP candidates to minimize the squared
 * reconstruction error of the normalized rotated row (quantize_clipped); ties keep the larger
 * alpha. alpha = 1 reproduces orc_quantize_rows. A zero row gets scale 0 and codes 0.
 * alpha_idx [rows] (or NULL) receives the chosen candidate, err [rows * ORC_NCLIP] (or NULL)
 * every candidate's error. Rotation always on. */
int orc_quantize_rows_mse(const void *x, int dtype, int64_t rows, int64_t K, int bits,
                          int8_t *codes, float *scales, int32_t *alpha_idx, double *err) {
  if (K <= 0 || K % ORC_BLOCK != 0 || (bits != 8 && bits != 4) || rows < 0) return -2;
  const float qmax = (bits == 8) ? 127.0f : 7.0f;
  const float c = orc_inv_sqrt_block();
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < rows; r++) {
    float *u = (float *)malloc((size_t)K * sizeof(float));
    int8_t *q = (int8_t *)malloc((size_t)K);
    for (int64_t k = 0; k < K; k++) u[k] = load_elem(x, dtype, r * K + k);
    for (int64_t b = 0; b < K / ORC_BLOCK; b++) orc_fwht128(u + b * ORC_BLOCK);
    float a = 0.0f;
    for (int64_t k = 0; k < K; k++) a = fmaxf(a, fabsf(u[k]));
    if (a == 0.0f) {
      scales[r] = 0.0f;
      memset(codes + r * K, 0, (size_t)K);
      if (alpha_idx) alpha_idx[r] = 0;
      if (err)
        for (int i = 0; i < ORC_NCLIP; i++) err[r * ORC_NCLIP + i] = 0.0;
    } else {
      int best = 0;
      double best_e = 0.0;
      for (int i = 0; i < ORC_NCLIP; i++) {
        double e;
        quantize_clipped(u, K, a * orc_clip_alpha(i), qmax, c, q, &e);
        if (err) err[r * ORC_NCLIP + i] = e;
        if (i == 0 || e < best_e) {
          best = i;
          best_e = e;
        }
      }
      double e;
      scales[r] = quantize_clipped(u, K, a * orc_clip_alpha(best), qmax, c, codes + r * K, &e);
      if (alpha_idx) alpha_idx[r] = best;
    }
    free(q);
    free(u);
  }
  return 0;
}

/* Tensor-wise scale (the HSWQ model card's int8_tensorwise variant, here after the same
 * rotation): one absmax A over the whole rotated tensor; every row is quantized with
 * inv = fl(q_max / A) and gets the same scale fl(fl(A * c) / q_max). A zero tensor, or one whose
 * A is too small for a finite inv, gets scales 0 and codes 0. pre (or NULL) receives
 * fl(u * inv). Rotation always on. */
int orc_quantize_tensorwise(const void *x, int dtype, int64_t rows, int64_t K, int bits,
                            int8_t *codes, float *scales, float *pre) {
  if (K <= 0 || K % ORC_BLOCK != 0 || (bits != 8 && bits != 4) || rows < 0) return -2;
  const float qmax = (bits == 8) ? 127.0f : 7.0f;
  const float c = orc_inv_sqrt_block();
  float *u = (float *)malloc((size_t)(rows * K > 0 ? rows * K : 1) * sizeof(float));
  float A = 0.0f;
#pragma omp parallel for schedule(static) reduction(max : A)
  for (int64_t r = 0; r < rows; r++) {
    float *ur = u + r * K;
    for (int64_t k = 0; k < K; k++) ur[k] = load_elem(x, dtype, r * K + k);
    for (int64_t b = 0; b < K / ORC_BLOCK; b++) orc_fwht128(ur + b * ORC_BLOCK);
    for (int64_t k = 0; k < K; k++) A = fmaxf(A, fabsf(ur[k]));
  }
  float inv = (A > 0.0f) ? qmax / A : 0.0f;
  if (isinf(inv)) inv = 0.0f;            /* reciprocal overflow: the zero-row rule */
  const float s = (inv != 0.0f) ? (A * c) / qmax : 0.0f;
  for (int64_t r = 0; r < rows; r++) {
    scales[r] = s;
    for (int64_t k = 0; k < K; k++) {
      const float p = u[r * K + k] * inv;
      codes[r * K + k] = (int8_t)nearbyintf(p);
      if (pre) pre[r * K + k] = p;
    }
  }
  free(u);
  return 0;
}

/* int4 packing: byte[r, j] = (q[r, 2j] & 0xF) | ((q[r, 2j+1] & 0xF) << 4), i.e. two's
 * complement nibbles, low nibble = even k. */
void orc_pack_int4(const int8_t *codes, int64_t rows, int64_t K, uint8_t *packed) {
  for (int64_t r = 0; r < rows; r++)
    for (int64_t j = 0; j < K / 2; j++) {
      uint8_t lo = (uint8_t)codes[r * K + 2 * j] & 0x0fu;
      uint8_t hi = (uint8_t)codes[r * K + 2 * j + 1] & 0x0fu;
      packed[r * (K / 2) + j] = (uint8_t)(lo | (hi << 4));
    }
}

/* Inverse of orc_pack_int4 (sign-extends each nibble). */
void orc_unpack_int4(const uint8_t *packed, int64_t rows, int64_t K, int8_t *codes) {
  for (int64_t r = 0; r < rows; r++)
    for (int64_t j = 0; j < K / 2; j++) {
      uint8_t byte = packed[r * (K / 2) + j];
      int lo = byte & 0x0f, hi = byte >> 4;
      codes[r * K + 2 * j] = (int8_t)(lo >= 8 ? lo - 16 : lo);
      codes[r * K + 2 * j + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
    }
}

/* ------------------------------------------------------------------------------------ */
/* Integer GEMM and the dequantizing epilogue.                                          */
/* ------------------------------------------------------------------------------------ */

/* acc[m, n] = sum_k A[m, k] * B[n, k], accumulated exactly in int64.
 * A: [M, K], B: [N, K] int8 codes (unpacked). Returns -1 if a sum does not fit int32. */
int orc_gemm_s32(const int8_t *A, const int8_t *B, int64_t M, int64_t N, int64_t K, int32_t *acc) {
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++) {
      int64_t s = 0;
      for (int64_t k = 0; k < K; k++) s += (int64_t)A[m * K + k] * (int64_t)B[n * K + k];
      if (s > INT32_MAX || s < INT32_MIN) bad = 1;
      acc[m * N + n] = (int32_t)s;
    }
  return bad ? -1 : 0;
}

/* Y[m, n] = cast( fma( f32(acc[m, n]), fl(s_w[n] * s_x[m]), bias[n] ) ), where f32() is the
 * round-to-nearest-even int32 -> binary32 conversion, bias = +0 when NULL, and cast is the
 * round-to-nearest-even conversion to binary16 (out_dtype 1) or bfloat16 (out_dtype 2).
 * Y holds raw 16-bit patterns. */
void orc_epilogue(const int32_t *acc, const float *sx, const float *sw, const float *bias,
                  int64_t M, int64_t N, int out_dtype, uint16_t *Y) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++) {
      float af = (float)acc[m * N + n];
      float sc = sw[n] * sx[m];
      float v = fmaf(af, sc, bias ? bias[n] : 0.0f);
      Y[m * N + n] = (out_dtype == ORC_F16) ? orc_f32_to_f16(v) : orc_f32_to_bf16(v);
    }
}

/* GELU, the activation between the two linears of an MLP pair (the pages leave the MLP's
 * activation unstated; the readings are the erf form for the ViT MLP and the tanh form for the
 * DiT MLP). Evaluated in binary64 from the binary32 pre-activation v:
 *   act 1, erf form:  0.5 v (1 + erf(v / sqrt 2)), written as 0.5 v erfc(-v / sqrt 2)
 *   act 2, tanh form: 0.5 v (1 + tanh(u)) with u = sqrt(2 / pi) (v + 0.044715 v^3), written
 *                     as v / (1 + exp(-2u))
 * The erfc and logistic forms are the same functions without the cancellation of 1 + erf and
 * 1 + tanh for negative v, so the result is accurate to a few binary64 ulps everywhere. */
double orc_gelu_f64(double v, int act) {
  if (act == 1) return 0.5 * v * erfc(-v / sqrt(2.0));
  if (act == 2) {
    const double u = sqrt(2.0 / acos(-1.0)) * (v + 0.044715 * v * v * v);
    return v / (1.0 + exp(-2.0 * u));
  }
  return v;
}

void orc_gelu_f64_array(const double *v, int64_t n, int act, double *g) {
  for (int64_t i = 0; i < n; i++) g[i] = orc_gelu_f64(v[i], act);
}

/* The epilogue with an activation: v = fma(f32(acc), fl(s_w * s_x), bias) as in orc_epilogue,
 * then g = GELU(v) in binary64 (act 1 or 2; act 0: g = v), rounded to nearest even once to
 * binary32 and then to binary16 / bfloat16. g64, when not NULL, receives the binary64 value
 * before both roundings. */
void orc_epilogue_act(const int32_t *acc, const float *sx, const float *sw, const float *bias,
                      int64_t M, int64_t N, int act, int out_dtype, uint16_t *Y, double *g64) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++) {
      float af = (float)acc[m * N + n];
      float sc = sw[n] * sx[m];
      float v = fmaf(af, sc, bias ? bias[n] : 0.0f);
      double g = orc_gelu_f64((double)v, act);
      float gf = (float)g;
      Y[m * N + n] = (out_dtype == ORC_F16) ? orc_f32_to_f16(gf) : orc_f32_to_bf16(gf);
      if (g64) g64[m * N + n] = g;
    }
}

/* Element-wise conversions over arrays (used by the tests). */
void orc_f32_to_f16_array(const float *x, int64_t n, uint16_t *y) {
  for (int64_t i = 0; i < n; i++) y[i] = orc_f32_to_f16(x[i]);
}
void orc_f32_to_bf16_array(const float *x, int64_t n, uint16_t *y) {
  for (int64_t i = 0; i < n; i++) y[i] = orc_f32_to_bf16(x[i]);
}
void orc_f16_to_f32_array(const uint16_t *x, int64_t n, float *y) {
  for (int64_t i = 0; i < n; i++) y[i] = orc_f16_to_f32(x[i]);
}
void orc_bf16_to_f32_array(const uint16_t *x, int64_t n, float *y) {
  for (int64_t i = 0; i < n; i++) y[i] = orc_bf16_to_f32(x[i]);
}
void orc_fwht128_rows(float *v, int64_t nblocks) {
  for (int64_t b = 0; b < nblocks; b++) orc_fwht128(v + b * ORC_BLOCK);
}
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  omp_set_num_threads(n);
#else
  (void)n;
#endif
}
int orc_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
