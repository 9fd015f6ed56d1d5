// api.hip -- the C ABI of libconvrot.so (declared and documented in include/convrot.h).
//
// Host side only: argument validation (a pure function of the arguments, no HIP call),
// workspace carving, and the launches of the two kernels on the caller's stream. Nothing is
// allocated. The only state is rq_rotq_linear_noalloc's static device scratch and the per-device
// cache of its address.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "convrot.h"
#include "internal.h"

namespace {

thread_local std::string g_detail;

constexpr int64_t kMaxK = 131072;          // int32 accumulators: 127^2 * K and 256 * 7^2 * K < 2^31
constexpr int64_t kMaxRowsOrCols = (int64_t(1) << 31) - 1;

rq_status fail(rq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
rq_status fail(rq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_detail = buf;
  return s;
}

rq_status ok() { return RQ_OK; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t elem_size(int32_t dt) { return dt == RQ_F32 ? 4 : 2; }

int64_t code_bytes(int64_t rows, int64_t K, int bits) { return bits == 8 ? rows * K : rows * K / 2; }

// FP6 tiles: 48 bytes per 64 codes, rows padded to whole panels.
int64_t fp6_bytes(int64_t rows, int64_t K, int64_t panel) { return (rows + panel - 1) / panel * panel * (K / 64) * 48; }

// Activation codes in a layout: the tiled layouts pad the rows to whole 256-row panels.
int64_t x_code_bytes(int64_t rows, int64_t K, int bits, int32_t layout) {
  if (layout == RQ_X_FP6) return fp6_bytes(rows, K, 256);
  const int64_t r = layout == RQ_X_TILED ? (rows + 255) / 256 * 256 : rows;
  return code_bytes(r, K, bits);
}

// Weight codes in a layout: FP6 tiles pad the rows to whole 128-row panels.
int64_t w_code_bytes(int64_t rows, int64_t K, int bits, int32_t layout) {
  return layout == RQ_W_FP6 ? fp6_bytes(rows, K, 128) : code_bytes(rows, K, bits);
}

// The activation layout the fused call uses inside its workspace: FP6 tiles to match FP6
// weights, else the tiled int layout.
int32_t fused_x_layout(const rq_qconfig* cfg) { return cfg->w_layout == RQ_W_FP6 ? RQ_X_FP6 : RQ_X_TILED; }

int code_layout(int32_t x_layout) {
  return x_layout == RQ_X_FP6 ? convrot::kCodeFp6X : x_layout == RQ_X_TILED ? convrot::kCodeTiled : convrot::kCodeRows;
}

int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

rq_status check_cfg(const rq_qconfig* cfg) {
  if (!cfg) return fail(RQ_EINVAL, "cfg is NULL");
  if (cfg->bits != 8 && cfg->bits != 4)
    return fail(RQ_EUNSUPPORTED, "bits = %d (supported: 8, 4)", cfg->bits);
  if (cfg->rot_kind != RQ_ROT_WHT)
    return fail(RQ_EUNSUPPORTED, "rot_kind = %d (supported: RQ_ROT_WHT)", cfg->rot_kind);
  if (cfg->rot_block != 128)
    return fail(RQ_EUNSUPPORTED, "rot_block = %d (supported: 128)", cfg->rot_block);
  if (cfg->x_layout != RQ_X_ROWS && cfg->x_layout != RQ_X_TILED && cfg->x_layout != RQ_X_FP6)
    return fail(RQ_EINVAL, "x_layout = %d (RQ_X_ROWS, RQ_X_TILED or RQ_X_FP6)", cfg->x_layout);
  if (cfg->w_layout != RQ_W_ROWS && cfg->w_layout != RQ_W_FP6)
    return fail(RQ_EINVAL, "w_layout = %d (RQ_W_ROWS or RQ_W_FP6)", cfg->w_layout);
  if ((cfg->x_layout == RQ_X_FP6 || cfg->w_layout == RQ_W_FP6) && cfg->bits != 4)
    return fail(RQ_EUNSUPPORTED, "FP6 code layouts hold 4-bit codes only (bits = %d)", cfg->bits);
  if (cfg->w_scale_mode != RQ_W_ABSMAX && cfg->w_scale_mode != RQ_W_MSE &&
      cfg->w_scale_mode != RQ_W_TENSOR)
    return fail(RQ_EINVAL, "w_scale_mode = %d (RQ_W_ABSMAX, RQ_W_MSE or RQ_W_TENSOR)",
                cfg->w_scale_mode);
  if (cfg->act != RQ_ACT_NONE && cfg->act != RQ_ACT_GELU_ERF && cfg->act != RQ_ACT_GELU_TANH)
    return fail(RQ_EINVAL, "act = %d (RQ_ACT_NONE, RQ_ACT_GELU_ERF or RQ_ACT_GELU_TANH)", cfg->act);
  return ok();
}

rq_status check_rows_k(int64_t rows, int64_t K, const char* what) {
  if (rows < 0) return fail(RQ_EINVAL, "%s rows = %lld < 0", what, (long long)rows);
  if (rows > kMaxRowsOrCols) return fail(RQ_EUNSUPPORTED, "%s rows = %lld >= 2^31", what, (long long)rows);
  if (K < 128 || K % 128 != 0 || K > kMaxK)
    return fail(RQ_EUNSUPPORTED, "K = %lld (need a multiple of 128 in [128, %lld])", (long long)K,
                (long long)kMaxK);
  return ok();
}

rq_status check_gemm_shape(int64_t M, int64_t N, int64_t K) {
  rq_status s = check_rows_k(M, K, "M");
  if (s) return s;
  if (N <= 0 || N % 16 != 0 || N > kMaxRowsOrCols)
    return fail(RQ_EUNSUPPORTED, "N = %lld (need a positive multiple of 16 below 2^31)", (long long)N);
  return ok();
}

rq_status check_ptr(const void* p, const char* name, bool required = true) {
  if (!p) return required ? fail(RQ_EINVAL, "%s is NULL", name) : ok();
  if (!aligned16(p)) return fail(RQ_EINVAL, "%s is not 16-byte aligned", name);
  return ok();
}

rq_status from_hip(hipError_t e, const char* where) {
  if (e == hipSuccess) return RQ_OK;
  return fail(RQ_EHIP, "%s: %s", where, hipGetErrorString(e));
}

rq_status check_rotate_args(const void* X, int32_t dt, int64_t rows, int64_t K, const rq_qconfig* cfg,
                            const void* Q, const float* S, const char* xname, bool activations) {
  rq_status s = check_cfg(cfg);
  if (s) return s;
  if (dt != RQ_F32 && dt != RQ_F16 && dt != RQ_BF16) return fail(RQ_EINVAL, "bad %s dtype %d", xname, dt);
  if ((s = check_rows_k(rows, K, xname))) return s;
  if (rows == 0) return ok();
  if ((s = check_ptr(X, xname))) return s;
  if ((s = check_ptr(Q, "codes output"))) return s;
  if (!S) return fail(RQ_EINVAL, "scale output is NULL");
  if ((reinterpret_cast<uintptr_t>(S) & 3u) != 0) return fail(RQ_EINVAL, "scale output is not 4-byte aligned");
  const int64_t xb = rows * K * elem_size(dt);
  const int64_t qb = activations ? x_code_bytes(rows, K, cfg->bits, cfg->x_layout)
                                 : w_code_bytes(rows, K, cfg->bits, cfg->w_layout);
  if (overlap(X, xb, Q, qb) || overlap(X, xb, S, rows * 4) || overlap(Q, qb, S, rows * 4))
    return fail(RQ_EINVAL, "input, codes and scales must not overlap");
  return ok();
}

// Everything of rq_rotq_linear's arguments but the workspace (M == 0 passes here).
rq_status check_linear_core(const void* X, int32_t x_dtype, int64_t M, int64_t K, const void* Wq,
                            const float* w_scale, int64_t N, const float* bias,
                            const rq_qconfig* cfg, const void* Y) {
  rq_status s = check_cfg(cfg);
  if (s) return s;
  if (x_dtype != RQ_F16 && x_dtype != RQ_BF16)
    return fail(x_dtype == RQ_F32 ? RQ_EUNSUPPORTED : RQ_EINVAL,
                "X dtype %d (supported: RQ_F16, RQ_BF16; Y has X's dtype)", x_dtype);
  if ((s = check_gemm_shape(M, N, K))) return s;
  if (M == 0) return ok();
  if ((s = check_ptr(X, "X"))) return s;
  if ((s = check_ptr(Wq, "Wq"))) return s;
  if ((s = check_ptr(w_scale, "w_scale"))) return s;
  if ((s = check_ptr(bias, "bias", false))) return s;
  if ((s = check_ptr(Y, "Y"))) return s;
  const int64_t xb = M * K * 2, wb = w_code_bytes(N, K, cfg->bits, cfg->w_layout), yb = M * N * 2;
  if (overlap(Y, yb, X, xb) || overlap(Y, yb, Wq, wb) || overlap(Y, yb, w_scale, N * 4) ||
      overlap(Y, yb, bias, N * 4))
    return fail(RQ_EINVAL, "Y overlaps an input");
  return ok();
}

// The workspace part: size, alignment and no overlap with the other buffers (M > 0).
rq_status check_linear_ws(const void* X, int64_t M, int64_t K, const void* Wq, const float* w_scale,
                          int64_t N, const float* bias, const rq_qconfig* cfg, const void* Y,
                          const void* ws, size_t ws_bytes) {
  rq_status s = check_ptr(ws, "workspace");
  if (s) return s;
  const size_t need = rq_rotq_linear_workspace_size(M, K, cfg);
  if (ws_bytes < need)
    return fail(RQ_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  const int64_t xb = M * K * 2, wb = w_code_bytes(N, K, cfg->bits, cfg->w_layout), yb = M * N * 2;
  if (overlap(Y, yb, ws, (int64_t)need))
    return fail(RQ_EINVAL, "Y overlaps the workspace");
  if (overlap(ws, (int64_t)need, X, xb) || overlap(ws, (int64_t)need, Wq, wb) ||
      overlap(ws, (int64_t)need, w_scale, N * 4) || overlap(ws, (int64_t)need, bias, N * 4))
    return fail(RQ_EINVAL, "workspace overlaps an input");
  return ok();
}

rq_status check_linear(const void* X, int32_t x_dtype, int64_t M, int64_t K, const void* Wq,
                       const float* w_scale, int64_t N, const float* bias, const rq_qconfig* cfg,
                       const void* Y, const void* ws, size_t ws_bytes) {
  rq_status s = check_linear_core(X, x_dtype, M, K, Wq, w_scale, N, bias, cfg, Y);
  if (s || M == 0) return s;
  return check_linear_ws(X, M, K, Wq, w_scale, N, bias, cfg, Y, ws, ws_bytes);
}

// The two kernels of the quantized linear on an already validated call; `workspace` holds at
// least rq_rotq_linear_workspace_size(M, K, cfg) bytes.
rq_status launch_linear(const void* X, int32_t x_dtype, int64_t M, int64_t K, const void* Wq,
                        const float* w_scale, int64_t N, const float* bias, const rq_qconfig* cfg,
                        void* Y, void* workspace, hipStream_t st) {
  // The workspace holds the codes in the tiled layout (FP6 tiles with FP6 weights), then x_scale.
  const int32_t xl = fused_x_layout(cfg);
  uint8_t* Xq = static_cast<uint8_t*>(workspace);
  float* sx = reinterpret_cast<float*>(Xq + round256(x_code_bytes(M, K, cfg->bits, xl)));
  rq_status s;
  if ((s = from_hip(convrot::launch_rotate_quant(X, x_dtype, M, K, cfg->bits, code_layout(xl), Xq, sx, st),
                    "rotate_quant launch")))
    return s;
  if (xl == RQ_X_FP6)
    return from_hip(convrot::launch_gemm_fp6(Xq, sx, Wq, w_scale, bias, M, N, K, Y, x_dtype, nullptr,
                                             cfg->act, st),
                    "gemm launch");
  return from_hip(convrot::launch_gemm(Xq, sx, Wq, w_scale, bias, M, N, K, cfg->bits, true, Y,
                                       x_dtype, nullptr, cfg->act, st),
                  "gemm launch");
}

// ---- The entry point that allocates nothing: its workspace is `scratch`, a file-scope device
// array (one copy per GPU, held until the process ends). Host code never passes the array's
// name to a kernel: it is a host-side stand-in there. Its device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and cached here.
__device__ __align__(256) uint8_t scratch[RQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

rq_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RQ_EUNSUPPORTED, "device %d (the static scratch serves devices 0..%d)", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return from_hip(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(RQ_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

rq_status check_gemm(const void* Xq, const float* x_scale, const void* Wq, const float* w_scale,
                     const float* bias, int64_t M, int64_t N, int64_t K, const rq_qconfig* cfg,
                     const void* out, int64_t out_elem) {
  rq_status s = check_cfg(cfg);
  if (s) return s;
  if ((s = check_gemm_shape(M, N, K))) return s;
  if (M == 0) return ok();
  if ((s = check_ptr(Xq, "Xq"))) return s;
  if ((s = check_ptr(Wq, "Wq"))) return s;
  if ((s = check_ptr(out, "output"))) return s;
  if (x_scale && (reinterpret_cast<uintptr_t>(x_scale) & 3u)) return fail(RQ_EINVAL, "x_scale misaligned");
  if ((s = check_ptr(w_scale, "w_scale", out_elem != 4))) return s;
  if ((s = check_ptr(bias, "bias", false))) return s;
  if (out_elem != 4 && !x_scale) return fail(RQ_EINVAL, "x_scale is NULL");
  if ((cfg->x_layout == RQ_X_FP6) != (cfg->w_layout == RQ_W_FP6))
    return fail(RQ_EINVAL, "FP6 activation codes go with FP6 weight codes (x_layout %d, w_layout %d)",
                cfg->x_layout, cfg->w_layout);
  const int64_t ob = M * N * out_elem;
  if (overlap(out, ob, Xq, x_code_bytes(M, K, cfg->bits, cfg->x_layout)) ||
      overlap(out, ob, Wq, w_code_bytes(N, K, cfg->bits, cfg->w_layout)) ||
      overlap(out, ob, x_scale, M * 4) || overlap(out, ob, w_scale, N * 4) || overlap(out, ob, bias, N * 4))
    return fail(RQ_EINVAL, "output overlaps an input");
  return ok();
}

}  // namespace

extern "C" {

const char* rq_status_string(rq_status s) {
  switch (s) {
    case RQ_OK: return "RQ_OK: success";
    case RQ_EINVAL: return "RQ_EINVAL: invalid argument (NULL, misaligned, negative size, bad dtype, overlap)";
    case RQ_EUNSUPPORTED: return "RQ_EUNSUPPORTED: shape or configuration outside the supported limits";
    case RQ_EWORKSPACE: return "RQ_EWORKSPACE: workspace too small";
    case RQ_EHIP: return "RQ_EHIP: HIP runtime error";
  }
  return "unknown rq_status";
}

const char* rq_last_error_detail(void) { return g_detail.c_str(); }

const char* rq_version(void) { return "0.1.0"; }

size_t rq_rotq_linear_workspace_size(int64_t M, int64_t K, const rq_qconfig* cfg) {
  if (check_cfg(cfg) != RQ_OK || M < 0 || K <= 0) return 0;
  return (size_t)(round256(x_code_bytes(M, K, cfg->bits, fused_x_layout(cfg))) + round256(M * 4));
}

size_t rq_weight_bytes(int64_t N, int64_t K, const rq_qconfig* cfg) {
  if (check_cfg(cfg) != RQ_OK || N < 0 || N > kMaxRowsOrCols || K <= 0 || K > kMaxK || K % 128)
    return 0;
  return (size_t)w_code_bytes(N, K, cfg->bits, cfg->w_layout);
}

size_t rq_codes_bytes(int64_t rows, int64_t K, const rq_qconfig* cfg) {
  if (check_cfg(cfg) != RQ_OK || rows < 0 || rows > kMaxRowsOrCols || K <= 0 || K > kMaxK || K % 128)
    return 0;
  return (size_t)x_code_bytes(rows, K, cfg->bits, cfg->x_layout);
}

rq_status rq_quantize_weights(const void* W, int32_t w_dtype, int64_t N, int64_t K,
                              const rq_qconfig* cfg, void* Wq, float* w_scale, void* stream) {
  rq_status s = check_rotate_args(W, w_dtype, N, K, cfg, Wq, w_scale, "W", false);
  if (s) return s;
  const bool fp6 = cfg->w_layout == RQ_W_FP6;
  if (cfg->w_scale_mode != RQ_W_ABSMAX)
    return from_hip(convrot::launch_weight_quant(cfg->w_scale_mode == RQ_W_MSE ? convrot::kWScaleMse
                                                                                : convrot::kWScaleTensor,
                                                 W, w_dtype, N, K, cfg->bits, fp6, Wq, w_scale,
                                                 static_cast<hipStream_t>(stream)),
                    "weight_quant launch");
  return from_hip(convrot::launch_rotate_quant(W, w_dtype, N, K, cfg->bits,
                                               fp6 ? convrot::kCodeFp6W : convrot::kCodeRows, Wq, w_scale,
                                               static_cast<hipStream_t>(stream)),
                  "rotate_quant launch");
}

rq_status rq_rotate_quantize(const void* X, int32_t x_dtype, int64_t M, int64_t K,
                             const rq_qconfig* cfg, void* Xq, float* x_scale, void* stream) {
  rq_status s = check_rotate_args(X, x_dtype, M, K, cfg, Xq, x_scale, "X", true);
  if (s) return s;
  return from_hip(convrot::launch_rotate_quant(X, x_dtype, M, K, cfg->bits, code_layout(cfg->x_layout),
                                               Xq, x_scale, static_cast<hipStream_t>(stream)),
                  "rotate_quant launch");
}

rq_status rq_check_rotq_linear_args(const void* X, int32_t x_dtype, int64_t M, int64_t K,
                                    const void* Wq, const float* w_scale, int64_t N,
                                    const float* bias, const rq_qconfig* cfg, const void* Y,
                                    const void* workspace, size_t ws_bytes) {
  return check_linear(X, x_dtype, M, K, Wq, w_scale, N, bias, cfg, Y, workspace, ws_bytes);
}

rq_status rq_rotq_linear(const void* X, int32_t x_dtype, int64_t M, int64_t K, const void* Wq,
                         const float* w_scale, int64_t N, const float* bias,
                         const rq_qconfig* cfg, void* Y, void* workspace, size_t ws_bytes,
                         void* stream) {
  rq_status s = check_linear(X, x_dtype, M, K, Wq, w_scale, N, bias, cfg, Y, workspace, ws_bytes);
  if (s || M == 0) return s;
  return launch_linear(X, x_dtype, M, K, Wq, w_scale, N, bias, cfg, Y, workspace,
                       static_cast<hipStream_t>(stream));
}

rq_status rq_rotq_linear_noalloc(const void* X, int32_t x_dtype, int64_t M, int64_t K,
                                 const void* Wq, const float* w_scale, int64_t N, const float* bias,
                                 const rq_qconfig* cfg, void* Y, void* stream) {
  // The size limit first, so that an oversized call gets this status whatever its pointers.
  rq_status s = check_cfg(cfg);
  if (s) return s;
  if ((s = check_gemm_shape(M, N, K))) return s;
  const size_t need = rq_rotq_linear_workspace_size(M, K, cfg);
  if (need > (size_t)RQ_NOALLOC_SCRATCH_BYTES)
    return fail(RQ_EWORKSPACE, "the call needs %zu bytes of workspace; the static scratch holds %zu "
                               "(use rq_rotq_linear with a caller workspace)",
                need, (size_t)RQ_NOALLOC_SCRATCH_BYTES);
  if ((s = check_linear_core(X, x_dtype, M, K, Wq, w_scale, N, bias, cfg, Y)) || M == 0) return s;
  void* ws = nullptr;
  if ((s = scratch_of_current_device(&ws))) return s;
  if ((s = check_linear_ws(X, M, K, Wq, w_scale, N, bias, cfg, Y, ws, RQ_NOALLOC_SCRATCH_BYTES))) return s;
  return launch_linear(X, x_dtype, M, K, Wq, w_scale, N, bias, cfg, Y, ws, static_cast<hipStream_t>(stream));
}

rq_status rq_gemm_dequant(const void* Xq, const float* x_scale, const void* Wq,
                          const float* w_scale, const float* bias, int64_t M, int64_t N,
                          int64_t K, const rq_qconfig* cfg, void* Y, int32_t y_dtype,
                          void* stream) {
  if (y_dtype != RQ_F16 && y_dtype != RQ_BF16)
    return fail(y_dtype == RQ_F32 ? RQ_EUNSUPPORTED : RQ_EINVAL, "Y dtype %d (supported: RQ_F16, RQ_BF16)", y_dtype);
  rq_status s = check_gemm(Xq, x_scale, Wq, w_scale, bias, M, N, K, cfg, Y, 2);
  if (s || M == 0) return s;
  if (cfg->x_layout == RQ_X_FP6)
    return from_hip(convrot::launch_gemm_fp6(Xq, x_scale, Wq, w_scale, bias, M, N, K, Y, y_dtype, nullptr,
                                             cfg->act, static_cast<hipStream_t>(stream)),
                    "gemm launch");
  return from_hip(convrot::launch_gemm(Xq, x_scale, Wq, w_scale, bias, M, N, K, cfg->bits,
                                       cfg->x_layout == RQ_X_TILED, Y, y_dtype, nullptr, cfg->act,
                                       static_cast<hipStream_t>(stream)),
                  "gemm launch");
}

rq_status rq_gemm_s32(const void* Xq, const void* Wq, int64_t M, int64_t N, int64_t K,
                      const rq_qconfig* cfg, int32_t* acc, void* stream) {
  rq_status s = check_gemm(Xq, nullptr, Wq, nullptr, nullptr, M, N, K, cfg, acc, 4);
  if (s || M == 0) return s;
  if (cfg->x_layout == RQ_X_FP6)
    return from_hip(convrot::launch_gemm_fp6(Xq, nullptr, Wq, nullptr, nullptr, M, N, K, acc, RQ_F16, acc,
                                             RQ_ACT_NONE, static_cast<hipStream_t>(stream)),
                    "gemm launch");
  return from_hip(convrot::launch_gemm(Xq, nullptr, Wq, nullptr, nullptr, M, N, K, cfg->bits,
                                       cfg->x_layout == RQ_X_TILED, acc, RQ_F16, acc, RQ_ACT_NONE,
                                       static_cast<hipStream_t>(stream)),
                  "gemm launch");
}

}  // extern "C"
