// internal.h -- declarations shared by the HIP translation units of libconvrot.so.
// Not part of the public ABI (see include/convrot.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

enum InDtype { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Weight-scale rules (values of rq_qconfig.w_scale_mode).
enum WScaleMode { kWScaleAbsmax = 0, kWScaleMse = 1, kWScaleTensor = 2 };

// Code layouts written by the quantizers (convrot.h): row-major int8 / packed int4, the tiled
// int layout (256-row panels), and FP6 tiles of 4-bit codes in 256-row (activation) or 128-row
// (weight) panels.
enum CodeLayout { kCodeRows = 0, kCodeTiled = 1, kCodeFp6X = 2, kCodeFp6W = 3 };

// Rotate + quantize `rows` rows of length K (dtype `dt`) into codes Q in `layout` (a CodeLayout;
// the FP6 layouts need bits == 4) and one fp32 scale per row. Arguments are pre-validated.
hipError_t launch_rotate_quant(const void* X, int dt, int64_t rows, int64_t K, int bits,
                               int layout, void* Q, float* S, hipStream_t stream);

// The weight quantizer's MSE-clipped (kWScaleMse) or tensor-wise (kWScaleTensor) scale rule:
// codes Wq (row-major int8 / packed int4, or FP6 tiles of 128-row panels when fp6) and one fp32
// scale per row. Arguments are pre-validated; N < 2^31.
hipError_t launch_weight_quant(int mode, const void* W, int dt, int64_t N, int64_t K, int bits,
                               bool fp6, void* Wq, float* S, hipStream_t stream);

// acc = Xq * Wq^T over K (codes of `bits` bits; Xq row-major or tiled when x_tiled, Wq
// row-major), then either the dequantizing epilogue into Y (out_dt kF16 / kBF16), with the
// activation `act` (gemm::ActKind) applied before the rounding, or, when acc32 != nullptr, the
// raw int32 accumulators (act ignored).
hipError_t launch_gemm(const void* Xq, const float* sx, const void* Wq, const float* sw,
                       const float* bias, int64_t M, int64_t N, int64_t K, int bits,
                       bool x_tiled, void* Y, int out_dt, int32_t* acc32, int act,
                       hipStream_t stream);

// 4-bit codes on the FP6 matrix cores: Xt and Wt in the FP6 tile layout of convrot.h (256-row
// and 128-row panels). K % 128 == 0. `act` as for launch_gemm.
hipError_t launch_gemm_fp6(const void* Xt, const float* sx, const void* Wt, const float* sw,
                           const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                           int out_dt, int32_t* acc32, int act, hipStream_t stream);

// The same GEMM with each CU's weight tile resident in LDS and eight independent waves
// (int8 codes in the tiled layout, K = 1024; gemm_rw.hip). launch_gemm takes it where
// gemm_rw_supported() holds.
bool gemm_rw_supported(int64_t M, int64_t N, int64_t Kb, int bits, bool x_tiled);
hipError_t launch_gemm_rw(const void* Xq, const float* sx, const void* Wq, const float* sw,
                          const float* bias, int64_t M, int64_t N, void* Y, int out_dt,
                          int32_t* acc32, int act, hipStream_t stream);

// The same GEMM on 256 x 256 tiles with 128-byte k steps (launch_gemm picks it for long K);
// it needs Kb (K in bytes of codes) to be a multiple of 128 and at least 256.
bool wide_gemm_supported(int64_t Kb);
hipError_t launch_gemm_wide(const void* Xq, const float* sx, const void* Wq, const float* sw,
                            const float* bias, int64_t M, int64_t N, int64_t K, int bits,
                            void* Y, int out_dt, int32_t* acc32, hipStream_t stream);

}  // namespace convrot
