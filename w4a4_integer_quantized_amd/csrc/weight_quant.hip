// weight_quant.hip -- the offline weight quantizer's two alternative scale rules.
//
// Both keep the rotation, rounding and storage of the absmax quantizer (convrot.h) and change
// only how the clipping threshold t of a row is chosen; a row is then quantized with
// inv = fl(q_max / t), scale = fl(fl(t * fl(1/sqrt 128)) / q_max),
// code = clamp(round_half_even(fl(u * inv)), -q_max, q_max), and t = 0 gives scale 0, codes 0.
//
//  * MSE-optimized clipping ("SAM 3.1 Multiplex INT8/INT4 ConvRot" page, "Quantization
//    recipe", step 3: after the block-Hadamard transform the converter picks the clipping scale
//    with the least squared error). Candidates t_i = fl(a * alpha_i), alpha_i = fl((100-i)/100),
//    i = 0..50, a = max |u| of the row; candidate i's error is
//    E_i = sum_k (u_k c - s_i q_ik)^2 in binary64, summed in increasing k (u_k c and s_i q_ik are
//    exact products; the difference, square and sum are rounded). The least E_i wins, the
//    smallest i (largest alpha) on a tie.
//  * Tensor-wise scale (the HSWQ ConvRot model card's int8_tensorwise; the "Explanation of INT8
//    ConvRot" taxonomy, scaling method "tensor-wise"): t = A, the absmax over the whole rotated
//    matrix, so every row gets the same scale.
//
// Work layout. One 64-lane wave per row (a workgroup of one wave), streaming the row's
// 128-blocks; lane l holds elements 2l and 2l+1 of the current block. Butterflies run in the
// fixed order h = 1 (inside the lane), then h = 2 .. 64 against lane l ^ (h/2) (ds_bpermute);
// the lane whose element has bit h set takes partner - mine, the other mine + partner.
// The MSE search gives candidate i to lane i: the block's 128 rotated values go to LDS and every
// candidate lane walks them in increasing k, so each E_i is accumulated in exactly the order
// that defines it and the choice is reproducible bit for bit. The row is read three times
// (absmax, search, quantize), recomputing the rotation each time; the repeats hit the caches.
// Tensor-wise runs three kernels: per-row absmax into the scale array, one workgroup that
// reduces it to A and writes A back to every entry, then a per-row quantize that reads its own
// entry as t and overwrites it with the scale -- no scratch memory beyond the outputs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace convrot {
namespace {

constexpr float kInvSqrtBlock = 0x1.6a09e6p-4f;  // binary32 nearest to 1/sqrt(128)
constexpr int kNClip = 51;                       // clipping candidates alpha = 1.00 .. 0.50

// Elements 2*lane and 2*lane+1 of the 128-block starting at element `blk0` (exact upcast).
template <int DT>
__device__ __forceinline__ void load_pair(const void* X, int64_t blk0, int lane, float& v0, float& v1) {
  const int64_t e = blk0 + 2 * lane;
  if constexpr (DT == kF32) {
    const float2 p = *reinterpret_cast<const float2*>(static_cast<const float*>(X) + e);
    v0 = p.x;
    v1 = p.y;
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(X) + e);
    if constexpr (DT == kF16) {
      v0 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xFFFFu)));
      v1 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
    } else {
      v0 = __uint_as_float(w << 16);
      v1 = __uint_as_float(w & 0xFFFF0000u);
    }
  }
}

// Unnormalized Walsh-Hadamard transform of one 128-block held two elements per lane.
template <int DT>
__device__ __forceinline__ void rotated_pair(const void* X, int64_t blk0, int lane, float& v0, float& v1) {
  load_pair<DT>(X, blk0, lane, v0, v1);
  const float s = v0 + v1, d = v0 - v1;  // h = 1
  v0 = s;
  v1 = d;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {      // h = 2m: partner lane l ^ m, same slot
    const float o0 = __shfl_xor(v0, m), o1 = __shfl_xor(v1, m);
    const bool upper = (lane & m) != 0;
    v0 = upper ? o0 - v0 : v0 + o0;
    v1 = upper ? o1 - v1 : v1 + o1;
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

template <int DT>
__device__ float row_absmax(const void* X, int64_t row0, int nb, int lane) {
  float a = 0.0f;
  for (int b = 0; b < nb; b++) {
    float v0, v1;
    rotated_pair<DT>(X, row0 + 128 * (int64_t)b, lane, v0, v1);
    a = fmaxf(a, fmaxf(fabsf(v0), fabsf(v1)));
  }
  return wave_max(a);
}

__device__ __forceinline__ float clamp_code(float p, float qmax) {
  return fminf(fmaxf(rintf(p), -qmax), qmax);
}

// FP6 E2M3 pattern of a code in [-7, 7] (1.0, 2.0, 1.5 * 2, 4.0, 1.25 * 4, 1.5 * 4, 1.75 * 4).
__device__ __forceinline__ uint32_t fp6_code(int q) {
  const uint32_t mag = q < 0 ? (uint32_t)(-q) : (uint32_t)q;
  const uint32_t m = (0x1E1C1A1814100800ull >> (8 * mag)) & 0xFFu;
  return m | (q < 0 ? 0x20u : 0u);
}

// Byte `b` (0..23) of the FP6 operand string of row `row`, slice `s`, half `h` in 128-row weight
// panels (the tile layout of convrot.h).
__device__ __forceinline__ int64_t fp6w_offset(int64_t row, int s, int h, int b, int nsl) {
  const int64_t base = ((row >> 7) * nsl + s) * (int64_t)(128 * 48);
  const int rr = (int)(row & 127);
  if (b < 16) return base + rr * 32 + 16 * (h ^ ((rr >> 3) & 1)) + b;
  return base + 128 * 32 + rr * 16 + 8 * (h ^ ((rr >> 4) & 1)) + (b - 16);
}

// The multiplier fl(q_max / t) of threshold t, or 0 -- the zero-row rule -- when t is 0 or too
// small for the quotient to be finite.
__device__ __forceinline__ float clip_inv(float t, float qmax) {
  const float inv = t > 0.0f ? __fdiv_rn(qmax, t) : 0.0f;
  return __builtin_isinf(inv) ? 0.0f : inv;
}

// Quantize one row against threshold t (t == 0, or a t whose multiplier overflows: codes 0 and
// scale 0); returns the row's scale. BITS = 6 stores 4-bit codes as FP6 weight tiles.
template <int DT, int BITS>
__device__ float quantize_row(const void* X, int64_t row, int64_t K, float t, uint8_t* Q, int lane) {
  const float qmax = BITS == 8 ? 127.0f : 7.0f;
  const float inv = clip_inv(t, qmax);
  const int nb = static_cast<int>(K / 128);
  for (int b = 0; b < nb; b++) {
    float v0, v1;
    rotated_pair<DT>(X, row * K + 128 * (int64_t)b, lane, v0, v1);
    const int q0 = static_cast<int>(clamp_code(__fmul_rn(v0, inv), qmax));
    const int q1 = static_cast<int>(clamp_code(__fmul_rn(v1, inv), qmax));
    if constexpr (BITS == 8) {
      const uint16_t pair = static_cast<uint16_t>((q0 & 0xFF) | ((q1 & 0xFF) << 8));
      *reinterpret_cast<uint16_t*>(Q + row * K + 128 * (int64_t)b + 2 * lane) = pair;
    } else if constexpr (BITS == 6) {
      // Lanes 2m and 2m+1 hold elements 4m .. 4m+3 of the block: one 24-bit field (3 bytes)
      // at byte 3 * (e % 32 / 4) of the string of slice 2b + e / 64, half (e / 32) & 1.
      const uint32_t mine = fp6_code(q0) | (fp6_code(q1) << 6);
      const uint32_t other = __shfl_xor(mine, 1);
      if ((lane & 1) == 0) {
        const uint32_t g = mine | (other << 12);
        const int e = (4 * (lane >> 1)) & 63;
        const int s = 2 * b + (lane >= 32 ? 1 : 0), h = (e >> 5) & 1, b0 = 3 * ((e & 31) >> 2);
#pragma unroll
        for (int k = 0; k < 3; k++) Q[fp6w_offset(row, s, h, b0 + k, (int)(K >> 6))] = static_cast<uint8_t>(g >> (8 * k));
      }
    } else {
      Q[row * (K / 2) + 64 * (int64_t)b + lane] = static_cast<uint8_t>((q0 & 0xF) | ((q1 & 0xF) << 4));
    }
  }
  return inv != 0.0f ? __fdiv_rn(__fmul_rn(t, kInvSqrtBlock), qmax) : 0.0f;
}

template <int DT, int BITS>
__global__ __launch_bounds__(64) void mse_clip_kernel(const void* __restrict__ X, int64_t K,
                                                      uint8_t* __restrict__ Q, float* __restrict__ S) {
  __shared__ float4 ublk[32];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int nb = static_cast<int>(K / 128);
  const float qmax = BITS == 8 ? 127.0f : 7.0f;

  const float a = row_absmax<DT>(X, row * K, nb, lane);
  float t = 0.0f;
  if (a > 0.0f) {
    // Candidate lane_i: t_i, inv_i, s_i exactly as the final quantization would use them.
    const int cand = lane < kNClip ? lane : 0;
    const float ti = __fmul_rn(a, __fdiv_rn(static_cast<float>(100 - cand), 100.0f));
    const float inv = clip_inv(ti, qmax);       // 0: this candidate quantizes the row to zero
    const double sd = inv != 0.0f ? static_cast<double>(__fdiv_rn(__fmul_rn(ti, kInvSqrtBlock), qmax)) : 0.0;
    const double cd = static_cast<double>(kInvSqrtBlock);
    double e = 0.0;
    for (int b = 0; b < nb; b++) {
      float v0, v1;
      rotated_pair<DT>(X, row * K + 128 * (int64_t)b, lane, v0, v1);
      reinterpret_cast<float2*>(ublk)[lane] = make_float2(v0, v1);
      __syncthreads();
      if (lane < kNClip) {
        for (int j = 0; j < 32; j++) {
          const float4 u4 = ublk[j];  // same address in every lane: a broadcast read
          const float us[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const float q = clamp_code(__fmul_rn(us[r], inv), qmax);
            const double d = static_cast<double>(us[r]) * cd - sd * static_cast<double>(q);
            e = e + d * d;
          }
        }
      }
      __syncthreads();
    }
    // Least error, smallest index among equals.
    double best_e = lane < kNClip ? e : INFINITY;
    int best_i = lane;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const double oe = __shfl_xor(best_e, m);
      const int oi = __shfl_xor(best_i, m);
      if (oe < best_e || (oe == best_e && oi < best_i)) {
        best_e = oe;
        best_i = oi;
      }
    }
    t = __fmul_rn(a, __fdiv_rn(static_cast<float>(100 - best_i), 100.0f));
  }
  const float s = quantize_row<DT, BITS>(X, row, K, t, Q, lane);
  if (lane == 0) S[row] = s;
}

template <int DT>
__global__ __launch_bounds__(64) void row_absmax_kernel(const void* __restrict__ X, int64_t K,
                                                        float* __restrict__ S) {
  const int64_t row = blockIdx.x;
  const float a = row_absmax<DT>(X, row * K, static_cast<int>(K / 128), threadIdx.x);
  if (threadIdx.x == 0) S[row] = a;
}

// One workgroup: A = max S[0..N), then S[r] = A for every r.
__global__ __launch_bounds__(1024) void broadcast_max_kernel(float* __restrict__ S, int64_t N) {
  __shared__ float part[16];
  float a = 0.0f;
  for (int64_t r = threadIdx.x; r < N; r += blockDim.x) a = fmaxf(a, S[r]);
  a = wave_max(a);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = a;
  __syncthreads();
  a = 0.0f;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); w++) a = fmaxf(a, part[w]);
  for (int64_t r = threadIdx.x; r < N; r += blockDim.x) S[r] = a;
}

template <int DT, int BITS>
__global__ __launch_bounds__(64) void quantize_given_kernel(const void* __restrict__ X, int64_t K,
                                                            uint8_t* __restrict__ Q, float* __restrict__ S) {
  const int64_t row = blockIdx.x;
  const float t = S[row];
  const float s = quantize_row<DT, BITS>(X, row, K, t, Q, threadIdx.x);
  if (threadIdx.x == 0) S[row] = s;
}

template <int DT, int BITS>
hipError_t launch_typed(int mode, const void* W, int64_t N, int64_t K, uint8_t* Q, float* S,
                        hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(N)), block(64);
  if (mode == kWScaleMse) {
    hipLaunchKernelGGL((mse_clip_kernel<DT, BITS>), grid, block, 0, stream, W, K, Q, S);
  } else {
    hipLaunchKernelGGL((row_absmax_kernel<DT>), grid, block, 0, stream, W, K, S);
    hipLaunchKernelGGL(broadcast_max_kernel, dim3(1), dim3(1024), 0, stream, S, N);
    hipLaunchKernelGGL((quantize_given_kernel<DT, BITS>), grid, block, 0, stream, W, K, Q, S);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(int mode, const void* W, int64_t N, int64_t K, int fmt, uint8_t* Q, float* S,
                     hipStream_t stream) {
  switch (fmt) {
    case 8: return launch_typed<DT, 8>(mode, W, N, K, Q, S, stream);
    case 4: return launch_typed<DT, 4>(mode, W, N, K, Q, S, stream);
    default: return launch_typed<DT, 6>(mode, W, N, K, Q, S, stream);
  }
}

}  // namespace

hipError_t launch_weight_quant(int mode, const void* W, int dt, int64_t N, int64_t K, int bits,
                               bool fp6, void* Wq, float* S, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  uint8_t* Q = static_cast<uint8_t*>(Wq);
  const int fmt = fp6 ? 6 : bits;
  switch (dt) {
    case kF32: return launch_dt<kF32>(mode, W, N, K, fmt, Q, S, stream);
    case kF16: return launch_dt<kF16>(mode, W, N, K, fmt, Q, S, stream);
    default: return launch_dt<kBF16>(mode, W, N, K, fmt, Q, S, stream);
  }
}

}  // namespace convrot
