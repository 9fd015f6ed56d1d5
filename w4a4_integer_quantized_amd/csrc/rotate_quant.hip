// rotate_quant.hip -- fused block-128 Walsh-Hadamard rotation + per-row absmax quantization.
//
// One kernel serves both sides of the method: the offline weight quantizer ("SAM 3.1 Multiplex
// INT8/INT4 ConvRot" page, "Quantization recipe": FP32 upcast, block-Hadamard transform,
// per-row scales) and the online activation quantizer ("TRELLIS.2 INT8 ConvRot in ComfyUI",
// "What ConvRot changes": the matching rotation applied to activations at run time, then
// dynamic per-token quantization). The arithmetic is fixed bit for bit (see convrot.h).
//
// Work layout (HBM-bound: one read of X, one write of the codes).
//   * A row is owned by T threads (T = 16, 32, 64, 128 or 256; T/16 lanes per block-piece
//     column); each thread holds P "pieces" of 8 consecutive elements, so K = 8 * T * P.
//     Piece p of thread t sits at element 8 * (T*p + 16*(t/16) + j(t)): every wave-wide load
//     is a contiguous run, and a 16-lane DPP row covers one 128-block.
//   * Inside a lane, the 8 elements of a piece take the butterfly stages h = 1, 2, 4.
//   * The stages h = 8, 16, 32, 64 pair pieces j and j ^ (1, 2, 4, 8). The lane->piece map
//     j(lambda) = lambda ^ (bit2(lambda) ? 3 : 0) turns those into lane masks 1, 2, 7 and 8,
//     which are single DPP row ops (quad_perm, quad_perm, row_half_mirror, row_ror:8).
//   * Sign tracking: in every cross-lane stage each lane computes mine + m * partner with
//     m = +1 on the lower and -1 on the upper lane of the pair. The upper lane then holds the
//     negated butterfly difference (fl is sign-symmetric, so this is exact); after the four
//     stages a lane's values are (-1)^popcount(j) times the true ones, which is folded into
//     the quantizer's multiplier. Absolute values are unaffected.
//   * Quantization: p = fl(u * inv) then fl(p + 1.5*2^23), whose low mantissa byte is the
//     round-half-even code (|p| <= q_max << 2^22), stored straight from the bit pattern.
// A second, generic kernel (two passes over the row: absmax, then recompute + quantize)
// covers block counts the register-resident kernel cannot hold.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace convrot {
namespace {

constexpr float kInvSqrtBlock = 0x1.6a09e6p-4f;  // binary32 nearest to 1/sqrt(128)
constexpr float kRoundMagic = 12582912.0f;       // 1.5 * 2^23

template <int DPP_CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), DPP_CTRL, 0xF, 0xF, true));
}

// 8 consecutive elements -> fp32 (exact upcast).
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&v)[8]) {
  if constexpr (DT == kF32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
    uint4 a = p[0], b = p[1];
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if constexpr (DT == kF16) {
        v[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] & 0xFFFFu)));
        v[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16)));
      } else {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  }
}

// Butterfly stages h = 1, 2, 4 on 8 consecutive elements.
__device__ __forceinline__ void fwht8(float (&v)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = __fadd_rn(a, b);
        v[i + h] = __fsub_rn(a, b);
      }
    }
  }
}

// Cross-lane stages h = 8, 16, 32, 64 (lane masks 1, 2, 7, 8), sign-tracked.
__device__ __forceinline__ void cross_stages(float (&v)[8], float m0, float m1, float m2, float m3) {
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = __builtin_fmaf(dpp_f<0xB1>(v[i]), m0, v[i]);   // quad_perm [1,0,3,2]
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = __builtin_fmaf(dpp_f<0x4E>(v[i]), m1, v[i]);   // quad_perm [2,3,0,1]
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = __builtin_fmaf(dpp_f<0x141>(v[i]), m2, v[i]);  // row_half_mirror
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = __builtin_fmaf(dpp_f<0x128>(v[i]), m3, v[i]);  // row_ror:8
}

__device__ __forceinline__ uint32_t code_bits(float u, float tinv) {
  return __float_as_uint(__fadd_rn(__fmul_rn(u, tinv), kRoundMagic));
}

// Quantize + store one piece (8 codes) at element offset `elem` of a row.
template <int BITS>
__device__ __forceinline__ void store_piece(void* Q, int64_t row_elem0, int64_t elem,
                                            const float (&v)[8], float tinv) {
  uint32_t y[8];
#pragma unroll
  for (int i = 0; i < 8; i++) y[i] = code_bits(v[i], tinv);
  if constexpr (BITS == 8) {
    uint2 o;
    o.x = (y[0] & 0xFFu) | ((y[1] & 0xFFu) << 8) | ((y[2] & 0xFFu) << 16) | (y[3] << 24);
    o.y = (y[4] & 0xFFu) | ((y[5] & 0xFFu) << 8) | ((y[6] & 0xFFu) << 16) | (y[7] << 24);
    *reinterpret_cast<uint2*>(static_cast<int8_t*>(Q) + row_elem0 + elem) = o;
  } else {
    uint32_t o = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) o |= (y[i] & 0xFu) << (4 * i);
    *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(Q) + (row_elem0 + elem) / 2) = o;
  }
}

__device__ __forceinline__ float wave_max(float a, int width) {
  for (int off = 1; off < width; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  return a;
}

// Row absmax over the T threads of a row (T <= 64: inside the wave; else through LDS).
__device__ __forceinline__ float row_max(float a, int T, float* red) {
  if (T <= 64) return wave_max(a, T);
  a = wave_max(a, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = a;
  __syncthreads();
  const int w0 = (threadIdx.x / T) * (T >> 6);
  float r = red[w0];
  for (int w = 1; w < (T >> 6); w++) r = fmaxf(r, red[w0 + w]);
  return r;
}

__device__ __forceinline__ void row_scalars(float a, float qmax, int j, float& tinv, float& scale) {
  const float inv = (a > 0.0f) ? __fdiv_rn(qmax, a) : 0.0f;
  scale = __fdiv_rn(__fmul_rn(a, kInvSqrtBlock), qmax);
  tinv = (__builtin_popcount(j) & 1) ? -inv : inv;
}

// Register-resident kernel: P pieces per thread, T threads per row, 256 threads per block.
template <int DT, int BITS, int P>
__global__ __launch_bounds__(256) void rotate_quant_kernel(const void* __restrict__ X, int64_t M,
                                                           int K, int T, void* __restrict__ Q,
                                                           float* __restrict__ S) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int t = tid % T;
  const int64_t row = (int64_t)blockIdx.x * (256 / T) + tid / T;
  const bool active = row < M;
  const int lam = t & 15;
  const int j = lam ^ (((lam >> 2) & 1) * 3);
  const int tb = t & ~15;
  const int64_t row_elem0 = row * (int64_t)K;

  float v[P][8];
#pragma unroll
  for (int p = 0; p < P; p++) {
    if (active) {
      load8<DT>(X, row_elem0 + 8 * (T * p + tb + j), v[p]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) v[p][i] = 0.0f;
    }
  }
  const float m0 = (j & 1) ? -1.0f : 1.0f, m1 = (j & 2) ? -1.0f : 1.0f;
  const float m2 = (j & 4) ? -1.0f : 1.0f, m3 = (j & 8) ? -1.0f : 1.0f;
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < P; p++) {
    fwht8(v[p]);
    cross_stages(v[p], m0, m1, m2, m3);
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(v[p][i]));
  }
  const float qmax = (BITS == 8) ? 127.0f : 7.0f;
  const float a = row_max(amax, T, red);
  float tinv, scale;
  row_scalars(a, qmax, j, tinv, scale);
  if (active) {
#pragma unroll
    for (int p = 0; p < P; p++) store_piece<BITS>(Q, row_elem0, 8 * (T * p + tb + j), v[p], tinv);
    if (t == 0) S[row] = scale;
  }
}

// Generic two-pass kernel: one 64-thread wave per row, any number of 128-blocks. Pass 1
// transforms every block to find the absmax; pass 2 re-reads, re-transforms and quantizes.
// The transform of a block is deterministic, so both passes see identical values.
template <int DT, int BITS>
__global__ __launch_bounds__(256) void rotate_quant_generic_kernel(const void* __restrict__ X,
                                                                   int64_t M, int K,
                                                                   void* __restrict__ Q,
                                                                   float* __restrict__ S) {
  const int tid = threadIdx.x;
  const int t = tid & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (tid >> 6);
  if (row >= M) return;                       // whole wave exits together (64 | 256)
  const int lam = t & 15;
  const int j = lam ^ (((lam >> 2) & 1) * 3);
  const int tb = t & ~15;
  const int64_t row_elem0 = row * (int64_t)K;
  const float m0 = (j & 1) ? -1.0f : 1.0f, m1 = (j & 2) ? -1.0f : 1.0f;
  const float m2 = (j & 4) ? -1.0f : 1.0f, m3 = (j & 8) ? -1.0f : 1.0f;
  const int nb = K / 128;                     // blocks; each 16-lane row of the wave takes one
  float amax = 0.0f;
  for (int b0 = 0; b0 < nb; b0 += 4) {
    if (b0 + (t >> 4) < nb) {
      float v[8];
      load8<DT>(X, row_elem0 + 8 * (16 * b0 + tb + j), v);
      fwht8(v);
      cross_stages(v, m0, m1, m2, m3);
#pragma unroll
      for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(v[i]));
    }
  }
  const float a = wave_max(amax, 64);
  const float qmax = (BITS == 8) ? 127.0f : 7.0f;
  float tinv, scale;
  row_scalars(a, qmax, j, tinv, scale);
  for (int b0 = 0; b0 < nb; b0 += 4) {
    // DPP needs all lanes of a 16-lane row active; the block index is uniform per DPP row.
    if (b0 + (t >> 4) < nb) {
      float v[8];
      const int64_t e = 8 * (16 * b0 + tb + j);
      load8<DT>(X, row_elem0 + e, v);
      fwht8(v);
      cross_stages(v, m0, m1, m2, m3);
      store_piece<BITS>(Q, row_elem0, e, v, tinv);
    }
  }
  if (t == 0) S[row] = scale;
}

template <int DT, int BITS, int P>
hipError_t launch_p(const void* X, int64_t M, int K, int T, void* Q, float* S, hipStream_t st) {
  const int rows_per_block = 256 / T;
  const int64_t blocks = (M + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((rotate_quant_kernel<DT, BITS, P>), dim3((unsigned)blocks), dim3(256), 0, st,
                     X, M, K, T, Q, S);
  return hipGetLastError();
}

template <int DT, int BITS>
hipError_t launch_bits(const void* X, int64_t M, int K, int T, int P, void* Q, float* S,
                       hipStream_t st) {
  switch (P) {
    case 1: return launch_p<DT, BITS, 1>(X, M, K, T, Q, S, st);
    case 2: return launch_p<DT, BITS, 2>(X, M, K, T, Q, S, st);
    case 3: return launch_p<DT, BITS, 3>(X, M, K, T, Q, S, st);
    case 4: return launch_p<DT, BITS, 4>(X, M, K, T, Q, S, st);
    case 5: return launch_p<DT, BITS, 5>(X, M, K, T, Q, S, st);
    case 6: return launch_p<DT, BITS, 6>(X, M, K, T, Q, S, st);
    case 7: return launch_p<DT, BITS, 7>(X, M, K, T, Q, S, st);
    case 8: return launch_p<DT, BITS, 8>(X, M, K, T, Q, S, st);
    default: {
      const int64_t blocks = (M + 3) / 4;
      hipLaunchKernelGGL((rotate_quant_generic_kernel<DT, BITS>), dim3((unsigned)blocks),
                         dim3(256), 0, st, X, M, K, Q, S);
      return hipGetLastError();
    }
  }
}

template <int DT>
hipError_t launch_dt(const void* X, int64_t M, int K, int bits, int T, int P, void* Q, float* S,
                     hipStream_t st) {
  return bits == 8 ? launch_bits<DT, 8>(X, M, K, T, P, Q, S, st)
                   : launch_bits<DT, 4>(X, M, K, T, P, Q, S, st);
}

}  // namespace

// Threads per row T = 16 * 2^t and pieces per thread P = (K/128) / 2^t: prefer 2 <= P <= 4
// (enough loads in flight, modest registers), else the largest T with P <= 8, else the
// generic kernel (P = 0).
void choose_rotate_quant_shape(int64_t K, int* T_out, int* P_out) {
  const int64_t nb = K / 128;
  int bestT = 0, bestP = 0;
  for (int t = 0; t <= 4; t++) {
    if (nb % (1 << t)) break;
    const int64_t P = nb >> t;
    if (P > 8) continue;
    const int T = 16 << t;
    if (bestP == 0) { bestT = T; bestP = (int)P; }
    if (P >= 2 && P <= 4) { bestT = T; bestP = (int)P; break; }
    if (bestP > 4 && P < bestP) { bestT = T; bestP = (int)P; }
  }
  *T_out = bestT;
  *P_out = bestP;
}

hipError_t launch_rotate_quant(const void* X, int dt, int64_t rows, int64_t K, int bits, void* Q,
                               float* S, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  int T, P;
  choose_rotate_quant_shape(K, &T, &P);
  switch (dt) {
    case kF32: return launch_dt<kF32>(X, rows, (int)K, bits, T, P, Q, S, stream);
    case kF16: return launch_dt<kF16>(X, rows, (int)K, bits, T, P, Q, S, stream);
    default: return launch_dt<kBF16>(X, rows, (int)K, bits, T, P, Q, S, stream);
  }
}

}  // namespace convrot
