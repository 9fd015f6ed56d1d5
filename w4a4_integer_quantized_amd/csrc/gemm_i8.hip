// gemm_i8.hip -- int8 x int8 -> int32 MFMA GEMM with the fused dequantizing epilogue.
//
// Computes acc[m, n] = sum_k Xq[m, k] * Wq[n, k] (both operands K-contiguous) and then
// Y[m, n] = fp16/bf16( fma(f32(acc), fl(w_scale[n] * x_scale[m]), bias[n]) ) -- the W8A8 /
// W4A4 "operations" of the "SAM 3.1 Multiplex INT8/INT4 ConvRot" page ("Quantization recipe")
// with the per-row weight scale and per-token activation scale. INT4 codes are multiplied on
// the INT8 matrix cores, the fallback the same page describes ("Downloads"); gfx950 has no
// int4 MFMA.
//
// Design (gfx950, 256 CUs in 8 XCDs, 160 KB LDS per CU, 64-wide waves):
//   * 256 x 256 output tile per 256-thread workgroup, 4 waves in 2 x 2, each wave 128 x 128
//     = 4 x 4 blocks of v_mfma_i32_32x32x32_i8 (256 int32 accumulators per lane).
//   * K is staged 128 bytes per step (128 int8 codes or 256 int4 codes) for both operands,
//     double-buffered in LDS (2 x 64 KB), filled with direct global->LDS 16-byte loads. Rows
//     are 128 B; the 16-byte chunk c of row r is stored at position c ^ swz(r) so the MFMA
//     fragment reads (ds_read_b128, 32 rows x 2 chunks per wave) are bank-conflict free.
//   * The MFMA "A" operand is a Wq row block and "B" an Xq row block, so each lane ends with
//     4 consecutive output columns of one token: 8-byte fp16/bf16 stores.
//   * INT4: a 16-byte chunk of packed codes (32 nibbles) becomes two MFMA operands,
//     (w << 4) & 0xF0F0F0F0 (even k) and w & 0xF0F0F0F0 (odd k): each byte is 16 * code,
//     exact for codes in [-8, 7]. Both operands get the same k permutation, so the sum is
//     unchanged; the accumulator is 256 * acc and an exact arithmetic shift by 8 recovers it.
//   * Workgroup -> tile map is XCD-aware: workgroups are dispatched round-robin over the 8
//     XCDs, so logical tile L runs on XCD L / ceil(tiles / 8); neighbouring tiles (same Xq
//     row panel, all of Wq) then share one XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;        // tokens per tile
constexpr int kBN = 256;        // output features per tile
constexpr int kBKB = 128;       // K bytes per stage
constexpr int kThreads = 256;
constexpr int kStageBytes = (kBM + kBN) * kBKB;   // 64 KB

enum OutKind { kOutS32 = 0, kOutF16 = 1, kOutBF16 = 2 };

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

typedef __attribute__((address_space(3))) void lds_void;

// One wave copies 8 rows x 128 B (1 KB) from global memory into LDS rows [row0, row0 + 8).
// Lane l fills LDS position (row0 + l/8, chunk l%8), which holds global chunk (l%8) ^ swz(row).
__device__ __forceinline__ void copy_rows(const uint8_t* __restrict__ g, int64_t ld, int row0,
                                          int grow0, int gmax, int k0, uint8_t* lds_tile,
                                          int lane) {
  const int r = row0 + (lane >> 3);
  const int c = (lane & 7) ^ swz(r);
  int gr = grow0 + r;
  gr = gr < gmax ? gr : gmax - 1;
  const uint8_t* src = g + (int64_t)gr * ld + k0 + 16 * c;
  __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(lds_tile + row0 * kBKB), 16, 0, 0);
}

__device__ __forceinline__ v4i read_frag(const uint8_t* lds_tile, int row, int chunk) {
  return *reinterpret_cast<const v4i*>(lds_tile + row * kBKB + ((chunk ^ swz(row)) << 4));
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <int BITS, int OUT>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(
    const uint8_t* __restrict__ Xq, const float* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const float* __restrict__ sw, const float* __restrict__ bias, void* __restrict__ Y, int M,
    int N, int Kb, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStageBytes];

  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + 7) >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= ntiles) return;
  const int tm = logical / tiles_n;
  const int tn = logical - tm * tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  v16i acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; a++)
#pragma unroll
    for (int b = 0; b < 4; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[a][b][r] = 0;

  auto issue = [&](int stage, int k0) {
    uint8_t* tX = lds + stage * kStageBytes;
    uint8_t* tW = tX + kBM * kBKB;
#pragma unroll
    for (int i = 0; i < 8; i++) copy_rows(Xq, Kb, (wave * 8 + i) * 8, m0, M, k0, tX, lane);
#pragma unroll
    for (int i = 0; i < 8; i++) copy_rows(Wq, Kb, (wave * 8 + i) * 8, n0, N, k0, tW, lane);
  };

  auto compute = [&](int stage) {
    const uint8_t* tX = lds + stage * kStageBytes;
    const uint8_t* tW = tX + kBM * kBKB;
    const int rsub = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const int chunk = 2 * ks + half;
      v4i wf[4], xf[4];
#pragma unroll
      for (int a = 0; a < 4; a++) wf[a] = read_frag(tW, wn * 128 + a * 32 + rsub, chunk);
#pragma unroll
      for (int b = 0; b < 4; b++) xf[b] = read_frag(tX, wm * 128 + b * 32 + rsub, chunk);
      if constexpr (BITS == 8) {
#pragma unroll
        for (int a = 0; a < 4; a++)
#pragma unroll
          for (int b = 0; b < 4; b++)
            acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[a], xf[b], acc[a][b], 0, 0, 0);
      } else {
        v4i wlo[4], whi[4], xlo[4], xhi[4];
#pragma unroll
        for (int a = 0; a < 4; a++)
#pragma unroll
          for (int e = 0; e < 4; e++) {
            wlo[a][e] = (wf[a][e] << 4) & 0xF0F0F0F0;
            whi[a][e] = wf[a][e] & 0xF0F0F0F0;
          }
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
          for (int e = 0; e < 4; e++) {
            xlo[b][e] = (xf[b][e] << 4) & 0xF0F0F0F0;
            xhi[b][e] = xf[b][e] & 0xF0F0F0F0;
          }
#pragma unroll
        for (int a = 0; a < 4; a++)
#pragma unroll
          for (int b = 0; b < 4; b++) {
            acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wlo[a], xlo[b], acc[a][b], 0, 0, 0);
            acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(whi[a], xhi[b], acc[a][b], 0, 0, 0);
          }
      }
    }
  };

  const int nk = Kb / kBKB;
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < nk) issue(cur ^ 1, (kt + 1) * kBKB);
    compute(cur);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // Epilogue. Lane l of block (a, b) holds D[n][m] for m = b*32 + l%32 and
  // n = a*32 + 8*(r/4) + 4*(l/32) + r%4, r = 0..15.
  const int msub = lane & 31, nq = 4 * (lane >> 5);
#pragma unroll
  for (int b = 0; b < 4; b++) {
    const int m = m0 + wm * 128 + b * 32 + msub;
    if (m >= M) continue;
    const float xs = (OUT == kOutS32) ? 0.0f : sx[m];
#pragma unroll
    for (int a = 0; a < 4; a++) {
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int n = n0 + wn * 128 + a * 32 + 8 * g + nq;
        if (n >= N) continue;
        int v[4];
#pragma unroll
        for (int e = 0; e < 4; e++) v[e] = (BITS == 4) ? (acc[a][b][4 * g + e] >> 8) : acc[a][b][4 * g + e];
        if constexpr (OUT == kOutS32) {
          int4 o = make_int4(v[0], v[1], v[2], v[3]);
          *reinterpret_cast<int4*>(static_cast<int32_t*>(Y) + (int64_t)m * N + n) = o;
        } else {
          const float4 s4 = *reinterpret_cast<const float4*>(sw + n);
          const float4 b4 = bias ? *reinterpret_cast<const float4*>(bias + n) : make_float4(0.f, 0.f, 0.f, 0.f);
          const float ws[4] = {s4.x, s4.y, s4.z, s4.w};
          const float bs[4] = {b4.x, b4.y, b4.z, b4.w};
          uint16_t h[4];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const float y = __builtin_fmaf(static_cast<float>(v[e]), __fmul_rn(ws[e], xs), bs[e]);
            h[e] = (OUT == kOutF16) ? f32_to_f16_rne(y) : f32_to_bf16_rne(y);
          }
          uint2 o;
          o.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
          o.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Y) + (int64_t)m * N + n) = o;
        }
      }
    }
  }
}

template <int BITS, int OUT>
hipError_t launch(const void* Xq, const float* sx, const void* Wq, const float* sw,
                  const float* bias, int64_t M, int64_t N, int64_t Kb, void* Y, hipStream_t st) {
  const int tiles_m = (int)((M + kBM - 1) / kBM);
  const int tiles_n = (int)((N + kBN - 1) / kBN);
  const int ntiles = tiles_m * tiles_n;
  const int grid = ((ntiles + 7) / 8) * 8;
  hipLaunchKernelGGL((gemm_kernel<BITS, OUT>), dim3(grid), dim3(kThreads), 0, st,
                     static_cast<const uint8_t*>(Xq), sx, static_cast<const uint8_t*>(Wq), sw,
                     bias, Y, (int)M, (int)N, (int)Kb, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const void* Xq, const float* sx, const void* Wq, const float* sw,
                       const float* bias, int64_t M, int64_t N, int64_t K, int bits, void* Y,
                       int out_dt, int32_t* acc32, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t Kb = bits == 8 ? K : K / 2;
  if (acc32) {
    return bits == 8 ? launch<8, kOutS32>(Xq, sx, Wq, sw, bias, M, N, Kb, acc32, stream)
                     : launch<4, kOutS32>(Xq, sx, Wq, sw, bias, M, N, Kb, acc32, stream);
  }
  if (out_dt == kF16)
    return bits == 8 ? launch<8, kOutF16>(Xq, sx, Wq, sw, bias, M, N, Kb, Y, stream)
                     : launch<4, kOutF16>(Xq, sx, Wq, sw, bias, M, N, Kb, Y, stream);
  return bits == 8 ? launch<8, kOutBF16>(Xq, sx, Wq, sw, bias, M, N, Kb, Y, stream)
                   : launch<4, kOutBF16>(Xq, sx, Wq, sw, bias, M, N, Kb, Y, stream);
}

}  // namespace convrot
