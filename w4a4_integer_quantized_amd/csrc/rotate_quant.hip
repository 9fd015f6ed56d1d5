// rotate_quant.hip -- fused block-128 Walsh-Hadamard rotation + per-row absmax quantization.
//
// One kernel serves both sides of the method: the offline weight quantizer ("SAM 3.1 Multiplex
// INT8/INT4 ConvRot" page, "Quantization recipe": FP32 upcast, block-Hadamard transform,
// per-row scales) and the online activation quantizer ("TRELLIS.2 INT8 ConvRot in ComfyUI",
// "What ConvRot changes": the matching rotation applied to activations at run time, then
// dynamic per-token quantization). The arithmetic is fixed bit for bit (see convrot.h).
//
// Work layout (HBM-bound: one read of X, one write of the codes).
//   * Main kernel (int8 / int4 codes, row-major or tiled; rotate_quant_coalesced_kernel): a
//     16-lane group covers a 128-block per load, lane u holding the 8-element chunk
//     c(u) = u ^ (3 * ((u >> 2) & 1)). Element 8c + r of the block has its bits r (h = 1, 2, 4)
//     inside the lane and its chunk bits (h = 8, 16, 32, 64) across the group; with this
//     relabelling of lanes, flipping chunk bit k is lane xor 1, 2, 7 or 8, i.e. the DPP
//     exchanges quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror and row_ror:8, each
//     fused into one v_fmac_f32. Every load instruction then reads whole consecutive blocks
//     (fully coalesced, nontemporal: X is read once) and the codes leave as 8-byte (int8) or
//     4-byte (int4) stores. These stay ordinary stores: the GEMM reads the codes next, and
//     nontemporal ones (which leave them out of the caches) measured about 45 us slower on the
//     following 41472 x 3072 x 1024 GEMM. A row of nb blocks takes 16 * G lanes, each lane
//     holding NI = nb / G <= 4 chunks: few values per lane keep registers low and many waves
//     resident, which is what hides the memory latency. Loads and stores are buffer operations
//     with 32-bit offsets from the workgroup's first row; int8 codes are packed by the
//     rounding add itself (SDWA byte select).
//   * A second register-resident kernel (rotate_quant_kernel) serves block counts the first
//     does not take and the FP6 tile layout: a 4-lane quad owns a 128-block, lane t holding the
//     32 consecutive elements 32*t .. 32*t + 31 (bits r, i in the lane, t across the quad), and
//     stores its 32 codes as one contiguous run. A row of nb blocks is owned by QPR = nb / BPQ
//     quads, each holding BPQ blocks; a row takes a slot of L lanes: the next power of two of
//     4*QPR when that fits a wave (idle quads re-read a valid block, are left out of the absmax
//     and store nothing), else exactly 4*QPR = 128..256 lanes over 2..4 waves that combine their
//     absmax through LDS.
//   * Butterfly stages in the fixed order h = 1, 2, 4, 8, 16, 32, 64. For fp16 input the first
//     stage also does the exact upcast: fma(x0, +-1, x1) on the two halves of a dword
//     (v_fma_mix_f32) is the single fp32 rounding of x0 +- x1.
//   * Sign tracking in the cross-lane stages: each lane computes mine + m * partner with
//     m = +1 on the lower and -1 on the upper lane of the pair. The upper lane then holds the
//     negated butterfly difference (fl is sign-symmetric, so this is exact); a lane's values are
//     then (-1)^popcount(j) times the true ones (j: the lane's cross-lane index bits; later
//     stages pair lanes with equal sign factors), which is folded into the quantizer's
//     multiplier. Absolute values are unaffected.
//   * Quantization: p = fl(u * inv) then fl(p + 1.5*2^23), whose low mantissa byte is the
//     round-half-even code (|p| <= q_max << 2^22).
// A third, generic kernel (two passes over the row: absmax, then recompute + quantize, one
// wave per row with 16 lanes per block) covers the remaining block counts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace convrot {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kInvSqrtBlock = 0x1.6a09e6p-4f;  // binary32 nearest to 1/sqrt(128)
constexpr float kRoundMagic = 12582912.0f;       // 1.5 * 2^23

template <int DPP_CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), DPP_CTRL, 0xF, 0xF, true));
}

// 16 bytes at p.
__device__ __forceinline__ u32x4 load16(const void* p) { return *static_cast<const u32x4*>(p); }

// 8 consecutive elements -> fp32 (exact upcast).
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&v)[8]) {
  if constexpr (DT == kF32) {
    const float* p = static_cast<const float*>(base) + elem;
    const u32x4 a = load16(p), b = load16(p + 4);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
    }
  } else {
    const u32x4 a = load16(static_cast<const uint16_t*>(base) + elem);
    const uint32_t w[4] = {a[0], a[1], a[2], a[3]};
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

// Byte offset of code byte kb (of Kb per row) of row `row`: row-major, or the tiled layout of
// convrot.h ([256-row panel][64-byte k step][256 rows][64 B]; Kb is a multiple of 64).
__device__ __forceinline__ int64_t code_offset(int64_t row, int64_t kb, int64_t Kb, bool tiled) {
  if (!tiled) return row * Kb + kb;
  return (((row >> 8) * (Kb >> 6) + (kb >> 6)) << 14) + ((row & 255) << 6) + (kb & 63);
}

// Quantize + store one piece (8 codes) at `dst` (their bytes are contiguous in both layouts).
template <int BITS>
__device__ __forceinline__ void store_piece(uint8_t* dst, const float (&v)[8], float tinv) {
  uint32_t y[8];
#pragma unroll
  for (int i = 0; i < 8; i++) y[i] = code_bits(v[i], tinv);
  if constexpr (BITS == 8) {
    uint2 o;
    o.x = (y[0] & 0xFFu) | ((y[1] & 0xFFu) << 8) | ((y[2] & 0xFFu) << 16) | (y[3] << 24);
    o.y = (y[4] & 0xFFu) | ((y[5] & 0xFFu) << 8) | ((y[6] & 0xFFu) << 16) | (y[7] << 24);
    *reinterpret_cast<uint2*>(dst) = o;
  } else {
    uint32_t o = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) o |= (y[i] & 0xFu) << (4 * i);
    *reinterpret_cast<uint32_t*>(dst) = o;
  }
}

__device__ __forceinline__ float wave_max(float a, int width) {
  for (int off = 1; off < width; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  return a;
}

// The row's multiplier and scale. A row whose absmax is zero, or too small for fl(q_max / a)
// to be finite, is quantized as a zero row: multiplier 0 (every code 0) and scale 0.
__device__ __forceinline__ void row_scalars(float a, float qmax, int j, float& tinv, float& scale) {
  float inv = (a > 0.0f) ? __fdiv_rn(qmax, a) : 0.0f;
  if (__builtin_isinf(inv)) inv = 0.0f;
  scale = inv != 0.0f ? __fdiv_rn(__fmul_rn(a, kInvSqrtBlock), qmax) : 0.0f;
  tinv = (__builtin_popcount(j) & 1) ? -inv : inv;
}

// Butterfly on the two fp16 halves a (low) and b (high) of a dword, fused with the exact
// upcast: v_fma_mix_f32 takes fp16 operands exactly and rounds a*(+-1) + b once to fp32, i.e.
// fl(a + b) and fl(a - b). (Written out because the compiler turns fma(x, 1, y) into an add
// and then needs separate conversions.)
__device__ __forceinline__ void bfly_f16(uint32_t w, float& lo, float& hi) {
  asm("v_fma_mix_f32 %0, %2, 1.0, %2 op_sel:[0,0,1] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mix_f32 %1, %2, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,1]"
      : "=&v"(lo), "=v"(hi)
      : "v"(w));
}

// Load piece (8 elements) and apply butterfly stage h = 1 (with the upcast).
template <int DT>
__device__ __forceinline__ void load_stage1(const void* base, int64_t elem, float (&v)[8]) {
  if constexpr (DT == kF16) {
    const u32x4 a = load16(static_cast<const uint16_t*>(base) + elem);
    bfly_f16(a[0], v[0], v[1]);
    bfly_f16(a[1], v[2], v[3]);
    bfly_f16(a[2], v[4], v[5]);
    bfly_f16(a[3], v[6], v[7]);
  } else {
    load8<DT>(base, elem, v);
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float a = v[i], b = v[i + 1];
      v[i] = __fadd_rn(a, b);
      v[i + 1] = __fsub_rn(a, b);
    }
  }
}

// Stages h = 2, 4 inside a piece.
__device__ __forceinline__ void stages_2_4(float (&v)[8]) {
#pragma unroll
  for (int h = 2; h < 8; h <<= 1) {
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

__device__ __forceinline__ void bfly_pieces(float (&x)[8], float (&y)[8]) {
#pragma unroll
  for (int r = 0; r < 8; r++) {
    const float a = x[r], b = y[r];
    x[r] = __fadd_rn(a, b);
    y[r] = __fsub_rn(a, b);
  }
}

// Code bytes of 8 quantized values -> int8 pair of dwords or one int4 dword.
__device__ __forceinline__ uint32_t pack4_i8(uint32_t y0, uint32_t y1, uint32_t y2, uint32_t y3) {
  const uint32_t lo = __builtin_amdgcn_perm(y1, y0, 0x0c0c0400u);   // [y0.b0, y1.b0, 0, 0]
  const uint32_t hi = __builtin_amdgcn_perm(y3, y2, 0x04000c0cu);   // [0, 0, y2.b0, y3.b0]
  return lo | hi;
}

// Quantize + store the 32 consecutive codes of v[0..3] at `dst` (32 or 16 contiguous bytes in
// both layouts: a lane's run never crosses a 64-byte k step).
template <int BITS>
__device__ __forceinline__ void quant_store32(uint8_t* dst, const float (&v)[4][8], float tinv) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    uint32_t y[8];
#pragma unroll
    for (int r = 0; r < 8; r++) y[r] = code_bits(v[i][r], tinv);
    if constexpr (BITS == 8) {
      w[2 * i] = pack4_i8(y[0], y[1], y[2], y[3]);
      w[2 * i + 1] = pack4_i8(y[4], y[5], y[6], y[7]);
    } else {
      uint32_t o = 0;
#pragma unroll
      for (int r = 0; r < 8; r++) o |= (y[r] & 0xFu) << (4 * r);
      w[i] = o;
    }
  }
  if constexpr (BITS == 8) {
    uint4* p = reinterpret_cast<uint4*>(dst);
    p[0] = make_uint4(w[0], w[1], w[2], w[3]);
    p[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---- FP6 tiles (4-bit codes stored as FP6 E2M3 for the FP6 matrix cores; see convrot.h) ----
// Byte `b` (0..23) of the 24-byte operand string of row `row`, 64-element slice `s`, half `h`,
// in panels of P rows: plane 1 (bytes 0..15, 32 B per row) then plane 2 (bytes 16..23, 16 B per
// row), each with its two halves swapped on row bit 3 (plane 1) or bit 4 (plane 2).
__device__ __forceinline__ int64_t fp6_offset(int64_t row, int s, int h, int b, int P, int nsl) {
  const int64_t base = ((row / P) * nsl + s) * (int64_t)(P * 48);
  const int rr = (int)(row % P);
  if (b < 16) return base + rr * 32 + 16 * (h ^ ((rr >> 3) & 1)) + b;
  return base + P * 32 + rr * 16 + 8 * (h ^ ((rr >> 4) & 1)) + (b - 16);
}

// FP6 E2M3 bytes of four codes given as two's-complement bytes in [-7, 7]: byte permutes look
// the low three bits up in {0, 8, 16, 20, 24, 26, 28, 30} (0, 1.0, 2.0, 1.5 * 2, 4.0,
// 1.25 * 4, 1.5 * 4, 1.75 * 4) for non-negative codes and in the patterns of -(8 - j) (sign bit
// 32 set) for negative ones, and a bytewise select by the sign picks one.
__device__ __forceinline__ uint32_t fp6_bytes(uint32_t d) {
  const uint32_t j = d & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(0x1E1C1A18u, 0x14100800u, j);
  const uint32_t neg = __builtin_amdgcn_perm(0x28303438u, 0x3A3C3E00u, j);
  const uint32_t s = ((d >> 7) & 0x01010101u) * 0xFFu;   // 0xFF in the bytes of negative codes
  return (neg & s) | (pos & ~s);
}

// Four 6-bit codes (the low six bits of each byte of c) -> one 24-bit field, code i at bit 6i.
__device__ __forceinline__ uint32_t pack6x4(uint32_t c) {
  uint32_t g = (c & 0x3Fu) | ((c >> 2) & ~0x3Fu);
  g = (g & 0xFFFu) | ((c >> 4) & ~0xFFFu);
  return (g & 0x3FFFFu) | ((c >> 6) & ~0x3FFFFu);
}

// Quantize the 32 consecutive values of v[0..3] (one lane's operand string: half h of slice s)
// and store them as FP6 tiles.
__device__ __forceinline__ void quant_store32_fp6(uint8_t* Q, int64_t row, int s, int h, int P, int nsl,
                                                  const float (&v)[4][8], float tinv) {
  uint32_t g[8];
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int q = 0; q < 2; q++) {
      uint32_t y[4];
#pragma unroll
      for (int r = 0; r < 4; r++) y[r] = code_bits(v[i][4 * q + r], tinv);
      g[2 * i + q] = pack6x4(fp6_bytes(pack4_i8(y[0], y[1], y[2], y[3])));
    }
  }
  const uint4 lo = make_uint4(g[0] | (g[1] << 24), (g[1] >> 8) | (g[2] << 16), (g[2] >> 16) | (g[3] << 8),
                              g[4] | (g[5] << 24));
  const uint2 hi = make_uint2((g[5] >> 8) | (g[6] << 16), (g[6] >> 16) | (g[7] << 8));
  *reinterpret_cast<uint4*>(Q + fp6_offset(row, s, h, 0, P, nsl)) = lo;
  *reinterpret_cast<uint2*>(Q + fp6_offset(row, s, h, 16, P, nsl)) = hi;
}

// The same for one piece of 8 consecutive values (elements 8q .. 8q+7 of the string, 6 bytes at
// byte 6q), written as three 16-bit words (each lies within one plane).
__device__ __forceinline__ void store_piece_fp6(uint8_t* Q, int64_t row, int s, int h, int q, int P, int nsl,
                                                const float (&v)[8], float tinv) {
  uint32_t g[2];
#pragma unroll
  for (int k = 0; k < 2; k++) {
    uint32_t y[4];
#pragma unroll
    for (int r = 0; r < 4; r++) y[r] = code_bits(v[4 * k + r], tinv);
    g[k] = pack6x4(fp6_bytes(pack4_i8(y[0], y[1], y[2], y[3])));
  }
  const uint16_t w[3] = {static_cast<uint16_t>(g[0] & 0xFFFFu),
                         static_cast<uint16_t>((g[0] >> 16) | ((g[1] & 0xFFu) << 8)),
                         static_cast<uint16_t>(g[1] >> 8)};
#pragma unroll
  for (int k = 0; k < 3; k++) *reinterpret_cast<uint16_t*>(Q + fp6_offset(row, s, h, 6 * q + 2 * k, P, nsl)) = w[k];
}

// Register-resident kernel: BPQ blocks per quad, QPR quads per row, rows in slots of L lanes
// (blockDim.x = 256 with 256 / L rows per workgroup, or blockDim.x = L > 64 with one row).
template <int DT, int BITS, int BPQ>
__global__ __launch_bounds__(256) void rotate_quant_kernel(const void* __restrict__ X, int64_t M,
                                                           int K, int L, int qpr,
                                                           uint8_t* __restrict__ Q,
                                                           float* __restrict__ S, int layout) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  // L is a power of two <= 64 (256 / L rows per block) or the whole block (one row).
  const bool one_row = L > 64;
  const int lg = __builtin_ctz(one_row ? 64 : L);
  const int t = one_row ? tid : (tid & (L - 1));
  const int64_t row = one_row ? (int64_t)blockIdx.x : ((int64_t)blockIdx.x << (8 - lg)) + (tid >> lg);
  const bool active = row < M;
  const int q = t >> 2, tq = t & 3;
  const bool qvalid = q < qpr;
  const int qc = qvalid ? q : qpr - 1;
  // Rows past the end and idle quads re-read valid data (never stored): no divergent path.
  const int64_t load_elem0 = (active ? row : M - 1) * (int64_t)K;

  float v[BPQ][4][8];
#pragma unroll
  for (int be = 0; be < BPQ; be++) {
    const int64_t blk = load_elem0 + (int64_t)(be * qpr + qc) * 128;
#pragma unroll
    for (int i = 0; i < 4; i++) load_stage1<DT>(X, blk + 32 * tq + 8 * i, v[be][i]);
  }
  const float m0 = (tq & 1) ? -1.0f : 1.0f, m1 = (tq & 2) ? -1.0f : 1.0f;
  float amax = 0.0f;
#pragma unroll
  for (int be = 0; be < BPQ; be++) {
#pragma unroll
    for (int i = 0; i < 4; i++) stages_2_4(v[be][i]);
    bfly_pieces(v[be][0], v[be][1]);     // h = 8
    bfly_pieces(v[be][2], v[be][3]);
    bfly_pieces(v[be][0], v[be][2]);     // h = 16
    bfly_pieces(v[be][1], v[be][3]);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int r = 0; r < 8; r++) v[be][i][r] = __builtin_fmaf(dpp_f<0xB1>(v[be][i][r]), m0, v[be][i][r]);   // h = 32
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int r = 0; r < 8; r++) v[be][i][r] = __builtin_fmaf(dpp_f<0x4E>(v[be][i][r]), m1, v[be][i][r]);   // h = 64
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int r = 0; r < 8; r += 2) amax = fmaxf(amax, fmaxf(fabsf(v[be][i][r]), fabsf(v[be][i][r + 1])));
  }
  amax = qvalid ? amax : 0.0f;
  float a;
  if (L <= 64) {
    a = wave_max(amax, L);
  } else {
    a = wave_max(amax, 64);
    if ((tid & 63) == 0) red[tid >> 6] = a;
    __syncthreads();
    a = red[0];
    for (int w = 1; w < (L >> 6); w++) a = fmaxf(a, red[w]);
  }
  const float qmax = (BITS == 8) ? 127.0f : 7.0f;
  float tinv, scale;
  row_scalars(a, qmax, tq, tinv, scale);
  if (active && qvalid) {
#pragma unroll
    for (int be = 0; be < BPQ; be++) {
      if constexpr (BITS == 6) {
        // Lane tq holds half tq & 1 of 64-element slice tq >> 1 of its block.
        quant_store32_fp6(Q, row, 2 * (be * qpr + q) + (tq >> 1), tq & 1, layout, K >> 6, v[be], tinv);
      } else {
        const int64_t Kb = (int64_t)K * BITS / 8;
        const int64_t kb = ((int64_t)(be * qpr + q) * 128 + 32 * tq) * BITS / 8;
        quant_store32<BITS>(Q + code_offset(row, kb, Kb, layout != 0), v[be], tinv);
      }
    }
  }
  if (active && t == 0) S[row] = scale;
}

// Generic two-pass kernel: one 64-thread wave per row, any number of 128-blocks. Pass 1
// transforms every block to find the absmax; pass 2 re-reads, re-transforms and quantizes.
// The transform of a block is deterministic, so both passes see identical values.
template <int DT, int BITS>
__global__ __launch_bounds__(256) void rotate_quant_generic_kernel(const void* __restrict__ X,
                                                                   int64_t M, int K,
                                                                   uint8_t* __restrict__ Q,
                                                                   float* __restrict__ S,
                                                                   int layout) {
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
      if constexpr (BITS == 6) {
        // Element e of the row: slice e / 64, half (e / 32) & 1, piece (e / 8) & 3 of the string.
        store_piece_fp6(Q, row, (int)(e >> 6), (int)(e >> 5) & 1, (int)(e >> 3) & 3, layout, K >> 6, v, tinv);
      } else {
        store_piece<BITS>(Q + code_offset(row, e * BITS / 8, (int64_t)K * BITS / 8, layout != 0), v, tinv);
      }
    }
  }
  if (t == 0) S[row] = scale;
}

// ---- Coalesced register-resident kernel (int8 / int4 codes, row-major or tiled) ----
// v[r] = partner(v[r]) * m + v[r] on 8 registers, the partner read through DPP (CTRL): one
// v_fmac_f32 with a DPP source per value, i.e. the single rounding of v +- partner. Each
// instruction reads only the register it writes, so only the first can follow the VALU write of
// its source; the leading s_nop covers the DPP read-after-write (and exec-write) wait states.
#define RQ_FMAC_DPP8(CTRL)                                                                        \
  asm volatile("s_nop 4\n\t"                                                                      \
               "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                \
               "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                \
               "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                \
               "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                \
               "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                \
               "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                \
               "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                \
               "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"                    \
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),         \
                 "+v"(v[6]), "+v"(v[7])                                                           \
               : "v"(m))

// Cross-lane stages h = 8, 16, 32, 64 on a chunk held by lane u of a 16-lane group with chunk
// index c(u) = u ^ (3 * ((u >> 2) & 1)): flipping bit k of c is lane xor 1, 2, 7, 8, i.e.
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror and row_ror:8. Sign-tracked with
// m_k = -1 on the lane whose bit k of c is set, as in the quad scheme above.
__device__ __forceinline__ void stage_h8(float (&v)[8], float m) { RQ_FMAC_DPP8("quad_perm:[1,0,3,2]"); }
__device__ __forceinline__ void stage_h16(float (&v)[8], float m) { RQ_FMAC_DPP8("quad_perm:[2,3,0,1]"); }
__device__ __forceinline__ void stage_h32(float (&v)[8], float m) { RQ_FMAC_DPP8("row_half_mirror"); }
__device__ __forceinline__ void stage_h64(float (&v)[8], float m) { RQ_FMAC_DPP8("row_ror:8"); }
#undef RQ_FMAC_DPP8

// max(a, |x|, |y|) in one instruction.
__device__ __forceinline__ float max_abs2(float a, float x, float y) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(r) : "v"(x), "v"(y), "v"(a));
  return r;
}

// Max over the 16 lanes of a DPP row (the same four exchanges as the stages), each step one
// v_max_f32 with a DPP source (s_nop 1: the wait states of a DPP read after a VALU write).
__device__ __forceinline__ float row16_max(float a) {
  asm volatile("s_nop 1\n\t"
               "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
               "s_nop 1\n\t"
               "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
               "s_nop 1\n\t"
               "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
               "s_nop 1\n\t"
               "v_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf"
               : "+v"(a));
  return a;
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// The int8 codes of 8 values as two dwords: p = fl(u * tinv), then fl(p + 1.5 * 2^23), whose low
// byte is the code, written straight into byte i of the dword by the add itself (SDWA
// dst_sel:BYTE_i, the other bytes kept).
__device__ __forceinline__ u32x2 quant8_i8(const float (&v)[8], float tinv) {
  const float magic = kRoundMagic;
  uint32_t d[2];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const float p0 = __fmul_rn(v[4 * h], tinv), p1 = __fmul_rn(v[4 * h + 1], tinv);
    const float p2 = __fmul_rn(v[4 * h + 2], tinv), p3 = __fmul_rn(v[4 * h + 3], tinv);
    uint32_t w;
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD"
        : "=v"(w) : "v"(p0), "v"(magic));
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(w) : "v"(p1), "v"(magic));
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(w) : "v"(p2), "v"(magic));
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(w) : "v"(p3), "v"(magic));
    d[h] = w;
  }
  return u32x2{d[0], d[1]};
}

// The int4 codes of 8 values, code i in bits 4i .. 4i+3.
__device__ __forceinline__ uint32_t quant8_i4(const float (&v)[8], float tinv) {
  uint32_t o = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) o |= (code_bits(v[i], tinv) & 0xFu) << (4 * i);
  return o;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rq_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr int kNt = 2;   // buffer-load cache policy: nontemporal (X is streamed once)

// A row of nb = G * NI blocks takes a slot of S = 16 * G lanes: 16-lane group g (0..G-1) holds
// blocks g, g + G, ..., g + (NI - 1) * G, lane u of the group the chunk c(u) (elements 8c .. 8c+7)
// of each. So load i of a slot reads G consecutive blocks (256 * G contiguous bytes of fp16/bf16,
// lanes in a permuted order): fully coalesced, and nontemporal since X is read exactly once.
// Stages h = 1, 2, 4 run inside a lane, h = 8 .. 64 across the group (stage_h8 .. stage_h64).
// S = 16, 32 or 64 lanes (R = 256 / S rows per 256-thread workgroup), or S = 128, 192, 256
// (R = 1 row per workgroup of S threads, the waves combining their absmax through LDS).
// Loads and stores are buffer operations on resources based at the workgroup's first row (its R
// rows lie in one 256-row panel of the tiled layout, as R divides 256): 32-bit offsets whose
// per-load step is uniform, and rows past M read as zeros (their codes are not stored).
template <int DT, int BITS, int NI, bool TILED>
__global__ __launch_bounds__(256) void rotate_quant_coalesced_kernel(const void* __restrict__ X,
                                                                     int64_t M, int K, int S,
                                                                     uint8_t* __restrict__ Q,
                                                                     float* __restrict__ scales) {
  constexpr int kEs = DT == kF32 ? 4 : 2;
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const bool multi = S > 64;
  const int lg = __builtin_ctz(multi ? 64 : S);
  const int R = multi ? 1 : 256 >> lg;              // rows per workgroup
  const int t = multi ? tid : (tid & (S - 1));
  const int r = multi ? 0 : tid >> lg;              // row slot within the workgroup
  const int64_t row0 = (int64_t)blockIdx.x * R;
  const int64_t row = row0 + r;
  const bool active = row < M;
  const int rows_here = (int)(M - row0 < R ? M - row0 : R);
  const int G = S >> 4;
  const int g = t >> 4, u = t & 15;
  const int c = u ^ (3 * ((u >> 2) & 1));

  const __amdgpu_buffer_rsrc_t xrs =
      rq_rsrc(static_cast<const uint8_t*>(X) + row0 * K * kEs, (uint32_t)(rows_here * K * kEs));
  const uint32_t xoff = (uint32_t)((r * K + g * 128 + 8 * c) * kEs);
  const int xstep = G * 128 * kEs;
  float v[NI][8];
#pragma unroll
  for (int i = 0; i < NI; i++) {
    if constexpr (DT == kF16) {
      const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff, i * xstep, kNt));
      bfly_f16(a[0], v[i][0], v[i][1]);
      bfly_f16(a[1], v[i][2], v[i][3]);
      bfly_f16(a[2], v[i][4], v[i][5]);
      bfly_f16(a[3], v[i][6], v[i][7]);
    } else {
      if constexpr (DT == kF32) {
        const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff, i * xstep, kNt));
        const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff + 16, i * xstep, kNt));
#pragma unroll
        for (int j = 0; j < 4; j++) {
          v[i][j] = __uint_as_float(a[j]);
          v[i][4 + j] = __uint_as_float(b[j]);
        }
      } else {
        const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff, i * xstep, kNt));
#pragma unroll
        for (int j = 0; j < 4; j++) {
          v[i][2 * j] = __uint_as_float(a[j] << 16);
          v[i][2 * j + 1] = __uint_as_float(a[j] & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float x0 = v[i][j], x1 = v[i][j + 1];
        v[i][j] = __fadd_rn(x0, x1);
        v[i][j + 1] = __fsub_rn(x0, x1);
      }
    }
  }
  const float m0 = (c & 1) ? -1.0f : 1.0f, m1 = (c & 2) ? -1.0f : 1.0f;
  const float m2 = (c & 4) ? -1.0f : 1.0f, m3 = (c & 8) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < NI; i++) stages_2_4(v[i]);
#pragma unroll
  for (int i = 0; i < NI; i++) stage_h8(v[i], m0);
#pragma unroll
  for (int i = 0; i < NI; i++) stage_h16(v[i], m1);
#pragma unroll
  for (int i = 0; i < NI; i++) stage_h32(v[i], m2);
#pragma unroll
  for (int i = 0; i < NI; i++) stage_h64(v[i], m3);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NI; i++)
#pragma unroll
    for (int j = 0; j < 8; j += 2) amax = max_abs2(amax, v[i][j], v[i][j + 1]);
  float a = row16_max(amax);
  if (S >= 32) a = fmaxf(a, __shfl_xor(a, 16, 64));
  if (S >= 64) a = fmaxf(a, __shfl_xor(a, 32, 64));
  if (multi) {
    if ((tid & 63) == 0) red[tid >> 6] = a;
    __syncthreads();
    a = red[0];
    for (int w = 1; w < (S >> 6); w++) a = fmaxf(a, red[w]);
  }
  const float qmax = (BITS == 8) ? 127.0f : 7.0f;
  float tinv, scale;
  row_scalars(a, qmax, c, tinv, scale);
  if (active) {
    // Code byte kb = (block * 128 + 8c) * BITS / 8 of the row; load i is block g + i * G.
    const int Kb = K * BITS / 8;
    const int kb0 = (g * 128 + 8 * c) * BITS / 8;
    uint32_t qbase_rows, qoff;
    int qstep;
    if constexpr (TILED) {
      qbase_rows = 256u * (uint32_t)Kb;           // the panel
      qoff = (uint32_t)(((kb0 >> 6) << 14) + ((int)(row & 255) << 6) + (kb0 & 63));
      qstep = (G * 128 * BITS / 8 / 64) << 14;    // k steps per load, times the step stride
    } else {
      qbase_rows = (uint32_t)(rows_here * Kb);
      qoff = (uint32_t)(r * Kb + kb0);
      qstep = G * 128 * BITS / 8;
    }
    uint8_t* const qb = TILED ? Q + (row0 >> 8) * 256 * (int64_t)Kb : Q + row0 * (int64_t)Kb;
    const __amdgpu_buffer_rsrc_t qrs = rq_rsrc(qb, qbase_rows);
#pragma unroll
    for (int i = 0; i < NI; i++) {
      if constexpr (BITS == 8)
        __builtin_amdgcn_raw_buffer_store_b64(quant8_i8(v[i], tinv), qrs, qoff, i * qstep, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b32(quant8_i4(v[i], tinv), qrs, qoff, i * qstep, 0);
    }
    if (t == 0) scales[row] = scale;
  }
}

// Slot of the coalesced kernel for nb blocks per row: G in {1, 2, 4, 8, 12, 16} (S = 16 * G
// lanes) with nb = G * NI, NI <= 4; {0, 0} when there is none. Below 24 blocks the smallest
// such G (rows within one wave: at K = 1024, 32 lanes per row measured 23.3 us against 30.4 for
// 128), from 24 blocks the largest (fewer values per lane across more waves: at K = 4096 int8,
// 16.0 us with 256 lanes per row against 19.4 with 128; at K = 6144, 31.7 against 32.9).
struct RqCoalesced {
  int G;
  int NI;
};

RqCoalesced choose_coalesced(int64_t nb) {
  const int gs[6] = {1, 2, 4, 8, 12, 16};
  for (int i = 0; i < 6; i++) {
    const int G = nb < 24 ? gs[i] : gs[5 - i];
    if (nb % G == 0 && nb / G <= 4) return {G, (int)(nb / G)};
  }
  return {0, 0};
}

template <int DT, int BITS, int NI, bool TILED>
hipError_t launch_coalesced_ni(const void* X, int64_t M, int K, int G, uint8_t* Q, float* S,
                               hipStream_t st) {
  const int lanes = 16 * G;
  const int threads = lanes <= 64 ? 256 : lanes;
  const int rows_per_block = threads / lanes;
  const int64_t blocks = (M + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((rotate_quant_coalesced_kernel<DT, BITS, NI, TILED>), dim3((unsigned)blocks),
                     dim3(threads), 0, st, X, M, K, lanes, Q, S);
  return hipGetLastError();
}

template <int DT, int BITS, bool TILED>
hipError_t launch_coalesced_t(const void* X, int64_t M, int K, RqCoalesced sh, uint8_t* Q, float* S,
                              hipStream_t st) {
  switch (sh.NI) {
    case 1: return launch_coalesced_ni<DT, BITS, 1, TILED>(X, M, K, sh.G, Q, S, st);
    case 2: return launch_coalesced_ni<DT, BITS, 2, TILED>(X, M, K, sh.G, Q, S, st);
    case 3: return launch_coalesced_ni<DT, BITS, 3, TILED>(X, M, K, sh.G, Q, S, st);
    default: return launch_coalesced_ni<DT, BITS, 4, TILED>(X, M, K, sh.G, Q, S, st);
  }
}

template <int DT, int BITS>
hipError_t launch_coalesced(const void* X, int64_t M, int K, RqCoalesced sh, uint8_t* Q, float* S,
                            int tiled, hipStream_t st) {
  return tiled ? launch_coalesced_t<DT, BITS, true>(X, M, K, sh, Q, S, st)
               : launch_coalesced_t<DT, BITS, false>(X, M, K, sh, Q, S, st);
}

struct RqShape {
  int bpq;   // blocks per quad; 0 = generic kernel
  int qpr;   // quads per row
  int L;     // lanes per row slot
};

template <int DT, int BITS, int BPQ>
hipError_t launch_fast(const void* X, int64_t M, int K, RqShape sh, uint8_t* Q, float* S, int layout,
                       hipStream_t st) {
  const int threads = sh.L <= 64 ? 256 : sh.L;
  const int rows_per_block = threads / sh.L;
  const int64_t blocks = (M + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((rotate_quant_kernel<DT, BITS, BPQ>), dim3((unsigned)blocks), dim3(threads), 0,
                     st, X, M, K, sh.L, sh.qpr, Q, S, layout);
  return hipGetLastError();
}

template <int DT, int BITS>
hipError_t launch_bits(const void* X, int64_t M, int K, RqShape sh, uint8_t* Q, float* S, int layout,
                       hipStream_t st) {
  switch (sh.bpq) {
    case 1: return launch_fast<DT, BITS, 1>(X, M, K, sh, Q, S, layout, st);
    case 2: return launch_fast<DT, BITS, 2>(X, M, K, sh, Q, S, layout, st);
    case 3: return launch_fast<DT, BITS, 3>(X, M, K, sh, Q, S, layout, st);
    case 4: return launch_fast<DT, BITS, 4>(X, M, K, sh, Q, S, layout, st);
    default: {
      const int64_t blocks = (M + 3) / 4;
      hipLaunchKernelGGL((rotate_quant_generic_kernel<DT, BITS>), dim3((unsigned)blocks),
                         dim3(256), 0, st, X, M, K, Q, S, layout);
      return hipGetLastError();
    }
  }
}

// `layout`: 0 row-major, 1 tiled int codes, or the panel height (256 or 128) of FP6 tiles when
// FMT == 6 (4-bit codes stored as FP6).
template <int DT>
hipError_t launch_dt(const void* X, int64_t M, int K, int fmt, RqShape sh, uint8_t* Q, float* S,
                     int layout, hipStream_t st) {
  const RqCoalesced co = choose_coalesced(K / 128);
  if (fmt != 6 && co.G != 0) {
    return fmt == 8 ? launch_coalesced<DT, 8>(X, M, K, co, Q, S, layout, st)
                    : launch_coalesced<DT, 4>(X, M, K, co, Q, S, layout, st);
  }
  switch (fmt) {
    case 8: return launch_bits<DT, 8>(X, M, K, sh, Q, S, layout, st);
    case 4: return launch_bits<DT, 4>(X, M, K, sh, Q, S, layout, st);
    default: return launch_bits<DT, 6>(X, M, K, sh, Q, S, layout, st);
  }
}

}  // namespace

// The smallest blocks-per-quad BPQ (1..4, dividing nb) whose row fits a slot: 4*nb/BPQ lanes
// padded to a power of two <= 64, or exactly 128, 192 or 256 lanes. Others (e.g. nb = 17)
// take the generic kernel.
RqShape choose_rotate_quant_shape(int64_t K) {
  const int64_t nb = K / 128;
  for (int bpq = 1; bpq <= 4; bpq++) {
    if (nb % bpq) continue;
    const int64_t lanes = 4 * (nb / bpq);
    if (lanes <= 64) {
      int L = 4;
      while (L < lanes) L <<= 1;
      return {bpq, (int)(nb / bpq), L};
    }
    if (lanes % 64 == 0 && lanes <= 256) return {bpq, (int)(nb / bpq), (int)lanes};
  }
  return {0, 0, 64};
}

hipError_t launch_rotate_quant(const void* X, int dt, int64_t rows, int64_t K, int bits, int layout,
                               void* Q, float* S, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const RqShape sh = choose_rotate_quant_shape(K);
  uint8_t* q = static_cast<uint8_t*>(Q);
  int fmt = bits, arg = layout == kCodeTiled ? 1 : 0;
  if (layout == kCodeFp6X || layout == kCodeFp6W) {
    fmt = 6;
    arg = layout == kCodeFp6X ? 256 : 128;
  }
  switch (dt) {
    case kF32: return launch_dt<kF32>(X, rows, (int)K, fmt, sh, q, S, arg, stream);
    case kF16: return launch_dt<kF16>(X, rows, (int)K, fmt, sh, q, S, arg, stream);
    default: return launch_dt<kBF16>(X, rows, (int)K, fmt, sh, q, S, arg, stream);
  }
}

}  // namespace convrot
