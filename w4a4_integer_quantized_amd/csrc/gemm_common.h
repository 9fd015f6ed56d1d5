// gemm_common.h -- pieces shared by the GEMM kernels (int8 MFMA and FP6 MFMA paths): tile
// shape, output kinds, the two-rounding fp16/bf16 pack and the dequantizing tile epilogue.
// Device code only; each translation unit gets its own copy (everything is inline).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {
namespace gemm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 256;                       // tokens per tile
constexpr int kBN = 128;                       // output features per tile
constexpr int kNumCUs = 256;                   // MI355X

enum OutKind { kOutS32 = 0, kOutF16 = 1, kOutBF16 = 2 };

typedef __attribute__((address_space(3))) void lds_void;

// The epilogue rounds twice by definition: fma -> binary32, then binary32 -> fp16/bf16. The
// empty asm pins each value as a binary32 register so the compiler cannot fuse the conversion
// into the fma (v_fma_mix* rounds once, straight to fp16, which differs on rare ties).
// gfx950 converts a pair with one v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint32_t pack2(float a, float b, int out) {
  asm volatile("" : "+v"(a), "+v"(b));
  const f32x2 v = {a, b};
  if (out == kOutF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// The MLP activation applied to the binary32 pre-activation v before the fp16/bf16 rounding
// (act 0: none; 1: GELU, erf form; 2: GELU, tanh form), with the native v_exp_f32 (2^x) and
// v_rcp_f32 (1/x), each within about 1 ulp, so that the epilogue's extra VALU work stays small:
//  * erf form: x Phi(x) = 0.5 x erfc(-x / sqrt 2), erfc by the Chebyshev-fitted form of Press et
//    al., Numerical Recipes, section 6.2 ("erfcc"): for z = |y|, t = 1 / (1 + z/2),
//    erfc(z) = t exp(-z^2 + P(t)) with a degree-9 polynomial P (fractional error below 1.2e-7),
//    and erfc(-z) = 2 - erfc(z).
//  * tanh form: 0.5 x (1 + tanh u) = x logistic(2u), u = sqrt(2/pi) (x + 0.044715 x^3), the
//    logistic taken as 1 / (1 + e) or e / (1 + e) with e = exp(-2|u|) <= 1, which never
//    overflows.
// Neither form cancels for negative x, so the relative error is a few binary32 ulps plus the
// rounding of the exponent's argument, amplified as the tail steepens (about z^2 and 2|u|
// ulps); the rounded output can differ from the correctly rounded one only next to a rounding
// midpoint. Results below the binary32 normal range may come out as zero.
enum ActKind { kActNone = 0, kActGeluErf = 1, kActGeluTanh = 2 };

template <int ACT>
__device__ __forceinline__ float activate(float v) {
  constexpr float kLog2e = 1.44269504088896341f;
  if constexpr (ACT == kActGeluErf) {
    const float z = fabsf(v) * 0.707106781186547524f;          // |y|, y = -v / sqrt 2
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, z, 1.0f));
    float p = 0.17087277f;
    p = __builtin_fmaf(p, t, -0.82215223f);
    p = __builtin_fmaf(p, t, 1.48851587f);
    p = __builtin_fmaf(p, t, -1.13520398f);
    p = __builtin_fmaf(p, t, 0.27886807f);
    p = __builtin_fmaf(p, t, -0.18628806f);
    p = __builtin_fmaf(p, t, 0.09678418f);
    p = __builtin_fmaf(p, t, 0.37409196f);
    p = __builtin_fmaf(p, t, 1.00002368f);
    p = __builtin_fmaf(p, t, -1.26551223f);
    // 2^32 * exp(-z^2 + P): scaled so that no intermediate leaves the binary32 normal range
    // while the result is inside it (the native exp2 flushes subnormal results).
    const float e32 = __builtin_amdgcn_exp2f(__builtin_fmaf(__builtin_fmaf(-z, z, p), kLog2e, 32.0f));
    if (v <= 0.0f) return (0.5f * 0x1p-32f * v * t) * e32;           // 0.5 v erfc(|y|)
    return (0.5f * v) * (2.0f - t * (0x1p-32f * e32));                // 0.5 v (2 - erfc(|y|))
  } else if constexpr (ACT == kActGeluTanh) {
    const float m = v * __builtin_fmaf(0.044715f, v * v, 1.0f);       // v + 0.044715 v^3
    // e = exp(-2|u|) = 2^(-2 sqrt(2/pi) log2(e) |m|), computed as 2^32 e (see above)
    const float e32 = __builtin_amdgcn_exp2f(__builtin_fmaf(-2.30220819814432500f, fabsf(m), 32.0f));
    const float r = __builtin_amdgcn_rcpf(__builtin_fmaf(0x1p-32f, e32, 1.0f));
    if (m >= 0.0f) return v * r;
    return ((0x1p-32f * v) * e32) * r;
  } else {
    return v;
  }
}

// The tile's epilogue for NB consecutive 32-row blocks of this wave: acc[a][b] holds the
// 32 x 32 accumulator block of W rows a*32.. and tile rows row0 + b*32... Lane l holds
// D[n][m] for m = b*32 + l%32 and n = a*32 + 8*(r/4) + 4*(l/32) + r%4, r = 0..15. Either raw
// int32 accumulators (OUT == kOutS32) or the dequantizing epilogue through `stage`, this wave's
// LDS staging block of 32*NB rows x 256 B. `scales` holds the tile's w_scale [128], bias [128]
// and x_scale [256], parked in LDS before the k loop.
// Accumulator element r of a block as the int32 the epilogue consumes: int MFMA blocks hold
// 256 * acc for 4-bit codes on the int8 path (undone by an exact shift); float MFMA blocks (the
// FP6 path) hold acc itself, an integer below 2^24 in magnitude and therefore exact.
template <int BITS>
__device__ __forceinline__ int acc_int(const v16i& blk, int r) { return BITS == 4 ? (blk[r] >> 8) : blk[r]; }
template <int BITS>
__device__ __forceinline__ int acc_int(const v16f& blk, int r) { return static_cast<int>(blk[r]); }
template <int BITS>
__device__ __forceinline__ float acc_float(const v16i& blk, int r) { return static_cast<float>(acc_int<BITS>(blk, r)); }
template <int BITS>
__device__ __forceinline__ float acc_float(const v16f& blk, int r) { return blk[r]; }

template <int BITS, int OUT, int NB, int ACT, typename AccBlk>
__device__ __forceinline__ void tile_epilogue(AccBlk (&acc)[4][NB], const float* scales, uint8_t* stage,
                                              int row0, int lane, int m0, int n0, int M, int N,
                                              void* __restrict__ Y) {
  const int msub = lane & 31, half = lane >> 5;
  if constexpr (OUT == kOutS32) {
#pragma unroll
    for (int b = 0; b < NB; b++) {
      const int m = m0 + row0 + b * 32 + msub;
      if (m >= M) continue;
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const int n = n0 + a * 32 + 8 * g + 4 * half;
          if (n >= N) continue;
          int v[4];
#pragma unroll
          for (int e = 0; e < 4; e++) v[e] = acc_int<BITS>(acc[a][b], 4 * g + e);
          *reinterpret_cast<int4*>(static_cast<int32_t*>(Y) + (int64_t)m * N + n) = make_int4(v[0], v[1], v[2], v[3]);
        }
    }
  } else {
    const float* e_sw = scales;
    const float* e_b = e_sw + kBN;
    const float* e_sx = e_b + kBN;
    float xs[NB];
#pragma unroll
    for (int b = 0; b < NB; b++) xs[b] = e_sx[row0 + b * 32 + msub];
#pragma unroll
    for (int a = 0; a < 4; a++) {
      float4 s4[4], b4[4];
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int col = a * 32 + 8 * g + 4 * half;
        s4[g] = *reinterpret_cast<const float4*>(e_sw + col);
        b4[g] = *reinterpret_cast<const float4*>(e_b + col);
      }
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int col = a * 32 + 8 * g + 4 * half;   // tile-local output column
        const float ws[4] = {s4[g].x, s4[g].y, s4[g].z, s4[g].w};
        const float bs[4] = {b4[g].x, b4[g].y, b4[g].z, b4[g].w};
#pragma unroll
        for (int b = 0; b < NB; b++) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            y[e] = activate<ACT>(
                __builtin_fmaf(acc_float<BITS>(acc[a][b], 4 * g + e), __fmul_rn(ws[e], xs[b]), bs[e]));
          }
          uint2 o;
          o.x = pack2(y[0], y[1], OUT);
          o.y = pack2(y[2], y[3], OUT);
          const int row = b * 32 + msub;
          const int chunk = (col >> 3) ^ (row & 15);
          // Rows r and r + 16 share a chunk position; their 8-byte halves are swapped so the
          // 32 lanes of a write hit distinct banks (undone when the row is read back).
          const int hpos = half ^ ((row >> 4) & 1);
          *reinterpret_cast<uint2*>(stage + row * 256 + chunk * 16 + hpos * 8) = o;
        }
      }
    }
    // Read back whole rows (16 lanes x 16 B = one 256-byte row segment, 4 rows per read), all
    // reads first, then the streaming stores. A wave's LDS operations complete in order, so the
    // reads see its own writes above.
    constexpr int kIt = 8 * NB;
    uint4 v[kIt];
#pragma unroll
    for (int it = 0; it < kIt; it++) {
      const int row = it * 4 + (lane >> 4);
      v[it] = *reinterpret_cast<const uint4*>(stage + row * 256 + (lane & 15) * 16);
      // Rows with bit 4 set hold their 8-byte halves swapped (see the writes); bit 4 of row is
      // (it >> 2) & 1 for every lane, so this is a compile-time register swap.
      if ((it >> 2) & 1) v[it] = make_uint4(v[it].z, v[it].w, v[it].x, v[it].y);
    }
#pragma unroll
    for (int it = 0; it < kIt; it++) {
      const int row = it * 4 + (lane >> 4);
      const int m = m0 + row0 + row;
      const int n = n0 + 8 * ((lane & 15) ^ (row & 15));
      if (m < M && n < N) {
        // Streaming store: Y is written once and not re-read here, so it should not evict
        // the Wq / Xq panels that neighbouring tiles re-read from L2. An activated output is
        // the next linear's input, read right away: it is stored normally, so that it can
        // still be in the Infinity Cache when the next rotate + quantize reads it.
        v4i* dst = reinterpret_cast<v4i*>(static_cast<uint16_t*>(Y) + (int64_t)m * N + n);
        if constexpr (ACT == kActNone) {
          __builtin_nontemporal_store(__builtin_bit_cast(v4i, v[it]), dst);
        } else {
          *dst = __builtin_bit_cast(v4i, v[it]);
        }
      }
    }
  }
}

// tile_epilogue with the launch's activation: one uniform branch per tile, so the variant
// without an activation carries no activation code.
template <int BITS, int OUT, int NB, typename AccBlk>
__device__ __forceinline__ void tile_epilogue_act(int act, AccBlk (&acc)[4][NB], const float* scales,
                                                  uint8_t* stage, int row0, int lane, int m0, int n0,
                                                  int M, int N, void* __restrict__ Y) {
  if constexpr (OUT == kOutS32) {
    tile_epilogue<BITS, OUT, NB, kActNone>(acc, scales, stage, row0, lane, m0, n0, M, N, Y);
  } else {
    if (act == kActNone) {
      tile_epilogue<BITS, OUT, NB, kActNone>(acc, scales, stage, row0, lane, m0, n0, M, N, Y);
    } else if (act == kActGeluErf) {
      tile_epilogue<BITS, OUT, NB, kActGeluErf>(acc, scales, stage, row0, lane, m0, n0, M, N, Y);
    } else {
      tile_epilogue<BITS, OUT, NB, kActGeluTanh>(acc, scales, stage, row0, lane, m0, n0, M, N, Y);
    }
  }
}

}  // namespace gemm
}  // namespace convrot
