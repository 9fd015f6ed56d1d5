// gemm_fp6.hip -- W4A4 GEMM on gfx950's FP6 matrix cores, with the dequantizing epilogue.
//
// The same product as the int8 path (acc[m, n] = sum_k Xq[m, k] * Wq[n, k] for 4-bit codes in
// [-7, 7], then Y = fp16/bf16(fma(f32(acc), fl(w_scale[n] * x_scale[m]), bias[n])); "SAM 3.1
// Multiplex INT8/INT4 ConvRot" page, "Quantization recipe" and "Downloads": INT4 matrix
// multiplication where the hardware has it). gfx950 has no int4 MFMA, but every code in
// [-7, 7] is exactly an FP6 E2M3 value (0, 1 = 2^0, 2 = 2^1, 3 = 1.5 * 2, 4 = 2^2, 5 = 1.25 * 4,
// 6 = 1.5 * 4, 7 = 1.75 * 4, and signs), every product of two codes is an integer of magnitude
// at most 49, and the fp32 accumulator stays an exact integer while |acc| <= 49 * K < 2^24 for
// every K this library accepts. So v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in FP6
// and unit scales (E8M0 127) computes acc exactly, at twice the int8 MFMA rate and 64 k per
// instruction.
//
// Operands come in the FP6 tile layout of convrot.h: per 64-element k slice, a panel of P rows
// (256 for activations, 128 for weights) is one contiguous P * 48-byte block made of two
// planes. Plane 1 holds the first 16 bytes of each lane-half's 24-byte operand string (P rows x
// 32 B), plane 2 the last 8 bytes (P rows x 16 B), each with a row-dependent swap of its two
// halves that keeps the fragment reads free of LDS bank conflicts (16-byte reads: halves swap
// on row bit 3; 8-byte reads: on row bit 4). A fragment is one ds_read_b128 from plane 1 and
// one ds_read_b64 from plane 2: six registers, exactly the MFMA's FP6 operand.
//
// Pipeline (per 64-element step, a 3-deep LDS ring filled by direct global->LDS loads two steps
// ahead: the activation tile as three 1 KB copies per wave, the weight tile as two): the four MFMAs of the wave's first token block run while the loads of step
// kt+2 issue; then the wave waits for its loads of step kt+1, passes the barrier, and reads the
// next step's fragments one by one right after the MFMA that last used each register, under the
// MFMAs of the second token block. As in the int8 kernel, launches with no more tiles than CUs
// put eight waves on each tile, in two groups that split the k steps and exchange accumulator
// halves through LDS at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.h"
#include "internal.h"

namespace convrot {
namespace {

using namespace gemm;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int kRowB = 48;                         // bytes per row per 64-element slice
constexpr int kTileX6 = kBM * kRowB;              // 12 KB
constexpr int kTileW6 = kBN * kRowB;              // 6 KB
constexpr int kStage6 = kTileX6 + kTileW6;        // 18 KB
constexpr int kStages6 = 3;
constexpr int kThreads6 = 256;
constexpr int kLoads6 = 5;                        // per wave per step: 3 + 2 copies of 1 KB
static_assert(kLoads6 == 5, "the vmcnt(5) waits below count five loads per step");
constexpr int kFmtFp6 = 2;                        // MFMA operand format code: FP6 E2M3
constexpr int kUnitScale = 127;                   // E8M0 exponent of 2^0

template <int SPLIT>
constexpr int lds_bytes6() {
  // The ring, or the epilogue's staging / the accumulator exchange when larger (both reuse the
  // ring after the k loop), then the parked scales.
  constexpr int ring = kStages6 * SPLIT * kStage6;
  constexpr int after = SPLIT == 1 ? 4 * 64 * 256 : 8 * 64 * 64 * 4;
  return (ring > after ? ring : after) + (2 * kBN + kBM) * 4;
}

// Fragment of a 32-row block: rows row .. row+31 of a P-row tile (lane l takes row + l % 32,
// operand half l / 32).
// The empty asm hides how the 8-byte reads of different fragments relate, so the compiler keeps
// one ds_read_b64 per fragment, loading straight into the operand's last two registers (two
// merged 64-bit reads land in other registers and cost moves plus a wait before the MFMA).
// Plain vector loads (not HIP's uint4 / uint2 structs) keep the compiler's LDS-DMA wait logic
// from treating them as possibly aliasing the ring stages being filled, which would force a
// full vmcnt(0) drain before every read.
template <int P>
__device__ __forceinline__ v8i read_frag6(const uint8_t* tile, int row, int half) {
  const v4i a = *reinterpret_cast<const v4i*>(tile + row * 32 + 16 * (half ^ ((row >> 3) & 1)));
  int off2 = P * 32 + row * 16 + 8 * (half ^ ((row >> 4) & 1));
  asm volatile("" : "+v"(off2));
  const v2i b = *reinterpret_cast<const v2i*>(tile + off2);
  v8i f;
  f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
  f[4] = b[0]; f[5] = b[1]; f[6] = 0; f[7] = 0;
  return f;
}

template <int OUT, int SPLIT>
__global__ __launch_bounds__(kThreads6 * SPLIT, 2 / SPLIT) void gemm_fp6_kernel(
    const uint8_t* __restrict__ Xt, const float* __restrict__ sx, const uint8_t* __restrict__ Wt,
    const float* __restrict__ sw, const float* __restrict__ bias, void* __restrict__ Y, int M,
    int N, int K, int tiles_m, int tiles_n, int act) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[lds_bytes6<SPLIT>()];
  constexpr int kSlot = SPLIT * kStage6;                 // one ring stage, all groups
  constexpr int kScales = lds_bytes6<SPLIT>() - (2 * kBN + kBM) * 4;

  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + 7) >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= ntiles) return;
  const int tm = logical / tiles_n;
  const int tn = logical - tm * tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = wave_all & 3;
  const int grp = wave_all >> 2;

  float my_sw = 0.0f, my_b = 0.0f, my_sx = 0.0f;
  if constexpr (OUT != kOutS32) {
    const int n = n0 + (int)threadIdx.x, m = m0 + (int)threadIdx.x;
    if (threadIdx.x < kBN && n < N) {
      my_sw = sw[n];
      my_b = bias ? bias[n] : 0.0f;
    }
    if (threadIdx.x < kBM && m < M) my_sx = sx[m];
  }

  v16f acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; a++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[a][b][r] = 0.0f;

  const int nsl = K >> 6;                                // 64-element slices in K
  uint8_t* const ring = lds + grp * kStage6;
  const uint8_t* const xsrc = Xt + (int64_t)tm * nsl * kTileX6;
  const uint8_t* const wsrc = Wt + (int64_t)tn * nsl * kTileW6;
  // Step j of this group is slice SPLIT * j + grp: its activation tile (12 KB) as 12 copies of
  // 1 KB, three per wave, and its weight tile (6 KB) as 6 copies of 1 KB, two per wave: wave w
  // copies chunks w and (w + 4) % 6, so chunks 0 and 1 are copied twice with identical bytes
  // (every wave then issues the same five loads; 12-byte direct loads would leave 4-byte gaps
  // in LDS, one per lane).
  auto issue = [&](int stage, int j) {
    const int s = SPLIT * j + grp;
    uint8_t* tX = ring + stage * kSlot;
    uint8_t* tW = tX + kTileX6;
    const uint8_t* gx = xsrc + (int64_t)s * kTileX6;
    const uint8_t* gw = wsrc + (int64_t)s * kTileW6;
#pragma unroll
    for (int i = 0; i < 3; i++) {
      const int c = wave * 3 + i;
      __builtin_amdgcn_global_load_lds((const void*)(gx + c * 1024 + lane * 16), (lds_void*)(tX + c * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int c = i == 0 ? wave : (wave + 4) % 6;
      __builtin_amdgcn_global_load_lds((const void*)(gw + c * 1024 + lane * 16), (lds_void*)(tW + c * 1024), 16, 0, 0);
    }
  };

  const int rsub = lane & 31, fhalf = lane >> 5;
  v8i wf[4], xf[2];
  auto read_w = [&](int stage, int a) {
    return read_frag6<kBN>(ring + stage * kSlot + kTileX6, a * 32 + rsub, fhalf);
  };
  auto read_x = [&](int stage, int b) {
    return read_frag6<kBM>(ring + stage * kSlot, wave * 64 + b * 32 + rsub, fhalf);
  };
  auto mfma = [&](int a, int b) {
    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[a], xf[b], acc[a][b], kFmtFp6, kFmtFp6, 0,
                                                                 kUnitScale, 0, kUnitScale);
  };

  // Why the ring is race free: the loads issued at the start of step kt fill stage
  // (kt+2) % 3 = (kt-1) % 3. Every wave read its last fragments of that stage (step kt-1's)
  // during step kt-2 and waited for those reads (lgkmcnt(0)) before the barrier of step kt-1,
  // which the loads follow. The reads of stage (kt+1) % 3 follow the barrier of step kt, which
  // every wave passes only after its own loads of step kt+1 have landed.
  auto body = [&](auto load_tag, auto mid_tag, int kt) {
    constexpr bool LOAD = decltype(load_tag)::value;
    constexpr bool MID = decltype(mid_tag)::value;
    if constexpr (LOAD) issue((kt + 2) % kStages6, kt + 2);
#pragma unroll
    for (int a = 0; a < 4; a++) mfma(a, 0);
    if constexpr (LOAD) {
#pragma unroll
      for (int i = 0; i < kLoads6; i++) {
        if (i < 4) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);              // VMEM (global -> LDS)
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MID) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if constexpr (LOAD) {
        asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const int nxt = (kt + 1) % kStages6;
      xf[0] = read_x(nxt, 0);
#pragma unroll
      for (int a = 0; a < 4; a++) {
        mfma(a, 1);
        wf[a] = read_w(nxt, a);
      }
      xf[1] = read_x(nxt, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // DS read: next xf[0]
#pragma unroll
      for (int a = 0; a < 4; a++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA (a, 1)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);      // DS read: next wf[a]
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // DS read: next xf[1]
    } else {
#pragma unroll
      for (int a = 0; a < 4; a++) mfma(a, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nk = nsl / SPLIT;                 // steps per group (the launcher checks divisibility)
  issue(0, 0);
  if (nk > 1) {
    issue(1, 1);
    asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  if constexpr (OUT != kOutS32) {
    float* e_sw = reinterpret_cast<float*>(lds + kScales);
    if (threadIdx.x < kBN) {
      e_sw[threadIdx.x] = my_sw;
      e_sw[kBN + threadIdx.x] = my_b;
    }
    if (threadIdx.x < kBM) e_sw[2 * kBN + threadIdx.x] = my_sx;
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  xf[0] = read_x(0, 0);
  xf[1] = read_x(0, 1);
#pragma unroll
  for (int a = 0; a < 4; a++) wf[a] = read_w(0, a);
  int kt = 0;
  for (; kt + 2 < nk; kt++) body(std::true_type{}, std::true_type{}, kt);
  if (kt + 1 < nk) body(std::false_type{}, std::true_type{}, kt++);
  body(std::false_type{}, std::false_type{}, kt);
  __syncthreads();

  const float* scales = reinterpret_cast<const float*>(lds + kScales);
  if constexpr (SPLIT == 1) {
    tile_epilogue_act<4, OUT, 2>(act, acc, scales, lds + wave * (64 * 256), wave * 64, lane, m0, n0, M, N, Y);
  } else {
    // Group g finishes row block b = g: it sends its partial sums of block 1 - g to the partner
    // wave (wave_all ^ 4) and adds the partner's partials of block g (exact: integers < 2^24).
    // Exchange layout: [wave_all][a][r4][lane] of 16-byte float4.
    float4* xch = reinterpret_cast<float4*>(lds);
    auto slot = [&](int w, int a, int r4) { return xch + ((w * 4 + a) * 4 + r4) * 64 + lane; };
    auto finish = [&](auto keep_tag) {
      constexpr int KB = decltype(keep_tag)::value;
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++)
          *slot(wave_all, a, r4) = make_float4(acc[a][1 - KB][4 * r4], acc[a][1 - KB][4 * r4 + 1],
                                               acc[a][1 - KB][4 * r4 + 2], acc[a][1 - KB][4 * r4 + 3]);
      __syncthreads();
      v16f keep[4][1];
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
          const float4 o = *slot(wave_all ^ 4, a, r4);
          keep[a][0][4 * r4] = acc[a][KB][4 * r4] + o.x;
          keep[a][0][4 * r4 + 1] = acc[a][KB][4 * r4 + 1] + o.y;
          keep[a][0][4 * r4 + 2] = acc[a][KB][4 * r4 + 2] + o.z;
          keep[a][0][4 * r4 + 3] = acc[a][KB][4 * r4 + 3] + o.w;
        }
      __syncthreads();   // every exchange read is done before the staging below reuses LDS
      tile_epilogue_act<4, OUT, 1>(act, keep, scales, lds + wave_all * (32 * 256), wave * 64 + KB * 32, lane,
                               m0, n0, M, N, Y);
    };
    if (grp == 0) {
      finish(std::integral_constant<int, 0>{});
    } else {
      finish(std::integral_constant<int, 1>{});
    }
  }
}

template <int OUT>
hipError_t launch6(const void* Xt, const float* sx, const void* Wt, const float* sw,
                   const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int act, hipStream_t st) {
  const int tiles_m = (int)((M + kBM - 1) / kBM);
  const int tiles_n = (int)((N + kBN - 1) / kBN);
  const int ntiles = tiles_m * tiles_n;
  const int grid = ((ntiles + 7) / 8) * 8;
  const int64_t nsl = K / 64;
  if (ntiles <= kNumCUs && nsl % 2 == 0 && nsl >= 16) {
    hipLaunchKernelGGL((gemm_fp6_kernel<OUT, 2>), dim3(grid), dim3(2 * kThreads6), 0, st,
                       static_cast<const uint8_t*>(Xt), sx, static_cast<const uint8_t*>(Wt), sw,
                       bias, Y, (int)M, (int)N, (int)K, tiles_m, tiles_n, act);
  } else {
    hipLaunchKernelGGL((gemm_fp6_kernel<OUT, 1>), dim3(grid), dim3(kThreads6), 0, st,
                       static_cast<const uint8_t*>(Xt), sx, static_cast<const uint8_t*>(Wt), sw,
                       bias, Y, (int)M, (int)N, (int)K, tiles_m, tiles_n, act);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp6(const void* Xt, const float* sx, const void* Wt, const float* sw,
                           const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                           int out_dt, int32_t* acc32, int act, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (acc32) return launch6<kOutS32>(Xt, sx, Wt, sw, bias, M, N, K, acc32, kActNone, stream);
  if (out_dt == kF16) return launch6<kOutF16>(Xt, sx, Wt, sw, bias, M, N, K, Y, act, stream);
  return launch6<kOutBF16>(Xt, sx, Wt, sw, bias, M, N, K, Y, act, stream);
}

}  // namespace convrot
