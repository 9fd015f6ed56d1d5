// hbm_ceiling.hip -- memory ceilings for the rotate+quantize roofline (libconvrot_ceiling.so).
//
// Measurement support, not part of the method: kernels with exactly the memory traffic of the
// coalesced rotate+quantize kernel (rotate_quant.hip) and none of its arithmetic, so that a
// benchmark can state how close that kernel comes to what the same loads and stores reach on
// their own. Same slot geometry (16 * G lanes per row of nb = G * NI 128-element blocks, 256
// threads per workgroup or one row per workgroup of 16 * G threads), the same 16-byte
// nontemporal buffer loads of the fp16/bf16 input and the same 8-byte stores of one code byte
// per element into the row-major or tiled layout.
//   mode 0: read X, write one byte per element (the high byte of each 16-bit element): 2:1
//   mode 1: read X only (an xor of everything a lane read, stored only if it hits a sentinel)
//   mode 2: write the code bytes only
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int MODE, bool TILED>
__global__ __launch_bounds__(256) void hbm_pattern_kernel(const void* __restrict__ X, int64_t M,
                                                          int K, int S, int NI,
                                                          uint8_t* __restrict__ Q) {
  const int tid = threadIdx.x;
  const bool multi = S > 64;
  const int lg = __builtin_ctz(multi ? 64 : S);
  const int R = multi ? 1 : 256 >> lg;
  const int t = multi ? tid : (tid & (S - 1));
  const int r = multi ? 0 : tid >> lg;
  const int64_t row0 = (int64_t)blockIdx.x * R;
  const int64_t row = row0 + r;
  const int rows_here = (int)(M - row0 < R ? M - row0 : R);
  const int G = S >> 4;
  const int g = t >> 4, c = t & 15;
  u32x4 a[4] = {};
  if constexpr (MODE != 2) {
    const __amdgpu_buffer_rsrc_t xrs =
        rsrc(static_cast<const uint8_t*>(X) + row0 * K * 2, (uint32_t)(rows_here * K * 2));
    const uint32_t xoff = (uint32_t)((r * K + g * 128 + 8 * c) * 2);
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (i < NI)
        a[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff, i * G * 256, 2));
  }
  if constexpr (MODE == 1) {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) x ^= a[i][0] ^ a[i][1] ^ a[i][2] ^ a[i][3];
    if (x == 0x9E3779B9u && row < M) Q[row] = 1;
    return;
  }
  if (row >= M) return;
  const int Kb = K;
  const int kb0 = g * 128 + 8 * c;
  uint32_t qoff, qbytes;
  int qstep;
  if constexpr (TILED) {
    qbytes = 256u * (uint32_t)Kb;
    qoff = (uint32_t)(((kb0 >> 6) << 14) + ((int)(row & 255) << 6) + (kb0 & 63));
    qstep = (2 * G) << 14;
  } else {
    qbytes = (uint32_t)(rows_here * Kb);
    qoff = (uint32_t)(r * Kb + kb0);
    qstep = G * 128;
  }
  uint8_t* const qb = TILED ? Q + (row0 >> 8) * 256 * (int64_t)Kb : Q + row0 * (int64_t)Kb;
  const __amdgpu_buffer_rsrc_t qrs = rsrc(qb, qbytes);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    if (i < NI) {
      u32x2 o;
      if constexpr (MODE == 0) {
        o = u32x2{__builtin_amdgcn_perm(a[i][1], a[i][0], 0x07050301u),
                  __builtin_amdgcn_perm(a[i][3], a[i][2], 0x07050301u)};
      } else {
        o = u32x2{(uint32_t)row, (uint32_t)(kb0 + i)};
      }
      __builtin_amdgcn_raw_buffer_store_b64(o, qrs, qoff, i * qstep, 0);
    }
  }
}

template <int MODE>
hipError_t launch(const void* X, int64_t M, int K, int G, int NI, bool tiled, void* Q,
                  hipStream_t st) {
  const int lanes = 16 * G;
  const int threads = lanes <= 64 ? 256 : lanes;
  const int rpb = threads / lanes;
  const int64_t blocks = (M + rpb - 1) / rpb;
  if (tiled)
    hipLaunchKernelGGL((hbm_pattern_kernel<MODE, true>), dim3((unsigned)blocks), dim3(threads), 0, st,
                       X, M, K, lanes, NI, static_cast<uint8_t*>(Q));
  else
    hipLaunchKernelGGL((hbm_pattern_kernel<MODE, false>), dim3((unsigned)blocks), dim3(threads), 0, st,
                       X, M, K, lanes, NI, static_cast<uint8_t*>(Q));
  return hipGetLastError();
}

}  // namespace

// mode 0 / 1 / 2 as above on X [M, K] of 16-bit elements (device) and Q, the code buffer of
// M x K bytes in the row-major layout or ceil(M / 256) * 256 x K bytes in the tiled one
// (device; mode 1 writes at most one byte per row). K must be a multiple of 128 whose block
// count nb = K / 128 is G * NI with G in {1, 2, 4, 8, 12, 16} and NI <= 4. Returns 0, 1 for
// invalid arguments, or 2 for a launch error. Asynchronous on `stream`.
extern "C" int rqc_hbm_pattern(int mode, const void* X, void* Q, int64_t M, int64_t K, int tiled,
                               void* stream) {
  if (mode < 0 || mode > 2 || !X || !Q || M <= 0 || K <= 0 || K % 128 != 0 || M >= (1LL << 31))
    return 1;
  const int64_t nb = K / 128;
  int G = 0, NI = 0;
  const int gs[6] = {1, 2, 4, 8, 12, 16};
  for (int g : gs) {
    if (nb % g == 0 && nb / g <= 4) {
      G = g;
      NI = (int)(nb / g);
      break;
    }
  }
  if (G == 0) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = mode == 0 ? launch<0>(X, M, (int)K, G, NI, tiled != 0, Q, st)
               : mode == 1 ? launch<1>(X, M, (int)K, G, NI, tiled != 0, Q, st)
                           : launch<2>(X, M, (int)K, G, NI, tiled != 0, Q, st);
  return e == hipSuccess ? 0 : 2;
}
