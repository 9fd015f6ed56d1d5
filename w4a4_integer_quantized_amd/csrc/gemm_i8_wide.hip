// gemm_i8_wide.hip -- the int8 MFMA GEMM on 256 x 256 tiles (launch_gemm picks it for long K).
//
// Computes acc[m, n] = sum_k Xq[m, k] * Wq[n, k] (both operands K-contiguous) and then
// Y[m, n] = fp16/bf16( fma(f32(acc), fl(w_scale[n] * x_scale[m]), bias[n]) ) -- the W8A8 /
// W4A4 operations of the "SAM 3.1 Multiplex INT8/INT4 ConvRot" release page ("Quantization
// recipe") with the per-row weight scale and per-token activation scale. INT4 codes are
// multiplied on the INT8 matrix cores, the fallback the same page describes ("Downloads");
// gfx950 has no int4 MFMA.
//
// Design (gfx950: 256 CUs in 8 XCDs, 160 KB LDS and 4 SIMDs per CU, 64-wide waves):
//   * One 256-thread workgroup per CU owns a 256 (tokens) x 256 (outputs) tile. Its 4 waves
//     (one per SIMD, up to 512 VGPR+AGPR each) form a 2 x 2 grid; each owns a 128 x 128
//     block as 4 x 4 tiles of v_mfma_i32_32x32x32_i8 (256 int32 accumulators per lane). A
//     wave reads 8 fragments per 16 MFMAs, and the tile needs 512 operand rows per 64K
//     outputs, which keeps both the LDS and the L2 -> LDS traffic per MFMA low.
//   * K is staged 128 bytes per step (128 int8 or 256 int4 codes) through two LDS stages of
//     (256 + 256) rows x 128 B, filled by direct global->LDS 16-byte loads that cover whole
//     128-byte row segments. The 16-byte chunk c of row r sits at c ^ swz(r), which keeps the
//     MFMA fragment reads (ds_read_b128, 32 rows x 2 chunks per wave) bank-conflict free.
//   * Per k step (4 slices of 32 bytes): the fragments of slice s+1 are read under the MFMAs
//     of slice s; before the last slice each wave waits for its loads of the next step, all
//     waves meet at a barrier, the loads of the step after next go into the stage just
//     drained, and slice 0 of the next step is read under the last MFMAs.
//   * The MFMA "A" operand is a Wq row block and "B" an Xq row block, so each lane ends with
//     4 consecutive output columns of one token. The epilogue converts them and parks each
//     wave's 128 x 128 output block in the (now free) stages, 16-byte chunks XOR-swizzled by
//     row, then writes it back as whole 256-byte row segments with 16-byte stores. w_scale,
//     bias and x_scale for the tile are loaded at kernel start and read from LDS.
//   * INT4: a 16-byte chunk of packed codes (32 nibbles) becomes two MFMA operands,
//     (w << 4) & 0xF0F0F0F0 (even k) and w & 0xF0F0F0F0 (odd k): each byte is 16 * code,
//     exact for codes in [-8, 7]. Both operands get the same k permutation, so the sum is
//     unchanged; the accumulator is 256 * acc and an exact arithmetic shift by 8 recovers it.
//   * Workgroups are dispatched round-robin over the 8 XCDs; each XCD owns a contiguous range
//     of Xq row panels and sweeps them in groups (token panel fastest, output panel slowest),
//     so its 4 MB L2 holds the group's Xq panels and the current Wq panel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 256;                       // tokens per tile
constexpr int kBN = 256;                       // output features per tile
constexpr int kBKB = 128;                      // K bytes per step
constexpr int kThreads = 256;
constexpr int kTileX = kBM * kBKB;             // 32 KB
constexpr int kStageBytes = (kBM + kBN) * kBKB;   // 64 KB
constexpr int kScaleOff = 2 * kStageBytes;        // 128 KB
constexpr int kLdsBytes = kScaleOff + (2 * kBN + kBM) * 4;
constexpr int kLoadsPerStep = kStageBytes / 1024 / 4;   // wave-wide 1 KB copies per wave: 16
constexpr int kGroupM = 4;                     // Xq row panels swept together per XCD

enum OutKind { kOutS32 = 0, kOutF16 = 1, kOutBF16 = 2 };

// Depends on r mod 32 only, so every 32-row fragment block of a wave shares one per-lane
// pattern (the block offsets become immediates).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 3); }

typedef __attribute__((address_space(3))) void lds_void;

// One wave copies 8 rows x 128 B (1 KB) of a K-contiguous operand into LDS rows
// [row0, row0 + 8) of a tile. Lane l fills LDS position (row0 + l/8, chunk l%8), which holds
// global chunk (l%8) ^ swz(row). Rows past the end of the operand re-read its last row (their
// results are never stored). `tile` is the operand's first row of this tile (wave-uniform) and
// `off` the lane's byte offset from it at k = 0: the row (clamped to the operand) times the row
// length, plus 16 * chunk.
__device__ __forceinline__ uint32_t copy_offset(int row0, int lane, int rows_left, int ld) {
  const int r = row0 + (lane >> 3);
  const int c = (lane & 7) ^ swz(r);
  const int rr = r < rows_left ? r : rows_left - 1;
  return (uint32_t)rr * (uint32_t)ld + 16u * (uint32_t)c;
}

__device__ __forceinline__ void copy_rows(const uint8_t* tile, uint32_t off, int row0,
                                          uint8_t* lds_tile) {
  __builtin_amdgcn_global_load_lds((const void*)(tile + off), (lds_void*)(lds_tile + row0 * kBKB), 16, 0, 0);
}

__device__ __forceinline__ v4i read_frag(const uint8_t* lds_tile, int row, int chunk) {
  return *reinterpret_cast<const v4i*>(lds_tile + row * kBKB + ((chunk ^ swz(row)) << 4));
}

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

template <int BITS, int OUT>
__global__ __launch_bounds__(kThreads, 1) void gemm_wide_kernel(
    const uint8_t* __restrict__ Xq, const float* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const float* __restrict__ sw, const float* __restrict__ bias, void* __restrict__ Y, int M,
    int N, int Kb, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];

  // Workgroups are dispatched round-robin over the 8 XCDs, so XCD x runs blockIdx % 8 == x.
  // XCD x owns the Xq row panels [x*P, x*P + P) and sweeps them in groups of kGroupM panels:
  // for each Wq panel (output tile column), all panels of the group, token panel fastest.
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int P = (tiles_m + 7) >> 3;
  const int tm_begin = xcd * P;
  const int tm_count = min(P, tiles_m - tm_begin);
  if (tm_count <= 0 || local >= tm_count * tiles_n) return;
  const int group = local / (kGroupM * tiles_n);
  const int r_in = local - group * kGroupM * tiles_n;
  const int g_eff = min(kGroupM, tm_count - group * kGroupM);
  const int tn = r_in / g_eff;
  const int tm = tm_begin + group * kGroupM + (r_in - tn * g_eff);
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;     // this wave: tokens wm*128.., outputs wn*128..

  // Per-tile epilogue operands, fetched now so their latency hides behind the k loop.
  float my_sw = 0.0f, my_b = 0.0f, my_sx = 0.0f;
  if constexpr (OUT != kOutS32) {
    const int n = n0 + (int)threadIdx.x, m = m0 + (int)threadIdx.x;
    if (n < N) {
      my_sw = sw[n];
      my_b = bias ? bias[n] : 0.0f;
    }
    if (m < M) my_sx = sx[m];
  }

  v16i acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; a++)
#pragma unroll
    for (int b = 0; b < 4; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[a][b][r] = 0;

  // Stage s holds the Xq tile (256 rows) then the Wq tile (256 rows), 128 B per row; each of
  // the 4 waves copies 64 Xq rows and 64 Wq rows. Byte offsets within a tile fit 32 bits
  // (256 rows x at most 64 KB per row).
  const uint8_t* xtile = Xq + (int64_t)m0 * Kb;
  const uint8_t* wtile = Wq + (int64_t)n0 * Kb;
  uint32_t xoff[8], woff[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    xoff[i] = copy_offset((wave * 8 + i) * 8, lane, M - m0, Kb);
    woff[i] = copy_offset((wave * 8 + i) * 8, lane, N - n0, Kb);
  }
  auto issue = [&](int stage, int k0) {
    uint8_t* tX = lds + stage * kStageBytes;
    uint8_t* tW = tX + kTileX;
#pragma unroll
    for (int i = 0; i < 8; i++) copy_rows(xtile + k0, xoff[i], (wave * 8 + i) * 8, tX);
#pragma unroll
    for (int i = 0; i < 8; i++) copy_rows(wtile + k0, woff[i], (wave * 8 + i) * 8, tW);
  };

  // Fragments of one 32-byte k slice: this wave's 4 Wq row blocks and 4 Xq row blocks.
  const int rsub = lane & 31, fhalf = lane >> 5;
  auto read_frags = [&](int stage, int ks, v4i (&wf)[4], v4i (&xf)[4]) {
    const uint8_t* tX = lds + stage * kStageBytes;
    const uint8_t* tW = tX + kTileX;
    const int chunk = 2 * ks + fhalf;
#pragma unroll
    for (int a = 0; a < 4; a++) wf[a] = read_frag(tW, wn * 128 + a * 32 + rsub, chunk);
#pragma unroll
    for (int b = 0; b < 4; b++) xf[b] = read_frag(tX, wm * 128 + b * 32 + rsub, chunk);
  };
  auto mfma_slice = [&](const v4i (&wf)[4], const v4i (&xf)[4]) {
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
          xlo[a][e] = (xf[a][e] << 4) & 0xF0F0F0F0;
          xhi[a][e] = xf[a][e] & 0xF0F0F0F0;
        }
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++) {
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wlo[a], xlo[b], acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(whi[a], xhi[b], acc[a][b], 0, 0, 0);
        }
    }
  };
  constexpr int kMfmaPerSlice = BITS == 8 ? 16 : 32;
  // MFMAs of one slice with the 8 fragment reads of the next slice interleaved.
  auto slice_with_reads = [&](const v4i (&wf)[4], const v4i (&xf)[4], int rstage, int rks,
                              v4i (&nwf)[4], v4i (&nxf)[4]) {
    read_frags(rstage, rks, nwf, nxf);
    mfma_slice(wf, xf);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerSlice - 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // The same with the loads of a k step interleaved as well (16 VMEM per wave).
  auto slice_with_reads_loads = [&](const v4i (&wf)[4], const v4i (&xf)[4], int rstage, int rks,
                                    v4i (&nwf)[4], v4i (&nxf)[4], int lstage, int lk0) {
    read_frags(rstage, rks, nwf, nxf);
    issue(lstage, lk0);
    mfma_slice(wf, xf);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // DS read
      __builtin_amdgcn_sched_group_barrier(0x020, kLoadsPerStep / 8, 0);   // VMEM (global -> LDS)
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerSlice - 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // k step kt from stage kt & 1 (fragments of its slice 0 already in registers). Slices 0..2
  // each read the next slice; then -- if there is a next step -- the wave waits for its own
  // loads of that step (nothing else is in flight) and for its fragment reads, passes the
  // barrier (after which every wave has finished reading this stage and the next stage has
  // landed), and reads slice 0 of step kt+1 under the MFMAs of slice 3 while issuing the loads
  // of step kt+2 into this stage when LOAD.
  auto kstep = [&](auto next_tag, auto load_tag, int kt, v4i (&wa)[4], v4i (&xa)[4]) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr bool LOAD = decltype(load_tag)::value;
    const int cur = kt & 1;
    v4i wb[4], xb[4];
    slice_with_reads(wa, xa, cur, 1, wb, xb);
    slice_with_reads(wb, xb, cur, 2, wa, xa);
    slice_with_reads(wa, xa, cur, 3, wb, xb);
    if constexpr (NEXT) {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (LOAD) {
        slice_with_reads_loads(wb, xb, cur ^ 1, 0, wa, xa, cur, (kt + 2) * kBKB);
      } else {
        slice_with_reads(wb, xb, cur ^ 1, 0, wa, xa);
      }
    } else {
      mfma_slice(wb, xb);
    }
  };

  // nk >= 2 (the launcher sends shorter K elsewhere): steps 0 .. nk-3 load two steps ahead,
  // step nk-2 has a successor but nothing left to load, step nk-1 is the last.
  const int nk = Kb / kBKB;
  issue(0, 0);
  issue(1, kBKB);
  // Stage 0 (and the epilogue operands, requested first) must land; stage 1 may stay in flight.
  asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  if constexpr (OUT != kOutS32) {
    float* e_sw = reinterpret_cast<float*>(lds + kScaleOff);
    e_sw[threadIdx.x] = my_sw;
    e_sw[kBN + threadIdx.x] = my_b;
    e_sw[2 * kBN + threadIdx.x] = my_sx;
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  v4i wa[4], xa[4];
  read_frags(0, 0, wa, xa);
  for (int kt = 0; kt < nk - 2; kt++) kstep(std::true_type{}, std::true_type{}, kt, wa, xa);
  kstep(std::true_type{}, std::false_type{}, nk - 2, wa, xa);
  kstep(std::false_type{}, std::false_type{}, nk - 1, wa, xa);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);

  // Epilogue. Lane l of block (a, b) holds D[n][m] for m = b*32 + l%32 and
  // n = a*32 + 8*(r/4) + 4*(l/32) + r%4, r = 0..15 (wave-local indices: tokens wm*128 + m,
  // outputs wn*128 + n of the tile).
  const int msub = lane & 31, half = lane >> 5;
  if constexpr (OUT == kOutS32) {
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int m = m0 + wm * 128 + b * 32 + msub;
      if (m >= M) continue;
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const int n = n0 + wn * 128 + a * 32 + 8 * g + 4 * half;
          if (n >= N) continue;
          int v[4];
#pragma unroll
          for (int e = 0; e < 4; e++) v[e] = (BITS == 4) ? (acc[a][b][4 * g + e] >> 8) : acc[a][b][4 * g + e];
          *reinterpret_cast<int4*>(static_cast<int32_t*>(Y) + (int64_t)m * N + n) = make_int4(v[0], v[1], v[2], v[3]);
        }
    }
  } else {
    // The stages are free now; the scales were parked at kScaleOff before the k loop.
    const float* e_sw = reinterpret_cast<const float*>(lds + kScaleOff) + wn * 128;
    const float* e_b = e_sw + kBN;
    const float* e_sx = reinterpret_cast<const float*>(lds + kScaleOff) + 2 * kBN + wm * 128;
    uint8_t* stage = lds + wave * (128 * 256);    // this wave's 128 x 128 fp16 block (32 KB)
    float xs[4];
#pragma unroll
    for (int b = 0; b < 4; b++) xs[b] = e_sx[b * 32 + msub];
#pragma unroll
    for (int a = 0; a < 4; a++) {
      __builtin_amdgcn_sched_barrier(0);
      float4 s4[4], b4[4];
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int col = a * 32 + 8 * g + 4 * half;
        s4[g] = *reinterpret_cast<const float4*>(e_sw + col);
        b4[g] = *reinterpret_cast<const float4*>(e_b + col);
      }
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int col = a * 32 + 8 * g + 4 * half;   // wave-local output column
        const float ws[4] = {s4[g].x, s4[g].y, s4[g].z, s4[g].w};
        const float bs[4] = {b4[g].x, b4[g].y, b4[g].z, b4[g].w};
#pragma unroll
        for (int b = 0; b < 4; b++) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const int v = (BITS == 4) ? (acc[a][b][4 * g + e] >> 8) : acc[a][b][4 * g + e];
            y[e] = __builtin_fmaf(static_cast<float>(v), __fmul_rn(ws[e], xs[b]), bs[e]);
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
    // Read back whole rows (16 lanes x 16 B = one 256-byte row segment, 4 rows per read) and
    // store them, 32 rows per batch. A wave's LDS operations complete in order, so the reads
    // see its own writes above.
#pragma unroll
    for (int h = 0; h < 4; h++) {
      __builtin_amdgcn_sched_barrier(0);
      uint4 v[8];
#pragma unroll
      for (int it = 0; it < 8; it++) {
        const int row = h * 32 + it * 4 + (lane >> 4);
        v[it] = *reinterpret_cast<const uint4*>(stage + row * 256 + (lane & 15) * 16);
        // Rows with bit 4 set hold their 8-byte halves swapped (see the writes); bit 4 of row is
        // (it >> 2) & 1 for every lane, so this is a compile-time register swap.
        if ((it >> 2) & 1) v[it] = make_uint4(v[it].z, v[it].w, v[it].x, v[it].y);
      }
#pragma unroll
      for (int it = 0; it < 8; it++) {
        const int row = h * 32 + it * 4 + (lane >> 4);
        const int m = m0 + wm * 128 + row;
        const int n = n0 + wn * 128 + 8 * ((lane & 15) ^ (row & 15));
        if (m < M && n < N) {
          // Streaming store: Y is written once and not re-read here, so it should not evict
          // the Wq / Xq panels that neighbouring tiles re-read from L2.
          v4i* dst = reinterpret_cast<v4i*>(static_cast<uint16_t*>(Y) + (int64_t)m * N + n);
          __builtin_nontemporal_store(__builtin_bit_cast(v4i, v[it]), dst);
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
  const int grid = 8 * ((tiles_m + 7) / 8) * tiles_n;   // see the XCD schedule in the kernel
  hipLaunchKernelGGL((gemm_wide_kernel<BITS, OUT>), dim3(grid), dim3(kThreads), 0, st,
                     static_cast<const uint8_t*>(Xq), sx, static_cast<const uint8_t*>(Wq), sw,
                     bias, Y, (int)M, (int)N, (int)Kb, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

bool wide_gemm_supported(int64_t Kb) { return Kb % kBKB == 0 && Kb >= 2 * kBKB; }

hipError_t launch_gemm_wide(const void* Xq, const float* sx, const void* Wq, const float* sw,
                            const float* bias, int64_t M, int64_t N, int64_t K, int bits, void* Y,
                            int out_dt, int32_t* acc32, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t Kb = bits == 8 ? K : K / 2;
  if (!wide_gemm_supported(Kb)) return hipErrorInvalidValue;
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
