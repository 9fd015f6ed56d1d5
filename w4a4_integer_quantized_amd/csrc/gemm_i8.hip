// gemm_i8.hip -- int8 x int8 -> int32 MFMA GEMM with the fused dequantizing epilogue.
//
// Computes acc[m, n] = sum_k Xq[m, k] * Wq[n, k] (both operands K-contiguous) and then
// Y[m, n] = fp16/bf16( fma(f32(acc), fl(w_scale[n] * x_scale[m]), bias[n]) ) -- the W8A8 /
// W4A4 "operations" of the "SAM 3.1 Multiplex INT8/INT4 ConvRot" page ("Quantization recipe")
// with the per-row weight scale and per-token activation scale. INT4 codes are multiplied on
// the INT8 matrix cores, the fallback the same page describes ("Downloads"); gfx950 has no
// int4 MFMA.
//
// Design (gfx950: 256 CUs in 8 XCDs, 160 KB LDS per CU, 64-wide waves, 512 VGPR+AGPR/SIMD):
//   * A 256-thread workgroup owns a 256 (tokens) x 128 (outputs) tile; its 4 waves each own
//     64 x 128 = 2 x 4 blocks of v_mfma_i32_32x32x32_i8 (128 int32 accumulators per lane).
//     Registers (<= 256 per lane) and LDS (74 KB) are sized so that TWO workgroups share a CU:
//     while one is in its epilogue, prologue or at a barrier, the other keeps the matrix cores
//     busy.
//   * K is staged 64 bytes per step (64 int8 or 128 int4 codes) through a 3-deep LDS ring
//     filled by direct global->LDS 16-byte loads (MUBUF buffer loads to LDS, see buffer_rsrc;
//     prefetch distance 2 steps). Rows are 64 B;
//     the 16-byte chunk c of row r sits at c ^ swz(r), which keeps the MFMA fragment reads
//     (ds_read_b128, 32 rows x 2 chunks per wave) free of bank conflicts on gfx950's LDS
//     (see swz). The fragment reads of the next slice are issued between the MFMAs of the
//     current one, MFMA first, so no wave waits on a read it has just issued.
//   * The MFMA "A" operand is a Wq row block and "B" an Xq row block, so each lane ends with
//     4 consecutive output columns of one token. The epilogue converts them and parks the
//     wave's 64 x 128 output block in LDS (16-byte chunks XOR-swizzled by row, 8-byte halves
//     swapped on rows with bit 4 set, which makes the 8-byte writes conflict free), then
//     writes it back as full 256-byte row segments with 16-byte stores. w_scale, bias and x_scale for the
//     tile are loaded at kernel start (latency hidden behind the mainloop) and read from LDS.
//   * INT4: a 16-byte chunk of packed codes (32 nibbles) becomes two MFMA operands,
//     (w << 4) & 0xF0F0F0F0 (even k) and w & 0xF0F0F0F0 (odd k): each byte is 16 * code,
//     exact for codes in [-8, 7]. Both operands get the same k permutation, so the sum is
//     unchanged; the accumulator is 256 * acc and an exact arithmetic shift by 8 recovers it.
//   * Launches with no more tiles than CUs and at least 16 k steps put eight waves on each
//     tile instead (one 512-thread workgroup per CU, 146 KB LDS): two groups of four take the
//     even and the odd k steps in lockstep, each with its own half of a doubled ring, then swap
//     halves of their accumulators through LDS so that each wave finishes one 32-row block.
//   * Launches with more tiles than CUs, int8 codes in the tiled layout and K of 1024, 1536
//     or 2048 bytes (any output: fp16/bf16 or the raw int32 accumulators) load each wave's Xq
//     fragments straight into registers
//     instead (gemm_xr_kernel): a wave multiplies only its own 64 Xq rows, so only Wq, which
//     the four waves share, goes through LDS.
//   * Launches with more tiles than CUs and at least 48 k steps use 256 x 256 tiles instead:
//     eight waves in two groups of four share one 256-row Xq stage and each takes its own
//     128-row half of a 256-row Wq stage (one 512-thread workgroup per CU, 132 KB LDS), which
//     cuts the operand bytes the CU's load path moves per MFMA by a third.
//   * Workgroup -> tile map is XCD-aware: workgroups are dispatched round-robin over the 8
//     XCDs, so logical tile L runs on XCD L / ceil(tiles / 8); neighbouring tiles (same Xq
//     row panel, all of Wq) then share one XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.h"
#include "internal.h"

namespace convrot {
namespace {

using namespace gemm;

constexpr int kBKB = 64;                       // K bytes per step
constexpr int kStages = 3;
constexpr int kThreads = 256;
constexpr int kTileX = kBM * kBKB;             // 16 KB
constexpr int kStageBytes = (kBM + kBN) * kBKB;   // 24 KB
constexpr int kLoadsPerStep = kStageBytes / 1024 / 4;   // wave-wide 1 KB copies per wave: 6

// gfx950 LDS: 64 banks of 4 bytes, 16 lanes of a ds_read_b128 per cycle, and address bit 9
// flips bank bit 5 (measured with the bank-conflict counter). With 64-byte rows that hardware
// hash already separates rows r and r + 8, so the swizzle only spreads rows r..r+7 (bits 1-2).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }

// Raw buffer resource (stride 0, gfx9 32-bit data-format word) over `bytes` bytes from `base`.
// The copies below go through MUBUF loads straight to LDS rather than the FLAT-encoded
// global_load_lds: the compiler counts a FLAT copy as an LDS access too and then waits for
// every copy in flight before each fragment read, while MUBUF copies leave its LDS-read waits
// partial (the kernels wait for their copies themselves, before each barrier). Each resource
// starts at its tile's first row, so the 32-bit offsets stay small for any operand size.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// One wave copies 16 rows x 64 B (1 KB) of a K-contiguous operand into LDS rows
// [row0, row0 + 16) of a tile. `rs` starts at the tile's first row (stride ld bytes) and holds
// `nrows` rows. Lane l fills LDS position (row0 + l/4, chunk l%4), which holds global chunk
// (l%4) ^ swz(row). Rows past the end of the operand re-read its last row (their results are
// never stored).
__device__ __forceinline__ void copy_rows(__amdgpu_buffer_rsrc_t rs, int ld, int row0, int nrows,
                                          int k0, uint8_t* lds_tile, int lane) {
  const int r = row0 + (lane >> 2);
  const int c = (lane & 3) ^ swz(r);
  const int gr = r < nrows ? r : nrows - 1;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_tile + row0 * kBKB), 16,
                                           gr * ld + k0 + 16 * c, 0, 0, 0);
}

// Tiled Xq ([256-row panel][64-byte k step][256 rows][64 B], rows padded to the panel): the
// 16 rows [row0, row0 + 16) of k step k0 / 64 are one contiguous 1 KB block. `rs` starts at
// the panel.
__device__ __forceinline__ void copy_rows_tiled(__amdgpu_buffer_rsrc_t rs, int row0, int k0,
                                                uint8_t* lds_tile, int lane) {
  const int r = row0 + (lane >> 2);
  const int c = (lane & 3) ^ swz(r);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_tile + row0 * kBKB), 16,
                                           (k0 << 8) + (r << 6) + 16 * c, 0, 0, 0);
}

// The two operands' resources for the tile at rows (m0, n0): Xq from its panel (tiled) or
// first row, Wq from row n0, rows clamped to the operand.
struct TileRsrc {
  __amdgpu_buffer_rsrc_t x, w;
  int xrows, wrows;
};
template <bool XT>
__device__ __forceinline__ TileRsrc tile_rsrc(const uint8_t* Xq, const uint8_t* Wq, int M, int N,
                                              int Kb, int m0, int n0, int bn) {
  TileRsrc t;
  t.xrows = M - m0 < kBM ? M - m0 : kBM;
  t.wrows = N - n0 < bn ? N - n0 : bn;
  t.x = XT ? buffer_rsrc(Xq + (int64_t)m0 * Kb, kBM * Kb)
           : buffer_rsrc(Xq + (int64_t)m0 * Kb, t.xrows * Kb);
  t.w = buffer_rsrc(Wq + (int64_t)n0 * Kb, t.wrows * Kb);
  return t;
}

__device__ __forceinline__ v4i read_frag(const uint8_t* lds_tile, int row, int chunk) {
  return *reinterpret_cast<const v4i*>(lds_tile + row * kBKB + ((chunk ^ swz(row)) << 4));
}

// SPLIT = 1: four waves own the tile and walk all of K. SPLIT = 2: eight waves in two groups of
// four; group g takes the k steps 2j + g (its own half of a doubled LDS ring, in lockstep with the
// other group at every barrier), then the groups exchange halves of their accumulators through
// LDS, each sums the 32-row block it finishes, and both run the epilogue on their half. It
// puts a whole CU's two wave slots per SIMD on one tile, for launches with too few tiles to give
// every CU two.
template <int SPLIT>
constexpr int lds_bytes() { return kStages * SPLIT * kStageBytes + (2 * kBN + kBM) * 4; }

template <int BITS, int OUT, bool XT, int SPLIT>
__global__ __launch_bounds__(kThreads * SPLIT, 2 / SPLIT) void gemm_kernel(
    const uint8_t* __restrict__ Xq, const float* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const float* __restrict__ sw, const float* __restrict__ bias, void* __restrict__ Y, int M,
    int N, int Kb, int tiles_m, int tiles_n, int act) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[lds_bytes<SPLIT>()];
  constexpr int kRing = kStages * SPLIT * kStageBytes;   // also where the scales are parked
  constexpr int kSlot = SPLIT * kStageBytes;              // one ring stage, all groups

  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + 7) >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= ntiles) return;
  const int tm = logical / tiles_n;
  const int tn = logical - tm * tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = wave_all & 3;          // wave within its group: tile rows wave*64 ..
  const int grp = wave_all >> 2;          // k-step group (0 when SPLIT == 1)

  // Per-tile epilogue operands, fetched now so their latency hides behind the mainloop.
  float my_sw = 0.0f, my_b = 0.0f, my_sx = 0.0f;
  if constexpr (OUT != kOutS32) {
    const int n = n0 + (int)threadIdx.x, m = m0 + (int)threadIdx.x;
    if (threadIdx.x < kBN && n < N) {
      my_sw = sw[n];
      my_b = bias ? bias[n] : 0.0f;
    }
    if (threadIdx.x < kBM && m < M) my_sx = sx[m];
  }

  v16i acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; a++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[a][b][r] = 0;

  // Stage s of this group holds the Xq tile (256 rows) then the Wq tile (128 rows), 64 B per
  // row, for k step SPLIT*j + grp.
  uint8_t* const ring = lds + grp * kStageBytes;
  const TileRsrc rs = tile_rsrc<XT>(Xq, Wq, M, N, Kb, m0, n0, kBN);
  auto issue = [&](int stage, int j) {
    const int k0 = (SPLIT * j + grp) * kBKB;
    uint8_t* tX = ring + stage * kSlot;
    uint8_t* tW = tX + kTileX;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if constexpr (XT) {
        copy_rows_tiled(rs.x, (wave * 4 + i) * 16, k0, tX, lane);
      } else {
        copy_rows(rs.x, Kb, (wave * 4 + i) * 16, rs.xrows, k0, tX, lane);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; i++) copy_rows(rs.w, Kb, (wave * 2 + i) * 16, rs.wrows, k0, tW, lane);
  };

  // Fragments of one 32-byte k slice: 4 Wq row blocks and this wave's 2 Xq row blocks.
  const int rsub = lane & 31, fhalf = lane >> 5;
  auto read_frags = [&](int stage, int ks, v4i (&wf)[4], v4i (&xf)[2]) {
    const uint8_t* tX = ring + stage * kSlot;
    const uint8_t* tW = tX + kTileX;
    const int chunk = 2 * ks + fhalf;
#pragma unroll
    for (int a = 0; a < 4; a++) wf[a] = read_frag(tW, a * 32 + rsub, chunk);
#pragma unroll
    for (int b = 0; b < 2; b++) xf[b] = read_frag(tX, wave * 64 + b * 32 + rsub, chunk);
  };
  auto mfma_slice = [&](const v4i (&wf)[4], const v4i (&xf)[2]) {
    if constexpr (BITS == 8) {
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 2; b++)
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[a], xf[b], acc[a][b], 0, 0, 0);
    } else {
      v4i wlo[4], whi[4], xlo[2], xhi[2];
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          wlo[a][e] = (wf[a][e] << 4) & 0xF0F0F0F0;
          whi[a][e] = wf[a][e] & 0xF0F0F0F0;
        }
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          xlo[b][e] = (xf[b][e] << 4) & 0xF0F0F0F0;
          xhi[b][e] = xf[b][e] & 0xF0F0F0F0;
        }
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 2; b++) {
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wlo[a], xlo[b], acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(whi[a], xhi[b], acc[a][b], 0, 0, 0);
        }
    }
  };

  // Software-pipelined k loop over a ring of 3 LDS stages (this group's step j lives in stage
  // j % 3).
  // Step j: the slice-1 fragments of step j are read and -- when LOAD -- the 6 direct-to-LDS
  // loads of step j+2 are issued under the 8 (int4: 16) MFMAs of slice 0; then -- when MID --
  // the wave waits for its own loads of step j+1 and for all its fragment reads, passes the
  // workgroup barrier, and reads slice 0 of step j+1 under the MFMAs of slice 1. LDS latency
  // and the barrier therefore overlap matrix work instead of following it.
  // Why the ring is race free: the loads issued in step j fill stage (j+2) % 3 = (j-1) % 3,
  // whose last reads (slice 1 of step j-1) every wave completed before the barrier of step
  // j-1; the reads of stage (j+1) % 3 follow the barrier of step j, which every wave passes
  // only after its loads of step j+1 have landed. With SPLIT = 2 both groups take the same
  // number of steps, so every barrier is passed by all eight waves.
  constexpr int kMfmaPerSlice = BITS == 8 ? 8 : 16;
  auto body = [&](auto load_tag, auto mid_tag, int kt, v4i (&wf0)[4], v4i (&xf0)[2]) {
    constexpr bool LOAD = decltype(load_tag)::value;
    constexpr bool MID = decltype(mid_tag)::value;
    const int cur = kt % kStages;
    v4i wf1[4], xf1[2];
    read_frags(cur, 1, wf1, xf1);
    if constexpr (LOAD) issue((kt + 2) % kStages, kt + 2);
    mfma_slice(wf0, xf0);
#pragma unroll
    for (int i = 0; i < 6; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // DS read (slice 1)
    }
    if constexpr (LOAD) {
#pragma unroll
      for (int i = 0; i < kLoadsPerStep; i++) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // VMEM (global -> LDS)
        if (i < kMfmaPerSlice - 6) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerSlice, 0);   // the rest of slice 0
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MID) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if constexpr (LOAD) {
        asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_frags((kt + 1) % kStages, 0, wf0, xf0);
    }
    mfma_slice(wf1, xf1);
    if constexpr (MID) {
#pragma unroll
      for (int i = 0; i < 6; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read (next slice 0)
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerSlice, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nk = Kb / kBKB / SPLIT;       // steps per group (the launcher checks divisibility)
  issue(0, 0);
  if (nk > 1) {
    issue(1, 1);
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  // The epilogue operands have landed too (they were requested first): park them in LDS.
  if constexpr (OUT != kOutS32) {
    float* e_sw = reinterpret_cast<float*>(lds + kRing);
    if (threadIdx.x < kBN) {
      e_sw[threadIdx.x] = my_sw;
      e_sw[kBN + threadIdx.x] = my_b;
    }
    if (threadIdx.x < kBM) e_sw[2 * kBN + threadIdx.x] = my_sx;
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  v4i wf0[4], xf0[2];
  read_frags(0, 0, wf0, xf0);
  int kt = 0;
  for (; kt + 2 < nk; kt++) body(std::true_type{}, std::true_type{}, kt, wf0, xf0);
  if (kt + 1 < nk) body(std::false_type{}, std::true_type{}, kt++, wf0, xf0);
  body(std::false_type{}, std::false_type{}, kt, wf0, xf0);
  __syncthreads();

  const float* scales = reinterpret_cast<const float*>(lds + kRing);
  if constexpr (SPLIT == 1) {
    tile_epilogue_act<BITS, OUT, 2>(act, acc, scales, lds + wave * (64 * 256), wave * 64, lane, m0, n0, M, N, Y);
  } else {
    // Group g finishes row block b = g of its four waves' rows: it sends its partial sums of
    // block 1 - g to the partner wave (wave_all ^ 4) and adds the partner's partials of block g.
    // Exchange layout: [wave_all][a][r4][lane] of 16-byte int4 (conflict-free 16-byte accesses).
    int4* xch = reinterpret_cast<int4*>(lds);
    auto slot = [&](int w, int a, int r4) { return xch + ((w * 4 + a) * 4 + r4) * 64 + lane; };
    auto finish = [&](auto keep_tag) {
      constexpr int KB = decltype(keep_tag)::value;   // the block this group finishes
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++)
          *slot(wave_all, a, r4) = make_int4(acc[a][1 - KB][4 * r4], acc[a][1 - KB][4 * r4 + 1],
                                             acc[a][1 - KB][4 * r4 + 2], acc[a][1 - KB][4 * r4 + 3]);
      __syncthreads();
      v16i keep[4][1];
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
          const int4 o = *slot(wave_all ^ 4, a, r4);
          keep[a][0][4 * r4] = acc[a][KB][4 * r4] + o.x;
          keep[a][0][4 * r4 + 1] = acc[a][KB][4 * r4 + 1] + o.y;
          keep[a][0][4 * r4 + 2] = acc[a][KB][4 * r4 + 2] + o.z;
          keep[a][0][4 * r4 + 3] = acc[a][KB][4 * r4 + 3] + o.w;
        }
      __syncthreads();   // every exchange read is done before the staging below reuses LDS
      tile_epilogue_act<BITS, OUT, 1>(act, keep, scales, lds + wave_all * (32 * 256), wave * 64 + KB * 32, lane,
                                  m0, n0, M, N, Y);
    };
    if (grp == 0) {
      finish(std::integral_constant<int, 0>{});
    } else {
      finish(std::integral_constant<int, 1>{});
    }
  }
}

// 256 x 256 tiles: eight waves in two groups of four; group g computes output columns
// 128g .. 128g+127 of the tile (its half of a 256-row Wq stage) against the shared 256-row Xq
// stage, so a CU moves two thirds of the operand bytes per MFMA of a 256 x 128 tile (32 KB
// instead of 48 KB per 256 x 256 outputs and 64-byte k step).
constexpr int kStageN2 = 2 * kBM * kBKB;              // 16 KB Xq + 16 KB Wq
constexpr int kScaleBlk = (2 * kBN + kBM) * 4;        // one group's [w_scale | bias | x_scale]
constexpr int kStageOut = 8 * 64 * 256;               // epilogue: 8 waves x 64 rows x 256 B
constexpr int kLdsN2 = (kStageOut > kStages * kStageN2 ? kStageOut : kStages * kStageN2) + 2 * kScaleBlk;

template <int BITS, int OUT, bool XT>
__global__ __launch_bounds__(512, 1) void gemm_n2_kernel(
    const uint8_t* __restrict__ Xq, const float* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const float* __restrict__ sw, const float* __restrict__ bias, void* __restrict__ Y, int M,
    int N, int Kb, int tiles_m, int tiles_n, int act) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsN2];
  constexpr int kScales = kLdsN2 - 2 * kScaleBlk;

  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + 7) >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= ntiles) return;
  const int tm = logical / tiles_n;
  const int tn = logical - tm * tiles_n;
  const int m0 = tm * kBM, n0 = tn * 256;

  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = wave_all & 3;
  const int grp = wave_all >> 2;

  float my_sw = 0.0f, my_b = 0.0f, my_sx = 0.0f;
  if constexpr (OUT != kOutS32) {
    const int n = n0 + (int)threadIdx.x, m = m0 + (int)(threadIdx.x & 255);
    if (threadIdx.x < 256 && n < N) {
      my_sw = sw[n];
      my_b = bias ? bias[n] : 0.0f;
    }
    if (m < M) my_sx = sx[m];
  }

  v16i acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; a++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[a][b][r] = 0;

  const TileRsrc rs = tile_rsrc<XT>(Xq, Wq, M, N, Kb, m0, n0, 256);
  auto issue = [&](int stage, int kt) {
    const int k0 = kt * kBKB;
    uint8_t* tX = lds + stage * kStageN2;
    uint8_t* tW = tX + kTileX;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int row0 = (wave_all * 2 + i) * 16;
      if constexpr (XT) {
        copy_rows_tiled(rs.x, row0, k0, tX, lane);
      } else {
        copy_rows(rs.x, Kb, row0, rs.xrows, k0, tX, lane);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; i++) copy_rows(rs.w, Kb, (wave_all * 2 + i) * 16, rs.wrows, k0, tW, lane);
  };

  const int rsub = lane & 31, fhalf = lane >> 5;
  auto read_frags = [&](int stage, int ks, v4i (&wf)[4], v4i (&xf)[2]) {
    const uint8_t* tX = lds + stage * kStageN2;
    const uint8_t* tW = tX + kTileX;
    const int chunk = 2 * ks + fhalf;
#pragma unroll
    for (int a = 0; a < 4; a++) wf[a] = read_frag(tW, grp * 128 + a * 32 + rsub, chunk);
#pragma unroll
    for (int b = 0; b < 2; b++) xf[b] = read_frag(tX, wave * 64 + b * 32 + rsub, chunk);
  };
  auto mfma_slice = [&](const v4i (&wf)[4], const v4i (&xf)[2]) {
    if constexpr (BITS == 8) {
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 2; b++)
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[a], xf[b], acc[a][b], 0, 0, 0);
    } else {
      v4i wlo[4], whi[4], xlo[2], xhi[2];
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          wlo[a][e] = (wf[a][e] << 4) & 0xF0F0F0F0;
          whi[a][e] = wf[a][e] & 0xF0F0F0F0;
        }
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          xlo[b][e] = (xf[b][e] << 4) & 0xF0F0F0F0;
          xhi[b][e] = xf[b][e] & 0xF0F0F0F0;
        }
#pragma unroll
      for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 2; b++) {
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wlo[a], xlo[b], acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(whi[a], xhi[b], acc[a][b], 0, 0, 0);
        }
    }
  };

  constexpr int kMfmaPerSlice = BITS == 8 ? 8 : 16;
  auto body = [&](auto load_tag, auto mid_tag, int kt, v4i (&wf0)[4], v4i (&xf0)[2]) {
    constexpr bool LOAD = decltype(load_tag)::value;
    constexpr bool MID = decltype(mid_tag)::value;
    const int cur = kt % kStages;
    v4i wf1[4], xf1[2];
    read_frags(cur, 1, wf1, xf1);
    if constexpr (LOAD) issue((kt + 2) % kStages, kt + 2);
    mfma_slice(wf0, xf0);
    // Two fragment reads after each of the first three MFMAs (measured 4-6% faster here than
    // one read per MFMA: the last read has five MFMAs to land instead of two).
#pragma unroll
    for (int i = 0; i < 3; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // DS read (slice 1)
    }
    if constexpr (LOAD) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // VMEM (global -> LDS)
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerSlice, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MID) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if constexpr (LOAD) {
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_frags((kt + 1) % kStages, 0, wf0, xf0);
    }
    mfma_slice(wf1, xf1);
    if constexpr (MID) {
#pragma unroll
      for (int i = 0; i < 3; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);      // DS read (next slice 0)
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerSlice, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nk = Kb / kBKB;
  issue(0, 0);
  if (nk > 1) {
    issue(1, 1);
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  if constexpr (OUT != kOutS32) {
    // Each group's scale block: [w_scale (its 128 columns) | bias | x_scale (all 256 rows)].
    float* e0 = reinterpret_cast<float*>(lds + kScales);
    if (threadIdx.x < 256) {
      const int g = threadIdx.x >> 7, c = threadIdx.x & 127;
      e0[g * (kScaleBlk / 4) + c] = my_sw;
      e0[g * (kScaleBlk / 4) + kBN + c] = my_b;
    }
    e0[(threadIdx.x >> 8) * (kScaleBlk / 4) + 2 * kBN + (threadIdx.x & 255)] = my_sx;
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  v4i wf0[4], xf0[2];
  read_frags(0, 0, wf0, xf0);
  int kt = 0;
  for (; kt + 2 < nk; kt++) body(std::true_type{}, std::true_type{}, kt, wf0, xf0);
  if (kt + 1 < nk) body(std::false_type{}, std::true_type{}, kt++, wf0, xf0);
  body(std::false_type{}, std::false_type{}, kt, wf0, xf0);
  __syncthreads();
  const float* scales = reinterpret_cast<const float*>(lds + kScales + grp * kScaleBlk);
  tile_epilogue_act<BITS, OUT, 2>(act, acc, scales, lds + wave_all * (64 * 256), wave * 64, lane, m0, n0 + 128 * grp, M, N, Y);
}

// Xq fragments straight into registers (int8 codes, tiled Xq; output fp16/bf16, or the int32
// accumulators for the same launches' bit-exact checks). In the
// 256 x 128 tile each wave multiplies only its own 64 Xq rows, so staging Xq through LDS buys
// no reuse: here each wave loads its two 32-row fragments per 32-byte slice with 16-byte global
// loads (lane l: row l % 32, 16-byte chunk 2 s + l / 32 of the step), two k steps ahead in three
// register sets, and only Wq (shared by the four waves) goes through a 3-deep LDS ring. Per
// k step the LDS reads drop from 6 to 4 fragments per slice. NK = Kb / 64 is a compile-time
// count so that the register sets are named statically (the k loop unrolls fully).
constexpr int kStageW = kBN * kBKB;                      // 8 KB of Wq per ring stage
constexpr int kStageOutXr = 4 * 64 * 256;                // epilogue staging: 4 waves x 16 KB
constexpr int kLdsXr = (kStageOutXr > kStages * kStageW ? kStageOutXr : kStages * kStageW) +
                       (2 * kBN + kBM) * 4;

template <int OUT, int NK>
__global__ __launch_bounds__(kThreads, 2) void gemm_xr_kernel(
    const uint8_t* __restrict__ Xq, const float* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const float* __restrict__ sw, const float* __restrict__ bias, void* __restrict__ Y, int M,
    int N, int Kb, int tiles_m, int tiles_n, int act) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsXr];
  constexpr int kScalesOff = kLdsXr - (2 * kBN + kBM) * 4;
  constexpr int nk = NK;

  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + 7) >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= ntiles) return;
  const int tm = logical / tiles_n;
  const int tn = logical - tm * tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  float my_sw = 0.0f, my_b = 0.0f, my_sx = 0.0f;
  if constexpr (OUT != kOutS32) {
    const int n = n0 + (int)threadIdx.x, m = m0 + (int)threadIdx.x;
    if (threadIdx.x < kBN && n < N) {
      my_sw = sw[n];
      my_b = bias ? bias[n] : 0.0f;
    }
    if (threadIdx.x < kBM && m < M) my_sx = sx[m];
  }

  v16i acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; a++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[a][b][r] = 0;

  // Tiled Xq: the panel's k step kk is a 256-row x 64-byte block at (tm * nk + kk) * 16 KB.
  const uint8_t* xbase = Xq + ((int64_t)tm * nk << 14) + (wave * 64 + (lane & 31)) * 64 + (lane >> 5) * 16;
  auto load_x = [&](int kk, v4i (&xr)[2][2]) __attribute__((always_inline)) {
    const uint8_t* p = xbase + ((int64_t)kk << 14);
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int s = 0; s < 2; s++) xr[b][s] = *reinterpret_cast<const v4i*>(p + b * 2048 + s * 32);
  };
  const int wrows = N - n0 < kBN ? N - n0 : kBN;
  const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(Wq + (int64_t)n0 * Kb, wrows * Kb);
  auto issue_w = [&](int slot, int kk) __attribute__((always_inline)) {
    uint8_t* tW = lds + slot * kStageW;
#pragma unroll
    for (int i = 0; i < 2; i++) copy_rows(wrs, Kb, (wave * 2 + i) * 16, wrows, kk * kBKB, tW, lane);
  };
  const int rsub = lane & 31, fhalf = lane >> 5;
  auto read_w = [&](int slot, int ks, v4i (&wf)[4]) __attribute__((always_inline)) {
    const uint8_t* tW = lds + slot * kStageW;
#pragma unroll
    for (int a = 0; a < 4; a++) wf[a] = read_frag(tW, a * 32 + rsub, 2 * ks + fhalf);
  };
  auto mfma_slice = [&](const v4i (&wf)[4], const v4i (&xr)[2][2], int s) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
      for (int b = 0; b < 2; b++)
        acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[a], xr[b][s], acc[a][b], 0, 0, 0);
  };

  // s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8),
  // issued through the builtin so that the compiler's own wait insertion accounts for them.
  constexpr int kWaitLgkm0 = 0xC07F;                                   // lgkmcnt(0)
  auto vm_wait = [](auto n_tag) __attribute__((always_inline)) {
    constexpr int n = decltype(n_tag)::value;
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
  };
  // Step kt computes with register set kt % 3 and at its start loads step kt + 2 into set
  // (kt + 2) % 3, which step kt - 1 has finished with; Wq runs two steps ahead through the LDS
  // ring, slot kt % 3. Loads per step, in issue order: 2 Wq copies, then 4 Xq loads.
  // Why the ring is race free: the copies issued in step kt fill slot (kt + 2) % 3 =
  // (kt - 1) % 3, whose last reads (slice 1 of step kt - 1, issued at that step's start) every
  // wave completed (lgkmcnt(0)) before the barrier of step kt - 1; the reads of slot
  // (kt + 1) % 3 follow the barrier of step kt, which every wave passes only after its own
  // copies of step kt + 1 have landed.
  v4i xs[3][2][2];
  issue_w(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_x(0, xs[0]);
  __builtin_amdgcn_sched_barrier(0);
  issue_w(1, 1);
  __builtin_amdgcn_sched_barrier(0);
  load_x(1, xs[1]);
  __builtin_amdgcn_sched_barrier(0);
  vm_wait(std::integral_constant<int, 10>{});   // Wq of step 0 landed (10 loads issued after it)
  if constexpr (OUT != kOutS32) {
    float* e_sw = reinterpret_cast<float*>(lds + kScalesOff);
    if (threadIdx.x < kBN) {
      e_sw[threadIdx.x] = my_sw;
      e_sw[kBN + threadIdx.x] = my_b;
    }
    if (threadIdx.x < kBM) e_sw[2 * kBN + threadIdx.x] = my_sx;
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  v4i wf0[4];
  read_w(0, 0, wf0);

  auto body = [&](auto load_tag, auto mid_tag, int kt, v4i (&xc)[2][2], v4i (&xn)[2][2]) __attribute__((always_inline)) {
    constexpr bool LOAD = decltype(load_tag)::value;    // kt + 2 < nk
    constexpr bool MID = decltype(mid_tag)::value;      // kt + 1 < nk
    v4i wf1[4];
    read_w(kt % kStages, 1, wf1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (LOAD) {
      issue_w((kt + 2) % kStages, kt + 2);
      __builtin_amdgcn_sched_barrier(0);
      load_x(kt + 2, xn);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_slice(wf0, xc, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MID) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      // Wq of step kt + 1 landed: issued after it were the 4 Xq loads of step kt + 1 and, when
      // LOAD, the 6 loads of step kt + 2.
      if constexpr (LOAD) {
        vm_wait(std::integral_constant<int, 10>{});
      } else {
        vm_wait(std::integral_constant<int, 4>{});
      }
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_w((kt + 1) % kStages, 0, wf0);
    }
    mfma_slice(wf1, xc, 1);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // DS read (next slice 0)
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  using T = std::true_type;
  using F = std::false_type;
#pragma unroll
  for (int kt = 0; kt < nk - 2; kt++) body(T{}, T{}, kt, xs[kt % 3], xs[(kt + 2) % 3]);
  body(F{}, T{}, nk - 2, xs[(nk - 2) % 3], xs[nk % 3]);
  body(F{}, F{}, nk - 1, xs[(nk - 1) % 3], xs[(nk + 1) % 3]);
  __syncthreads();
  const float* scales = reinterpret_cast<const float*>(lds + kScalesOff);
  tile_epilogue_act<8, OUT, 2>(act, acc, scales, lds + wave * (64 * 256), wave * 64, lane, m0, n0, M, N, Y);
}

template <int BITS, int OUT, bool XT>
hipError_t launch(const void* Xq, const float* sx, const void* Wq, const float* sw,
                  const float* bias, int64_t M, int64_t N, int64_t Kb, void* Y, int act, hipStream_t st) {
  const int tiles_m = (int)((M + kBM - 1) / kBM);
  const int tiles_n = (int)((N + kBN - 1) / kBN);
  const int ntiles = tiles_m * tiles_n;
  const int grid = ((ntiles + 7) / 8) * 8;
  // Too few tiles to give every CU two workgroups: put eight waves on each tile instead (the
  // k steps split between two wave groups), when the steps divide evenly and are long enough
  // (at least 8 per group) for the split to pay for the final exchange; measured 4-8% faster
  // on 168-tile launches with 64 steps, and slower with 1 step per group.
  // Enough tiles to fill the machine, int8 codes in the tiled layout and K = 1024, 1536 or
  // 2048 bytes: Xq fragments straight into registers; measured 5-7% faster than four waves
  // staging both operands through LDS (and 2% slower on int4 codes, whose unpacking keeps the
  // matrix cores the tighter limit).
  // Enough tiles to fill the machine and long K (at least 48 steps): 256 x 256 tiles halve the
  // operand bytes each CU moves per MFMA; measured 6-12% faster at K = 3072-6144 bytes, and
  // 5% slower at K = 1024 bytes, where the longer prologue and epilogue per tile dominate.
  if (ntiles <= kNumCUs && (Kb / kBKB) % 2 == 0 && Kb / kBKB >= 16) {
    hipLaunchKernelGGL((gemm_kernel<BITS, OUT, XT, 2>), dim3(grid), dim3(2 * kThreads), 0, st,
                       static_cast<const uint8_t*>(Xq), sx, static_cast<const uint8_t*>(Wq), sw,
                       bias, Y, (int)M, (int)N, (int)Kb, tiles_m, tiles_n, act);
    return hipGetLastError();
  }
  if constexpr (BITS == 8 && XT) {
    if (ntiles > kNumCUs && (Kb == 1024 || Kb == 1536 || Kb == 2048)) {
      auto k = Kb == 1024 ? gemm_xr_kernel<OUT, 16> : Kb == 1536 ? gemm_xr_kernel<OUT, 24> : gemm_xr_kernel<OUT, 32>;
      hipLaunchKernelGGL(k, dim3(grid), dim3(kThreads), 0, st, static_cast<const uint8_t*>(Xq), sx,
                         static_cast<const uint8_t*>(Wq), sw, bias, Y, (int)M, (int)N, (int)Kb,
                         tiles_m, tiles_n, act);
      return hipGetLastError();
    }
  }
  if (ntiles > kNumCUs && Kb >= 3072) {
    const int tiles_n2 = (int)((N + 255) / 256);
    const int ntiles2 = tiles_m * tiles_n2;
    hipLaunchKernelGGL((gemm_n2_kernel<BITS, OUT, XT>), dim3(((ntiles2 + 7) / 8) * 8), dim3(512), 0,
                       st, static_cast<const uint8_t*>(Xq), sx, static_cast<const uint8_t*>(Wq), sw,
                       bias, Y, (int)M, (int)N, (int)Kb, tiles_m, tiles_n2, act);
  } else {
    hipLaunchKernelGGL((gemm_kernel<BITS, OUT, XT, 1>), dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const uint8_t*>(Xq), sx, static_cast<const uint8_t*>(Wq), sw,
                       bias, Y, (int)M, (int)N, (int)Kb, tiles_m, tiles_n, act);
  }
  return hipGetLastError();
}

template <bool XT>
hipError_t launch_layout(const void* Xq, const float* sx, const void* Wq, const float* sw,
                         const float* bias, int64_t M, int64_t N, int64_t Kb, int bits, void* Y,
                         int out_dt, int32_t* acc32, int act, hipStream_t stream) {
  if (acc32) {
    return bits == 8 ? launch<8, kOutS32, XT>(Xq, sx, Wq, sw, bias, M, N, Kb, acc32, act, stream)
                     : launch<4, kOutS32, XT>(Xq, sx, Wq, sw, bias, M, N, Kb, acc32, act, stream);
  }
  if (out_dt == kF16)
    return bits == 8 ? launch<8, kOutF16, XT>(Xq, sx, Wq, sw, bias, M, N, Kb, Y, act, stream)
                     : launch<4, kOutF16, XT>(Xq, sx, Wq, sw, bias, M, N, Kb, Y, act, stream);
  return bits == 8 ? launch<8, kOutBF16, XT>(Xq, sx, Wq, sw, bias, M, N, Kb, Y, act, stream)
                   : launch<4, kOutBF16, XT>(Xq, sx, Wq, sw, bias, M, N, Kb, Y, act, stream);
}

}  // namespace

hipError_t launch_gemm(const void* Xq, const float* sx, const void* Wq, const float* sw,
                       const float* bias, int64_t M, int64_t N, int64_t K, int bits,
                       bool x_tiled, void* Y, int out_dt, int32_t* acc32, int act,
                       hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t Kb = bits == 8 ? K : K / 2;
  // Tiled activation codes (the fused path): these kernels measured fastest on every workload
  // shape. Row-major codes: they are also the default, except for K of 1536-3071 bytes on
  // enough tiles to fill the machine, where the 128-byte-row 256 x 256 kernel's lower operand
  // traffic per MFMA measured faster (by up to ~20%) than 64-byte row segments; from 3072 bytes
  // on, the eight-wave 256 x 256 kernel here measured faster still (by ~15%).
  // The 128-byte-row kernel has no activation variant; with one, the 64-byte-row kernels run.
  if (x_tiled && gemm_rw_supported(M, N, Kb, bits, x_tiled))
    return launch_gemm_rw(Xq, sx, Wq, sw, bias, M, N, Y, out_dt, acc32, act, stream);
  if (x_tiled)
    return launch_layout<true>(Xq, sx, Wq, sw, bias, M, N, Kb, bits, Y, out_dt, acc32, act, stream);
  const int64_t wide_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (act == kActNone && wide_gemm_supported(Kb) && Kb >= 1536 && Kb < 3072 && wide_tiles >= 192)
    return launch_gemm_wide(Xq, sx, Wq, sw, bias, M, N, K, bits, Y, out_dt, acc32, stream);
  return launch_layout<false>(Xq, sx, Wq, sw, bias, M, N, Kb, bits, Y, out_dt, acc32, act, stream);
}

}  // namespace convrot
