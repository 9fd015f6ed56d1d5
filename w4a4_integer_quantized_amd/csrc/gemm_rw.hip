// gemm_rw.hip -- int8 GEMM with the weight tile resident in LDS and eight independent waves.
//
// The same product and epilogue as gemm_i8.hip (acc[m, n] = sum_k Xq[m, k] * Wq[n, k] in int32,
// Y = fp16/bf16(fma(f32(acc), fl(w_scale[n] * x_scale[m]), bias[n]))): the W8A8 operations of
// the "SAM 3.1 Multiplex INT8/INT4 ConvRot" page ("Quantization recipe"), per-row weight scale
// and per-token activation scale. This kernel serves int8 codes with K = 1024 in the tiled
// activation layout, on launches with many 64-token blocks per output tile.
//
// Design (gfx950: 256 CUs in 8 XCDs of 32, 160 KB LDS per CU, 4 SIMDs per CU):
//   * One 512-thread workgroup per CU. The workgroup owns BN output features (an "n-tile")
//     for its whole life: their weight rows, all of K, are copied into LDS once (BN * 1 KB,
//     96 or 128 KB) in MFMA-fragment order, so every fragment read is one contiguous 1 KB block.
//     w_scale and bias for the n-tile are parked next to them.
//   * Each of the eight waves then walks its own sequence of 64-token blocks: it streams those
//     tokens' codes from global memory straight into registers (2 k steps ahead), multiplies
//     them against the resident weights with v_mfma_i32_16x16x64_i8 (A = 16 weight rows,
//     B = 16 tokens, both 64 bytes of K per lane group), and finishes each block with its own
//     epilogue through a private LDS staging area. No barrier follows the initial copy: the two
//     waves on each SIMD run unsynchronized, so one's epilogue overlaps the other's matrix work.
//   * With the 16 x 16 x 64 operand layout (lane l: row l % 16, bytes 16 (l / 16) .. +16 of a
//     64-byte k step) a 16-token fragment is 16 rows x 64 B, one contiguous 1 KB block of the
//     tiled activation layout, so each fragment load moves whole cache lines.
//   * Work map: workgroup b runs on XCD b % 8 (round-robin dispatch). The 32 workgroups of an
//     XCD split into NT n-tiles x G row groups (NT * G = 32); XCD x takes the x-th eighth of the
//     token blocks, split G ways. All workgroups of an XCD thus read the same token blocks at
//     about the same time, and each block of codes comes from HBM once per XCD and then from
//     that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.h"
#include "internal.h"

namespace convrot {
namespace {

using namespace gemm;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRwThreads = 512;
constexpr int kRwWaves = 8;
constexpr int kRwRows = 64;            // tokens per wave tile
constexpr int kRwDepth = 2;            // k steps of codes in flight ahead of the MFMAs
constexpr int kRwSets = 4;             // register sets of codes (a power of two > kRwDepth)

// Epilogue staging, per wave: two buffers of 16 tokens x 96 features in 192-byte rows; the
// 16-byte chunk c of row r sits at position (c + 3 (r / 2)) mod 12. Under gfx950's LDS bank
// model (64 banks of 4 bytes, address bit 9 folded into bank bit 5) the 8-byte writes of 32
// lanes are conflict free and the 16-byte row reads at most 2-way conflicted (checked
// exhaustively for every buffer offset used).
template <int BN> struct RwShape {
  static constexpr int NA = BN / 16;                       // 16-row weight blocks
  static constexpr int kPitch = 192;                       // staged row pitch in bytes
  static constexpr int kBuf = 16 * kPitch;                 // one staging buffer
  static constexpr int kStage = 2 * kBuf;                  // bytes per wave
  static constexpr int kWq = BN * 1024;                    // resident weights (K = 1024)
  static constexpr int kLds = kWq + kRwWaves * kStage + 2 * BN * 4 + 16;   // + block counter
};

__device__ __forceinline__ int stage_pos(int c, int r) {
  int p = c + 3 * (r >> 1);
  p = p >= 12 ? p - 12 : p;
  return p >= 12 ? p - 12 : p;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8):
// vmcnt(n) with lgkmcnt(0), or vmcnt(n) alone.
constexpr int vm_lgkm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// NT n-tiles per XCD times G row groups = 32 workgroups per XCD; rb_total 64-token blocks.
// The per-wave loop body (16 k steps and the epilogue) is one basic block: stores and the
// x_scale loads are buffer operations whose out-of-range lanes the hardware drops (stores) or
// zero-fills (loads), and the activation is a template parameter. With no branch inside,
// code generation cannot sink the next block's look-ahead loads below the MFMAs that hide
// them.
template <int OUT, int BN, int ACT>
__global__ __launch_bounds__(kRwThreads, 1) void gemm_rw_kernel(
    const uint8_t* __restrict__ Xq, const float* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const float* __restrict__ sw, const float* __restrict__ bias, void* __restrict__ Y, int M,
    int N, int NT, int G, int rb_total, uint32_t xq_bytes) {
  using S = RwShape<BN>;
  constexpr int NA = S::NA;
  constexpr int NK = 16;                 // 64-byte k steps (K = 1024)
  constexpr int Kb = NK * 64;
  constexpr int kOutBytes = OUT == kOutS32 ? 4 : 2;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[S::kLds];
  float* const e_sw = reinterpret_cast<float*>(lds + S::kWq + kRwWaves * S::kStage);
  float* const e_b = e_sw + BN;
  int* const next_block = reinterpret_cast<int*>(e_b + BN);

  const int xcd = blockIdx.x & 7;
  const int c = blockIdx.x >> 3;
  const int nt = c % NT, g = c / NT;
  const int n0 = nt * BN;
  const int parts = 8 * G, part = xcd * G + g;
  const int rb_lo = (int)((int64_t)rb_total * part / parts);
  const int rb_hi = (int)((int64_t)rb_total * (part + 1) / parts);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // 1. The n-tile's weights into LDS, fragment f = kk * NA + a at f * 1 KB: lane l holds row
  //    n0 + 16 a + l % 16, bytes 64 kk + 16 (l / 16) .. +16. Rows past N re-read the last row.
  //    Wave w copies fragments w + 8 i in increasing i, so its first half of the copies holds
  //    k steps 0..7 (fragments 0..47) and its second half k steps 8..15. The workgroup starts
  //    multiplying once the first half has landed; the first block waits for the second half
  //    (and passes a second barrier) before it reads the weights of k step 8.
  constexpr int kFrags = NA * NK;
  constexpr int kFillPerWave = kFrags / kRwWaves;             // 12 copies per wave
  static_assert(kFrags % kRwWaves == 0 && kFillPerWave % 2 == 0 &&
                    kRwWaves * (kFillPerWave / 2) == NA * (NK / 2),
                "each wave's first half of copies is exactly k steps 0..NK/2-1");
  {
    float my_sw = 0.0f, my_b = 0.0f;
    if constexpr (OUT != kOutS32) {
      // Issued before the copies, so that parking them in LDS waits for these loads only.
      if ((int)threadIdx.x < BN) {
        const int n = n0 + (int)threadIdx.x;
        my_sw = n < N ? sw[n] : 0.0f;
        my_b = (n < N && bias) ? bias[n] : 0.0f;
      }
    }
    const int wrows = N - n0 < BN ? N - n0 : BN;
    const __amdgpu_buffer_rsrc_t wrs = rw_rsrc(Wq + (int64_t)n0 * Kb, (uint32_t)wrows * Kb);
#pragma unroll
    for (int i = 0; i < kFillPerWave; i++) {
      const int f = wave + kRwWaves * i;
      const int kk = f / NA, a = f - kk * NA;
      int r = a * 16 + (lane & 15);
      r = r < wrows ? r : wrows - 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_void*)(lds + f * 1024), 16,
                                               r * Kb + kk * 64 + (lane >> 4) * 16, 0, 0, 0);
    }
    if constexpr (OUT != kOutS32) {
      if ((int)threadIdx.x < BN) {
        e_sw[threadIdx.x] = my_sw;
        e_b[threadIdx.x] = my_b;
      }
    }
    if (threadIdx.x == 0) *next_block = rb_lo + kRwWaves;
    // This wave's first half of the copies has landed (the second half may still be in
    // flight), and so have its LDS writes; then every wave's first half has.
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(kFillPerWave / 2));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }

  // 2. The workgroup's token blocks [rb_lo, rb_hi): wave w starts with block rb_lo + w and then
  //    claims the next unclaimed one from a counter in LDS, so that waves that run faster take
  //    more blocks and the workgroup's waves finish together. A wave claims its next block as
  //    it starts the current one, in time to load the next block's first k steps ahead.
  int rb = rb_lo + wave;
  if (rb >= rb_hi) {
    // Not reached under the launcher's rule (every wave has a first block); a wave without
    // one still passes the first block's barrier before it leaves.
    __builtin_amdgcn_s_barrier();
    return;
  }
  // One LDS atomic per claim: every lane adds (lane 0 adds 1, the others 0), lane 0's return
  // value is the claimed block. (No branch, so the block loop stays one basic block.)
  auto claim = [&]() __attribute__((always_inline)) {
    const int v = __hip_atomic_fetch_add(next_block, lane == 0 ? 1 : 0, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_WORKGROUP);
    return __builtin_amdgcn_readfirstlane(v);
  };
  const __amdgpu_buffer_rsrc_t xrs = rw_rsrc(Xq, xq_bytes);
  const __amdgpu_buffer_rsrc_t srs = rw_rsrc(sx, (uint32_t)M * 4u);
  // Lane offset within a 16-token fragment of the tiled layout (row l % 16, chunk l / 16).
  const int xlane = ((lane & 15) << 6) + ((lane >> 4) << 4);
  // Byte offset of block b's k step 0 (panel b / 4, quarter b % 4).
  auto block_base = [](int b) { return (int)((((b >> 2) * NK) << 14) + ((b & 3) << 12)); };
  // Per-lane offsets stay in one register each; everything uniform goes to the scalar offset.
  auto load_step = [&](int base, int kk, v4i (&x)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < 4; b++)
      x[b] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(xrs, xlane,
                                                                          base + (kk << 14) + (b << 10), 0));
  };
  auto read_w = [&](int kk, int a) __attribute__((always_inline)) {
    return *reinterpret_cast<const v4i*>(lds + (kk * NA + a) * 1024 + lane * 16);
  };

  v4i xs[kRwSets][4];
  v4i wf[NA];
  v4i acc[NA][4];
  int base = block_base(rb);
#pragma unroll
  for (int s = 0; s < kRwDepth; s++) load_step(base, s, xs[s]);
#pragma unroll
  for (int a = 0; a < NA; a++) wf[a] = read_w(0, a);
  uint8_t* const stage = lds + S::kWq + wave * S::kStage;
  const int r16 = lane & 15;               // token within a 16-token block (staging row)
  const int hq = lane >> 4;                // which 4 features of a 16-row weight block

  // The epilogue of a block is split up. Right after its k loop, the accumulators are
  // dequantized and packed to fp16/bf16: tokens 0..31 (rounds 0, 1) go straight into this
  // wave's two LDS staging buffers, tokens 32..63 (rounds 2, 3) stay in registers (pk). The
  // outputs then leave during the first four k steps of the wave's next block, one 16-token
  // round per step: (staged from pk,) read back as whole 192-byte row segments, stored after
  // the step's MFMAs. The LDS round trips and the stores thus overlap the next block's MFMAs;
  // the last block's outputs are flushed after the loop.
  static_assert(BN == 96, "the split epilogue stages 96 features per round");
  constexpr int kStoreAux = ACT == kActNone ? 2 : 0;        // bit 1: nt (streaming store)
  uint32_t pk[2][NA][2];
  __amdgpu_buffer_rsrc_t yrs_prev = rw_rsrc(Y, 0);
  auto out_rsrc = [&](int m_base) __attribute__((always_inline)) {
    // Starts at the block's first token and holds only its valid tokens: stores past M drop.
    const int rows_valid = M - m_base < kRwRows ? M - m_base : kRwRows;
    return rw_rsrc(static_cast<uint8_t*>(Y) + (int64_t)m_base * N * kOutBytes,
                   (uint32_t)(rows_valid * N * kOutBytes));
  };
  // Lane l writes, for weight block a, the 8 bytes of features 16 a + 4 (l / 16) .. +3 of token
  // l % 16 into staging buffer q.
  auto stage_write = [&](int q, int a, uint32_t lo, uint32_t hi) __attribute__((always_inline)) {
    const int cc = 2 * a + (hq >> 1);
    *reinterpret_cast<uint2*>(stage + q * S::kBuf + r16 * S::kPitch + stage_pos(cc, r16) * 16 + (hq & 1) * 8) =
        make_uint2(lo, hi);
  };
  // Read back buffer q and store it: the 16 rows x 12 chunks of 16 bytes are 192 chunks, three
  // full 64-lane instructions; chunk f = 64 it + l is chunk f % 12 of row f / 12. Per-lane
  // offsets (LDS and output) are computed once; the round's output offset is scalar.
  int rd_off[3], st_off[3];
#pragma unroll
  for (int it = 0; it < 3; it++) {
    const int f = it * 64 + lane, row = f / 12, j = f - row * 12;
    rd_off[it] = row * S::kPitch + stage_pos(j, row) * 16;
    st_off[it] = n0 + j * 8 < N ? (row * N + n0 + j * 8) * 2 : (int)0x80000000;
  }
  auto stage_read = [&](int q, u32x4 (&v)[3]) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < 3; it++) v[it] = *reinterpret_cast<const u32x4*>(stage + q * S::kBuf + rd_off[it]);
  };
  // Output offsets past every buffer (features past N) are dropped by the hardware, as are
  // rows past the block's valid tokens (the resource's size).
  auto store_round = [&](int r, const u32x4 (&v)[3]) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < 3; it++)
      __builtin_amdgcn_raw_buffer_store_b128(v[it], yrs_prev, st_off[it], r * 16 * N * 2, kStoreAux);
  };
  // Round r of the previous block's outputs, in k step r of the next block (or in the flush):
  // before the step's MFMAs, stage it (rounds 2, 3, from pk) and read it back; after them,
  // store it.
  auto round_read = [&](int r, u32x4 (&v)[3]) __attribute__((always_inline)) {
    if (r >= 2) {
#pragma unroll
      for (int a = 0; a < NA; a++) stage_write(r - 2, a, pk[r - 2][a][0], pk[r - 2][a][1]);
    }
    stage_read(r & 1, v);
  };

  // One 64-token block: 16 k steps, then the dequantization into pk. The first block is peeled
  // off the loop (it has no previous outputs to write), so that both paths into the loop
  // arrive with the same memory operations in flight and the compiler's wait counts at the
  // loop head stay as loose as in the loop.
  auto block = [&](int rb, int rb_next, auto prev_tag) __attribute__((always_inline)) {
    constexpr bool PREV = decltype(prev_tag)::value;
    constexpr bool FIRST = !PREV;                 // the peeled first block of the wave
    // The next block (this one again after the last: harmless in-bounds look-ahead loads).
    const int base_next = block_base(rb_next < rb_hi ? rb_next : rb);
    const int m_base = rb * kRwRows;
    // x_scale of this block's tokens for the epilogue (lane: token 16 b + l % 16; zero past M).
    float xsc[4];
    if constexpr (OUT != kOutS32) {
#pragma unroll
      for (int b = 0; b < 4; b++)
        xsc[b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               srs, r16 * 4, (m_base + b * 16) * 4, 0));
    }
    // k step kk: issue the code loads of step kk + 2 (of the next block in the last two
    // steps), stage round kk of the previous block's outputs (kk < 4), then the 4 NA MFMAs of
    // step kk, each weight fragment re-read for step kk + 1 right after its last MFMA of this
    // step, then store the staged round. The schedule is pinned: the scheduler may not move
    // the loads across steps, and each DS read follows its block's four MFMAs.
#pragma unroll
    for (int kk = 0; kk < NK; kk++) {
      if constexpr (FIRST) {
        if (kk == NK / 2 - 1) {
          // Step 7 reads the weights of step 8: wait for this wave's second half of the
          // copies (vm operations issued after them: the initial look-ahead loads, the
          // x_scale loads when there is an epilogue, and the first NK/2 - 1 steps' code
          // loads), then for every wave's.
          constexpr int kAfter = 4 * kRwDepth + (OUT != kOutS32 ? 4 : 0) + 4 * (NK / 2 - 1);
          __builtin_amdgcn_s_waitcnt(vm_wait(kAfter));
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const int ahead = kk + kRwDepth;
      if (ahead < NK) {
        load_step(base, ahead, xs[ahead & (kRwSets - 1)]);
      } else {
        load_step(base_next, ahead - NK, xs[ahead & (kRwSets - 1)]);
      }
      u32x4 vr[3];
      if constexpr (PREV && OUT != kOutS32) {
        if (kk < 4) round_read(kk, vr);
      }
      __builtin_amdgcn_sched_barrier(0);
      const v4i(&x)[4] = xs[kk & (kRwSets - 1)];
#pragma unroll
      for (int a = 0; a < NA; a++) {
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const v4i c0 = kk == 0 ? v4i{0, 0, 0, 0} : acc[a][b];
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[a], x[b], c0, 0, 0, 0);
        }
        wf[a] = read_w((kk + 1) & (NK - 1), a);
      }
#pragma unroll
      for (int a = 0; a < NA; a++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);     // 4 MFMAs of block a
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // its DS read for step kk + 1
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (PREV && OUT != kOutS32) {
        if (kk < 4) store_round(kk, vr);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // Lane l holds, for block (a, b), D[n][m] at n = 16 a + 4 (l / 16) + e (e = 0..3) and
    // token m = 16 b + l % 16.
    const __amdgpu_buffer_rsrc_t yrs = out_rsrc(m_base);
    if constexpr (OUT == kOutS32) {
#pragma unroll
      for (int b = 0; b < 4; b++)
#pragma unroll
        for (int a = 0; a < NA; a++) {
          const int n = n0 + a * 16 + 4 * hq;
          const int off = n < N ? ((b * 16 + r16) * N + n) * 4 : (int)0x80000000;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[a][b]), yrs, off, 0, 0);
        }
    } else {
      // Dequantize: y = act(fma(f32(acc), fl(w_scale[n] x_scale[m]), bias[n])), then two
      // roundings, binary32 then fp16/bf16 (pack2).
#pragma unroll
      for (int a = 0; a < NA; a++) {
        const int col = a * 16 + 4 * hq;          // n-tile feature of element 0
        const float4 s4 = *reinterpret_cast<const float4*>(e_sw + col);
        const float4 b4 = *reinterpret_cast<const float4*>(e_b + col);
        const float ws[4] = {s4.x, s4.y, s4.z, s4.w};
        const float bs[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int b = 0; b < 4; b++) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; e++)
            y[e] = activate<ACT>(
                __builtin_fmaf(static_cast<float>(acc[a][b][e]), __fmul_rn(ws[e], xsc[b]), bs[e]));
          const uint32_t lo = pack2(y[0], y[1], OUT), hi = pack2(y[2], y[3], OUT);
          if (b < 2) {
            stage_write(b, a, lo, hi);              // rounds 0, 1: straight into LDS
          } else {
            pk[b - 2][a][0] = lo;                   // rounds 2, 3: held until the next block
            pk[b - 2][a][1] = hi;
          }
        }
        // One weight block at a time: hoisting the scale reads of all six would hold 48
        // registers across the conversion.
        __builtin_amdgcn_sched_barrier(0);
      }
      yrs_prev = yrs;
    }
    return base_next;
  };
  int rb_next = claim();
  base = block(rb, rb_next, std::false_type{});
  for (rb = rb_next; rb < rb_hi; rb = rb_next) {
    rb_next = claim();
    base = block(rb, rb_next, std::true_type{});
  }
  if constexpr (OUT != kOutS32) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      u32x4 vr[3];
      round_read(r, vr);
      store_round(r, vr);
    }
  }
}

template <int OUT, int BN>
hipError_t launch_bn(const void* Xq, const float* sx, const void* Wq, const float* sw,
                     const float* bias, int64_t M, int64_t N, void* Y, int act, hipStream_t st) {
  const int NT = (int)((N + BN - 1) / BN);
  const int G = 32 / NT;
  const int rb_total = (int)((M + kRwRows - 1) / kRwRows);
  const int64_t xq_bytes = (M + 255) / 256 * 256 * 1024;
  auto k = act == kActGeluErf ? gemm_rw_kernel<OUT, BN, kActGeluErf>
         : act == kActGeluTanh ? gemm_rw_kernel<OUT, BN, kActGeluTanh>
                               : gemm_rw_kernel<OUT, BN, kActNone>;
  if constexpr (OUT == kOutS32) k = gemm_rw_kernel<OUT, BN, kActNone>;
  hipLaunchKernelGGL(k, dim3(8 * NT * G), dim3(kRwThreads), 0, st, static_cast<const uint8_t*>(Xq), sx,
                     static_cast<const uint8_t*>(Wq), sw, bias, Y, (int)M, (int)N, NT, G, rb_total,
                     (uint32_t)xq_bytes);
  return hipGetLastError();
}

// The n-tile width this kernel uses for N output features, or 0 when it does not take N: 96
// when N is 32 tiles of 96 (one n-tile per CU of an XCD).
int rw_tile(int64_t N) { return N == 32 * 96 ? 96 : 0; }

}  // namespace

bool gemm_rw_supported(int64_t M, int64_t N, int64_t Kb, int bits, bool x_tiled) {
  if (bits != 8 || !x_tiled || Kb != 1024) return false;
  const int bn = rw_tile(N);
  if (bn == 0) return false;
  const int64_t nt = (N + bn - 1) / bn, groups = 32 / nt;
  const int64_t rb_total = (M + kRwRows - 1) / kRwRows;
  // Every wave needs at least one token block of its own; the tiled codes and each block's
  // outputs must fit 32-bit buffer offsets.
  if (rb_total < 8 * groups * kRwWaves) return false;
  return (M + 255) / 256 * 256 * 1024 < (int64_t(1) << 31) && kRwRows * N * 4 < (int64_t(1) << 31);
}

hipError_t launch_gemm_rw(const void* Xq, const float* sx, const void* Wq, const float* sw,
                          const float* bias, int64_t M, int64_t N, void* Y, int out_dt,
                          int32_t* acc32, int act, hipStream_t stream) {
  if (acc32) return launch_bn<kOutS32, 96>(Xq, sx, Wq, sw, bias, M, N, acc32, act, stream);
  if (out_dt == kF16) return launch_bn<kOutF16, 96>(Xq, sx, Wq, sw, bias, M, N, Y, act, stream);
  return launch_bn<kOutBF16, 96>(Xq, sx, Wq, sw, bias, M, N, Y, act, stream);
}

}  // namespace convrot
