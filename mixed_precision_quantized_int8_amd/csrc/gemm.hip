// int8 x int8 -> int32 GEMM on the CDNA4 matrix cores, with the LLM.int8()
// epilogue fused: dequantization by the outer product of the row and column
// scales over 127^2, plus the fp16 product of the outlier columns.
//
// [blog, "Introduction to model quantization"]: vector-wise quantization
// multiplies the int8 matrices and denormalises with the outer product of the
// row absmax of the left operand and the column absmax of the right one.
// [blog, "A gentle summary of LLM.int8()"], steps 2-3, and [blog, "A closer
// look at the MatMul"]: the outlier columns are multiplied in fp16 against the
// matching weight rows and the two parts are added.
//
// Layout: Xq [M][K] and Wq [N][K] are both K-contiguous ("NT"), which is what
// the matrix-core operands want: each lane feeds 16 consecutive k of one row.
//
// Tiling (512 threads = 8 waves of 64, one workgroup per CU, two waves per
// SIMD so that one can issue matrix instructions while the other waits on a
// load or the LDS):
//   * workgroup tile 256 x 256, K step 128 bytes: every load instruction moves
//     8 rows x 128 bytes, whole cache lines (measured: feeding the tile's
//     panels this way is ~30 % faster than with 64-byte rows);
//   * the LDS holds 5 slots of 32 KB, each one operand panel (256 rows x 128
//     bytes) of one K step: while step kt is multiplied, B of step kt+1 and A
//     of step kt+2 are in flight (A of kt+1 was issued one step earlier), so
//     2.5 steps live in the 160 KB; loads go global -> LDS directly
//     (global_load_lds_dwordx4) with explicit vmcnt waits and a fence-free
//     barrier, so they stay in flight across it; past the last step they
//     re-read valid memory into a consumed slot, so the loop body has no
//     branches and the wait counts are fixed;
//   * each wave owns a 128 x 64 sub-tile = 8 x 4 blocks of
//     v_mfma_i32_16x16x64_i8 (128 int32 accumulators per lane).  Both int8
//     shapes run at ~99% of the peak in a sustained loop with all-zero
//     operands, but with random operands the board's power limit holds
//     32x32x32 to 3.3-3.5 POP/s and 16x16x64 to 3.9-4.1 POP/s (measured on
//     MI355X), so the smaller shape does more work per joule;
//   * software pipeline at quarter-step granularity: a 128-byte k-step is two
//     64-byte sub-steps; while the 16 MFMAs of one quarter (one sub-step, half
//     of the A blocks) run, the 4 or 8 fragments of the next quarter are read
//     from LDS into the other of two fixed register sets; reads and loads are
//     placed between the MFMAs with sched_group_barrier;
//   * LDS rows are 128 bytes = eight 16-byte chunks; chunk c of row r is
//     stored at c ^ ((r >> 1) & 7): the bank-conflict counter reads 0 for both
//     fragment patterns (16 consecutive rows per 16 lanes for the int8 loop, 32
//     per half-wave for the fp16 one);
//   * tiles are handed out XCD by XCD: workgroup b runs on XCD b % 8, and each
//     XCD takes a contiguous range of tiles ordered in groups of 8 tile-rows so
//     that concurrently running tiles share operand panels in that XCD's L2.
// Epilogue, one 32x32 block of the wave tile at a time (its four 16x16
// accumulator blocks rearranged into the 32x32 layout through 5 KB of LDS per
// wave): the int32 accumulators of the block are dequantized to fp32 (acc * sx * sw / 127^2),
// then the outlier product is accumulated onto them with
// v_mfma_f32_32x32x16_f16 from X_O [256 x 96] and the matching weight rows
// (transposed to [256 x 96]) staged in LDS once per tile (up to 96 outlier
// columns; beyond that the fragments are read from memory per block), the
// bias is added, and the block is stored as fp16.  The outlier count is read
// from device memory, so no host synchronization is needed.
// Zero-point mode (ZP): Xq holds unsigned codes minus 128 and sx the row's
// range / 255; the accumulators start at (128 - zp[m]) * wsum[n] (the split
// tail adds it to the summed partials), exact in int32 for K within the
// zero-point limit, and are dequantized by sx * sw / 127.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace i8l {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kSlots = 5;                  // LDS slots of one operand panel of one K step
constexpr int kSlot = kBM * kBK;           // 32 KB
constexpr int kGemmThreads = 512;
constexpr int kGroupM = 8;
__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & 7; }

// Tile order: linear tile index -> (tile row, tile column), in groups of
// kGroupM tile rows so that concurrently running tiles share operand panels.
__device__ __forceinline__ void tile_of(int tile, int nTm, int nTn, int& tm, int& tn) {
  const int per_group = kGroupM * nTn;
  const int g = tile / per_group;
  const int first_m = g * kGroupM;
  const int gm = min(nTm - first_m, kGroupM);
  const int in = tile - g * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}
// Workgroup b runs on XCD b % 8: each XCD takes a contiguous range of the
// first `count` tiles, so that its L2 serves neighbouring tiles.
__device__ __forceinline__ int xcd_tile(int bid, int count) {
  const int q = count >> 3, r = count & 7;
  const int xcd = bid & 7, local = bid >> 3;
  return xcd * q + min(xcd, r) + local;
}

// 16 bytes of zeros per lane for K-tail chunks (k >= K): the direct LDS loads
// always write their 16 bytes.
__device__ __attribute__((aligned(64))) int8_t g_zero_page[64];

#define I8L_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt((0xf) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}
// Workgroup barrier without a memory fence (outstanding LDS-DMA loads stay in
// flight); the memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// D layout of a 32x32 MFMA block: lane l holds column l % 32 and, in register
// r, row 8 * (r / 4) + 4 * (l / 32) + r % 4.
__device__ __forceinline__ int d_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
// D layout of a 16x16 MFMA block: lane l holds column l % 16 and, in register
// r, row 4 * (l / 16) + r.
// Per-wave LDS area that turns four 16x16 int32 blocks into the 32x32 layout
// above (rows of kCvS words: lanes 32-63 of a 32x32 read land 32 banks away
// from lanes 0-31).
constexpr int kCvS = 40;
constexpr int kCvWave = 32 * kCvS;   // words per wave

// SPLIT: the workgroups are the split tiles of the tail (S per tile), each on
// its own range of k-steps; they store their int32 partials and end.  FIX
// (with SPLIT): one workgroup per split tile, no main loop, the epilogue on
// the sum of the S partials; a launch of its own, so that the partials are
// visible to it without a fence per workgroup (a device-wide release writes
// the XCD's L2 back: ~60 us per split workgroup, measured).  Separate
// instantiations, so that the whole-tile kernel carries none of this.  ZP:
// zero-point epilogue.  F16: the operands are fp16 instead of int8 (a.K is
// then the row length in BYTES, twice the element count); the same panels,
// ring and fragments feed v_mfma_f32_16x16x32_f16, whose operand layout per
// lane (16 bytes of one row, the four 16-lane groups on consecutive 16-byte
// chunks) is that of the int8 instruction, into fp32 accumulators, stored as
// fp16 (round to nearest even) to a.Y.
template <bool OUT_I32, bool SPLIT, bool ZP, bool FIX = false, bool F16 = false>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_i8_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) int8_t smem[kSlots * kSlot];

  const int M = a.M, N = a.N, K = a.K;
  const int nkt = (K + kBK - 1) / kBK;   // k-steps of 128 bytes
  const int nTm = (M + kBM - 1) / kBM, nTn = (N + kBN - 1) / kBN;
  // Whole tiles first; then the split tiles of the tail, S workgroups each,
  // every one on its own range of k-steps [kb, kb + nk).
  int tile, kb = 0, nk = nkt, slot = -1, sidx = 0;
  if constexpr (!SPLIT) {
    tile = xcd_tile(blockIdx.x, a.full_tiles);
  } else if constexpr (FIX) {
    slot = blockIdx.x;
    tile = a.full_tiles + slot;
  } else {
    slot = blockIdx.x / a.split_S;
    sidx = blockIdx.x % a.split_S;
    tile = a.full_tiles + slot;
    kb = sidx * nkt / a.split_S;
    nk = (sidx + 1) * nkt / a.split_S - kb;
  }
  int tm, tn;
  tile_of(tile, nTm, nTn, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = (wave >> 2) * 128, wn = (wave & 3) * 64;
  const int l32 = lane & 31, lh = lane >> 5;

  // Direct global -> LDS loads.  One instruction moves 64 lanes x 16 bytes into
  // 1 KB of a slot (8 rows of 128 bytes); lane l lands at row 8*blk + l/8,
  // physical chunk l%8, so it fetches the logical chunk (l%8) ^ swz(row).
  // Wave w fills blocks 4w .. 4w+3 of a slot: 4 loads per operand and step.
  // Rows past M (or N) are clamped to the last row: they only feed outputs
  // that are never stored.  K-tail chunks read zeros from a device zero page.
  // Every address stays inside the operands.
  uint32_t rowA[4], rowB[4];   // byte offset of the (clamped) row inside the tile
  int cofs[4];                 // byte offset of the lane's logical 16-byte chunk
  const int lastA = min(M - m0, kBM) - 1, lastB = min(N - n0, kBN) - 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wave * 4 + i) * 8 + (lane >> 3);
    cofs[i] = ((lane & 7) ^ lds_swz(row)) * 16;
    rowA[i] = (uint32_t)(min(row, lastA) * K);
    rowB[i] = (uint32_t)(min(row, lastB) * K);
  }
  const int8_t* tileA = a.Xq + (size_t)m0 * K;
  const int8_t* tileB = a.Wq + (size_t)n0 * K;
  // Load i (0..3) of one operand of step kt into slot `sl`; branch-free so that
  // it can be placed between the MFMAs (K-tail chunks select the zero page).
  auto load = [&](int sl, int kt, bool isB, int i) {   // kt: step inside [kb, kb + nk)
    const int kk = (kb + kt) * kBK + cofs[i];
    const bool in = kk < K;
    const int8_t* g = in ? (isB ? tileB + rowB[i] : tileA + rowA[i]) + kk : g_zero_page;
    __builtin_amdgcn_global_load_lds((const void*)g, I8L_LDS(&smem[sl * kSlot + (wave * 4 + i) * 1024]),
                                     16, 0, 0);
  };
  // Step kt's A panel sits in slot (2 kt) % 5 and its B panel in (2 kt + 1) % 5.

  // Accumulators: 8 x 4 blocks of v_mfma_i32_16x16x64_i8 (F16:
  // v_mfma_f32_16x16x32_f16), 16 x 16 each; block (ia, jb) covers rows
  // wm + 16 ia, features wn + 16 jb.  Measured on MI355X with random operands
  // in a sustained loop: the 16x16 shapes reach 3.9-4.1 POP/s (int8) and 1.90
  // PFLOP/s (fp16) against 3.3-3.5 and 1.67 for the 32x32 ones (all ~99 % of
  // the peak with all-zero operands): under the board's power limit they do
  // more work per joule.
  constexpr int kAI = 8, kAJ = 4;
  typedef typename std::conditional<F16, v4f, v4i>::type blk_t;
  blk_t acc[kAI][kAJ];
#pragma unroll
  for (int i = 0; i < kAI; ++i)
#pragma unroll
    for (int j = 0; j < kAJ; ++j) acc[i][j] = blk_t{};
  if constexpr (ZP && !SPLIT && !F16) {
    // Zero-point correction as the accumulators' starting value: the MFMAs then
    // add sum_k (q - 128) w on top.  Every prefix sum stays within
    // 255 * 127 * K < 2^31 in magnitude, so nothing wraps.  Rows past M read 0
    // from the buffer resource (never stored).
    const buf_rsrc rz = make_rsrc(a.zp, (uint32_t)M * 4u);
    uint32_t wsv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + j * 16 + (lane & 15);
      wsv[j] = n < N ? (uint32_t)a.wsum[n] : 0u;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const v4i z = buf_load16(rz, (uint32_t)(m0 + wm + i * 16 + 4 * (lane >> 4)) * 4u);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = (int)((128u - (uint32_t)z[r]) * wsv[j]);
    }
  }
  // Scheduling masks for __builtin_amdgcn_sched_group_barrier.
  constexpr int kSchedMFMA = 0x008, kSchedVMEMRead = 0x020, kSchedDSRead = 0x100;

  if constexpr (!FIX) {
  // Main loop on v_mfma_i32_16x16x64_i8 (F16: v_mfma_f32_16x16x32_f16, whose
  // operand is also 16 bytes of one row per lane).  A 128-byte k-step is two
  // 64-byte sub-steps s; the operand of lane l is 16 bytes of row l % 16 at
  // logical chunk 4 s + l / 16 (the same chunk in A and B, so the products pair
  // the same k).  Quarter q of a step: sub-step q / 2, A blocks 4 (q % 2) .. +3, all
  // four B blocks: 16 MFMAs on 4 A and 4 B fragments.  Register sets: A in
  // fa0 / fa1 (even / odd quarters), B in fb0 / fb1 (sub-step 0 / 1).
  auto read_a = [&](int kt, int s, int h, v4i (&fa)[4]) {
    const int8_t* sA = &smem[((2 * kt) % kSlots) * kSlot];
    const int c = 4 * s + (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm + (4 * h + i) * 16 + (lane & 15);
      fa[i] = *reinterpret_cast<const v4i*>(&sA[row * kBK + ((c ^ lds_swz(row)) << 4)]);
    }
  };
  auto read_b = [&](int kt, int s, v4i (&fb)[4]) {
    const int8_t* sB = &smem[((2 * kt + 1) % kSlots) * kSlot];
    const int c = 4 * s + (lane >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn + j * 16 + (lane & 15);
      fb[j] = *reinterpret_cast<const v4i*>(&sB[row * kBK + ((c ^ lds_swz(row)) << 4)]);
    }
  };
  // MFMA e (0..15) of a quarter with A set h: A block 4 h + e / 4, B block e % 4
  auto mfma16 = [&](const v4i (&fa)[4], const v4i (&fb)[4], int h, int e) {
    const int i = e >> 2, j = e & 3;
    if constexpr (F16)
      acc[4 * h + i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          __builtin_bit_cast(v8h, fa[i]), __builtin_bit_cast(v8h, fb[j]), acc[4 * h + i][j], 0, 0, 0);
    else
      acc[4 * h + i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[4 * h + i][j], 0, 0, 0);
  };
  // 16 MFMAs with 4 fragment reads and 2 loads between them
  auto pattern_4r = [&]() {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVMEMRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 3, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // 16 MFMAs with 8 fragment reads and 2 loads between them
  auto pattern_8r = [&]() {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVMEMRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 3, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Slot schedule (5 slots, steps of two panels).  During iteration kt: step
  // kt is read from slots 2kt, 2kt+1; A of kt+1 (slot 2kt+2) was issued during
  // iteration kt-1; B of kt+1 goes to slot 2kt+3 (quarters 0-1) and A of kt+2
  // to slot 2kt+4 (quarters 2-3), all mod 5.  Slots 2kt+3 and 2kt+4 held step
  // kt-1, which every wave finished reading before the previous barrier.  The
  // barrier at the end of iteration kt needs step kt+1 complete: issued after
  // its last load are only the four A loads of kt+2, so vmcnt(4).  (Measured:
  // ~10 % faster than issuing two of the A loads after the barrier.)
  load(0, 0, false, 0); load(0, 0, false, 1); load(0, 0, false, 2); load(0, 0, false, 3);
  load(1, 0, true, 0); load(1, 0, true, 1); load(1, 0, true, 2); load(1, 0, true, 3);
  {
    const int k1 = min(1, nk - 1);
    load(2, k1, false, 0); load(2, k1, false, 1); load(2, k1, false, 2); load(2, k1, false, 3);
  }
  wait_vmcnt<4>();   // step 0 landed; A of step 1 may be in flight
  lds_barrier();

  v4i fa0[4], fa1[4], fb0[4], fb1[4];
  read_a(0, 0, 0, fa0);
  read_b(0, 0, fb0);
  for (int kt = 0; kt < nk; ++kt) {
    const int slB = (2 * kt + 3) % kSlots, slA = (2 * kt + 4) % kSlots;
    const int kB = min(kt + 1, nk - 1), kA = min(kt + 2, nk - 1);
    // ---- quarter 0 (sub-step 0, A 0-3): reads A 4-7 of sub-step 0; B loads 0-1
    wait_lgkmcnt0();
    read_a(kt, 0, 1, fa1);
    load(slB, kB, true, 0);
    load(slB, kB, true, 1);
#pragma unroll
    for (int e = 0; e < 16; ++e) mfma16(fa0, fb0, 0, e);
    pattern_4r();
    // ---- quarter 1 (sub-step 0, A 4-7): reads A 0-3 and B of sub-step 1; B loads 2-3
    wait_lgkmcnt0();
    read_a(kt, 1, 0, fa0);
    read_b(kt, 1, fb1);
    load(slB, kB, true, 2);
    load(slB, kB, true, 3);
#pragma unroll
    for (int e = 0; e < 16; ++e) mfma16(fa1, fb0, 1, e);
    pattern_8r();
    // ---- quarter 2 (sub-step 1, A 0-3): reads A 4-7 of sub-step 1; A loads 0-1 of kt+2
    wait_lgkmcnt0();
    read_a(kt, 1, 1, fa1);
    load(slA, kA, false, 0);
    load(slA, kA, false, 1);
#pragma unroll
    for (int e = 0; e < 16; ++e) mfma16(fa0, fb1, 0, e);
    pattern_4r();
    // ---- quarter 3 (sub-step 1, A 4-7): 12 of the 16 MFMAs go out before the
    // wait and the barrier, so the matrix pipe is busy while the waves
    // synchronize; then the reads of the next step's first quarter between
    // the last four (swept on MI355X: 4, 8, 12, 14, 16 before the barrier;
    // 12 best, ~1 % over 8 and ~4 % over 4)
    wait_lgkmcnt0();
    load(slA, kA, false, 2);
    load(slA, kA, false, 3);
#pragma unroll
    for (int e = 0; e < 12; ++e) mfma16(fa1, fb1, 1, e);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<4>();
    lds_barrier();
    // Step kt+1 is in every wave's view and step kt's slots are free.  On the
    // last step the fragment reads re-read step kt (landed, unused), so that
    // the registers keep fixed roles.
    {
      const int kn = kt + 1 < nk ? kt + 1 : kt;
      read_a(kn, 0, 0, fa0);
      read_b(kn, 0, fb0);
    }
#pragma unroll
    for (int e = 12; e < 16; ++e) mfma16(fa1, fb1, 1, e);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  }   // !FIX
  __syncthreads();   // all waves done with the ring before the epilogue reuses it

  // The values of 32x32 region (i, j) of the wave tile in the 32x32 D layout
  // (int8: the exact int32 sums), from its four 16x16 blocks (2i + bi, 2j + bj), through
  // the wave's kCvWave words of LDS at cv (the epilogue below is written for
  // that layout).
  auto to32 = [&](int* cv, int i, int j, int (&tot)[16]) {   // F16: fp32 bit patterns
    {
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // (element r taken as a value first: __builtin_bit_cast applied to
            // the vector subscript itself read element 0 for every r)
            int* dst = &cv[(16 * bi + 4 * (lane >> 4) + r) * kCvS + 16 * bj + (lane & 15)];
            if constexpr (F16) {
              const float v = acc[2 * i + bi][2 * j + bj][r];
              *dst = __float_as_int(v);
            } else {
              *dst = acc[2 * i + bi][2 * j + bj][r];
            }
          }
      // the wave's LDS writes before its reads of other lanes' values
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int r = 0; r < 16; ++r) tot[r] = cv[d_row(r, lane) * kCvS + l32];
      // the reads done before the area is written again
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  };

  if constexpr (F16) {
    // fp16 output, one 32x32 block at a time (rearranged by to32, then through
    // the same LDS area in row order) and out as 16-byte row pieces when
    // N % 8 == 0, else element by element
    constexpr int kTS = 40;
    int* cv = reinterpret_cast<int*>(&smem[0]) + wave * kCvWave;
    uint16_t* sT = reinterpret_cast<uint16_t*>(cv);
    const bool vec_store = (N & 7) == 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn + j * 32 + l32;
        int tb[16];
        to32(cv, i, j, tb);
        if (vec_store) {   // uniform
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sT[d_row(r, lane) * kTS + l32] = f2h(__int_as_float(tb[r]));
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          const int row = lane >> 1, c0 = (lane & 1) * 16;
          const v4i p0 = *reinterpret_cast<const v4i*>(&sT[row * kTS + c0]);
          const v4i p1 = *reinterpret_cast<const v4i*>(&sT[row * kTS + c0 + 8]);
          const int m = m0 + wm + i * 32 + row;
          const int nb = n0 + wn + j * 32 + c0;
          if (m < M) {
            if (nb < N) *reinterpret_cast<v4i*>(&a.Y[(size_t)m * N + nb]) = p0;
            if (nb + 8 < N) *reinterpret_cast<v4i*>(&a.Y[(size_t)m * N + nb + 8]) = p1;
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        } else if (n < N) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm + i * 32 + d_row(r, lane);
            if (m < M) a.Y[(size_t)m * N + n] = f2h(__int_as_float(tb[r]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    return;
  }

  if constexpr (SPLIT && !FIX) {
    // Split tile: store this K range's int32 partial and end; the fix-up
    // launch sums the S partials (exact integer sums, in any order).  The
    // partial is kept in register-fragment order (16-byte piece q of thread
    // t's values of block (i, j) at ((i*2 + j)*4 + q)*512 + t): the fix-up
    // workgroup has the same fragment layout, so each store and each read
    // covers 1 KB contiguous per wave.
    constexpr int kTile = kBM * kBN;
    v4i* mine = reinterpret_cast<v4i*>(a.part + (size_t)(slot * a.split_S + sidx) * kTile);
    int* cv = reinterpret_cast<int*>(&smem[0]) + wave * kCvWave;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        int tot[16];
        to32(cv, i, j, tot);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          mine[((i * 2 + j) * 4 + q) * kGemmThreads + t] =
              v4i{tot[4 * q], tot[4 * q + 1], tot[4 * q + 2], tot[4 * q + 3]};
        __builtin_amdgcn_sched_barrier(0);
      }
    return;
  }

  // Exact int32 value of fragment (i, j): the accumulators of a whole tile,
  // or, in the fix-up of a split tile, the sum of its S partials, read four at
  // a time with every load unconditional (partials past S read zero from the
  // range check), so that they are in flight together.
  auto tile_sum = [&](int* cv, int i, int j, int (&tot)[16]) {
    if constexpr (SPLIT) {
      constexpr int kTile = kBM * kBN;
      const buf_rsrc rp = make_rsrc(a.part + (size_t)slot * a.split_S * kTile,
                                    (uint32_t)(a.split_S * kTile * 4));
      const uint32_t fo = (uint32_t)(((i * 2 + j) * 4 * kGemmThreads + t) * 16);
#pragma unroll
      for (int r = 0; r < 16; ++r) tot[r] = 0;
      for (int s2 = 0; s2 < a.split_S; s2 += 4) {   // uniform
        v4i p[4][4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            p[k][q] = buf_load16(rp, (uint32_t)((s2 + k) * kTile * 4) + fo +
                                         (uint32_t)(q * kGemmThreads * 16));
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) tot[4 * q + e] += p[k][q][e];
      }
    } else {
      to32(cv, i, j, tot);
    }
  };

  if constexpr (OUT_I32) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn + j * 32 + l32;
        int tot[16];
        tile_sum(reinterpret_cast<int*>(&smem[0]) + wave * kCvWave, i, j, tot);
        if (n >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm + i * 32 + d_row(r, lane);
          if (m < M) a.acc[(size_t)m * N + n] = tot[r];
        }
      }
    return;
  } else {
    // Epilogue, one 32x32 block of the wave tile at a time (16 values per lane
    // live, so the accumulators can stay in the accumulation registers): the
    // int32 block is dequantized to fp32 (acc * sx[m] * sw[n] / 127^2), the
    // outlier product is accumulated onto it by the fp16 matrix cores from
    // X_O and the matching weight rows staged in LDS, and it is stored as fp16.
    // Up to kOutG outlier columns are staged once per tile; beyond that the
    // fragments are read straight from memory per block (correct, slower;
    // such inputs are rare).
    constexpr int kOutG = 96;                  // 3 chunks of 32 outlier columns
    constexpr int kOutC = kOutG / 8;           // 16-byte chunks per staged row
    const int n_out = *a.n_out;
    const int ngroups = (n_out + kOutG - 1) / kOutG;
    uint16_t* sAo = reinterpret_cast<uint16_t*>(&smem[0]);         // [256 rows][96 halves]
    uint16_t* sBo = sAo + kBM * kOutG;                             // [256 cols][96 halves]
    float* sSx = reinterpret_cast<float*>(sBo + kBN * kOutG);      // [256]
    float* sSw = sSx + kBM;                                        // [256], includes 1/127^2
    float* sBias = sSw + kBN;                                      // [256] (0 without bias)
    int* sZc = reinterpret_cast<int*>(sBias + kBN);                // [256] 128 - zp (ZP)
    int* sWs = sZc + kBM;                                          // [256] wsum (ZP)
    // Per wave, kCvWave words: first the int32 conversion of a 32x32 region
    // (to32), then the same block as fp16 in row order (kTS halves per row),
    // so that Y goes out in 16-byte row pieces instead of 2-byte column values.
    constexpr int kTS = 40;
    int* cvY = reinterpret_cast<int*>(sWs + kBN) + wave * kCvWave;
    uint16_t* sT = reinterpret_cast<uint16_t*>(cvY);
    static_assert(32 * kTS * 2 <= kCvWave * 4, "fp16 staging must fit the conversion area");
    static_assert(2 * kBM * kOutG * 2 + 5 * 256 * 4 + kGemmThreads / 64 * kCvWave * 4 <=
                      (int)sizeof(smem),
                  "epilogue staging must fit the LDS");
    // N % 8 == 0: every 8-column piece of a row lies wholly inside or outside
    // N and starts 16-byte aligned (Y is 16-byte aligned)
    const bool vec_store = (N & 7) == 0;
    // 16-byte chunk c of staged row r sits at c ^ ((r >> 2) & 3): conflict-free
    // fragment reads with the 192-byte row stride
    auto och = [](int r, int c) { return (c ^ ((r >> 2) & 3)) << 3; };
    if (t < kBM) {   // 512 threads: the first half fills the row/column tables
      sSx[t] = m0 + t < M ? a.sx[m0 + t] : 0.0f;
      sSw[t] = n0 + t < N ? a.sw[n0 + t] * (ZP ? 1.0f / 127.0f : 1.0f / 16129.0f) : 0.0f;
      sBias[t] = a.bias && n0 + t < N ? h2f(a.bias[n0 + t]) : 0.0f;
    } else if constexpr (ZP) {
      const int u = t - kBM;
      sZc[u] = m0 + u < M ? 128 - a.zp[m0 + u] : 0;
      sWs[u] = n0 + u < N ? a.wsum[n0 + u] : 0;
    }

    // fp16 bits of the outlier weight W[k][n]: the caller's fp16 row, or, with
    // W_rows NULL, rebuilt from the code Wq[n][k] and sw[n]
    auto wbits = [&](int k, int n) -> uint32_t {
      return a.W_rows ? (uint32_t)a.W_rows[(size_t)k * N + n]
                      : (uint32_t)dequant_w16(a.Wq[(size_t)n * K + k], a.sw[n]);
    };
    // X_O[., 0 .. 96) and rows idx[0 .. 96) of W (transposed to
    // [column][outlier]); zero past n_out and outside the matrix.  All loads
    // go out before any store and none sits behind a branch (X_O rows past
    // the tile read 0 from the buffer resource; indices past n_out read entry
    // 0 and are masked), so the staging costs about one memory round trip.
    auto stage_outliers = [&]() {
      constexpr int kPerT = kBM * kOutC / kGemmThreads;   // X_O chunks per thread
      const int rows = min(M - m0, kBM);
      const buf_rsrc rxo = make_rsrc(a.X_O + (size_t)m0 * K, (uint32_t)rows * (uint32_t)K * 2u);
      v4i xv[kPerT];
#pragma unroll
      for (int i = 0; i < kPerT; ++i) {
        const int q = t + i * kGemmThreads, row = q / kOutC, c = q % kOutC;
        xv[i] = buf_load16(rxo, (uint32_t)(row * K + c * 8) * 2u);
      }
      const int col = t & (kBN - 1);   // 512 threads: two per column, half the chunks each
      const int gn = n0 + col, gnc = gn < N ? gn : N - 1;
      const float sn = a.W_rows ? 0.0f : a.sw[gnc];
      // the thread's 6 chunks of 8 outlier rows in two passes of 3 (bounded
      // registers; the X_O loads above are still in flight during the first)
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int cb = (t >> 8) * (kOutC / 2) + pass * (kOutC / 4);
        uint32_t hv[kOutC / 4][8];
        if (a.W_rows) {   // uniform
#pragma unroll
          for (int ci = 0; ci < kOutC / 4; ++ci)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int j = (cb + ci) * 8 + e;
              hv[ci][e] = a.W_rows[(size_t)a.idx[j < n_out ? j : 0] * N + gnc];
            }
        } else {
#pragma unroll
          for (int ci = 0; ci < kOutC / 4; ++ci)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int j = (cb + ci) * 8 + e;
              hv[ci][e] = dequant_w16(a.Wq[(size_t)gnc * K + a.idx[j < n_out ? j : 0]], sn);
            }
        }
        if (pass == 0) {
#pragma unroll
          for (int i = 0; i < kPerT; ++i) {
            const int q = t + i * kGemmThreads, row = q / kOutC, c = q % kOutC;
            const int nv = n_out - c * 8;   // valid halves of this chunk
            v4i v = xv[i];
#pragma unroll
            for (int d = 0; d < 4; ++d)
              v[d] &= (int)((2 * d < nv ? 0xffffu : 0u) | (2 * d + 1 < nv ? 0xffff0000u : 0u));
            *reinterpret_cast<v4i*>(&sAo[row * kOutG + och(row, c)]) = v;
          }
        }
#pragma unroll
        for (int ci = 0; ci < kOutC / 4; ++ci) {
          uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = (cb + ci) * 8 + e;
            const uint32_t h = (j < n_out && gn < N) ? (hv[ci][e] & 0xffffu) : 0u;
            w[e >> 1] |= h << ((e & 1) * 16);
          }
          *reinterpret_cast<v4i*>(&sBo[col * kOutG + och(col, cb + ci)]) =
              v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        }
      }
    };
    if (ngroups == 1) stage_outliers();
    __syncthreads();

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float sxv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {   // rows 8q + 4*lh .. +3 of block i are contiguous
        const v4f v = *reinterpret_cast<const v4f*>(&sSx[wm + i * 32 + 8 * q + 4 * lh]);
#pragma unroll
        for (int e = 0; e < 4; ++e) sxv[4 * q + e] = v[e];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn + j * 32 + l32;
        const float swv = sSw[wn + j * 32 + l32];
        int tot[16];
        tile_sum(cvY, i, j, tot);
        if constexpr (ZP && SPLIT) {   // sum (q - zp) w = sum (q - 128) w + (128 - zp) S[n], mod 2^32
          const uint32_t wsv = (uint32_t)sWs[wn + j * 32 + l32];
#pragma unroll
          for (int r = 0; r < 16; ++r)
            tot[r] = (int)((uint32_t)tot[r] + (uint32_t)sZc[wm + i * 32 + d_row(r, lane)] * wsv);
        }
        v16f y;
#pragma unroll
        for (int r = 0; r < 16; ++r) y[r] = (float)tot[r] * (sxv[r] * swv);
        if (ngroups == 1) {   // uniform: staged fragments
          for (int cc = 0; cc < 3 && cc * 32 < n_out; ++cc) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int row = wm + i * 32 + l32, col = wn + j * 32 + l32;
              const int c = cc * 4 + 2 * h + lh;
              const v8h fa = *reinterpret_cast<const v8h*>(&sAo[row * kOutG + och(row, c)]);
              const v8h fb = *reinterpret_cast<const v8h*>(&sBo[col * kOutG + och(col, c)]);
              y = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, fb, y, 0, 0, 0);
            }
          }
        } else if (ngroups > 1) {   // many outliers: fragments straight from memory
          const int gm = m0 + wm + i * 32 + l32;
          for (int j0 = 0; j0 < n_out; j0 += 16) {
            const int jb = j0 + 8 * lh;
            uint32_t wa[4] = {0, 0, 0, 0}, wb[4] = {0, 0, 0, 0};
            for (int e = 0; e < 8; ++e) {
              const int jj = jb + e;
              if (jj < n_out) {
                if (gm < M) wa[e >> 1] |= (uint32_t)a.X_O[(size_t)gm * K + jj] << ((e & 1) * 16);
                if (n < N) wb[e >> 1] |= wbits(a.idx[jj], n) << ((e & 1) * 16);
              }
            }
            const v8h fa = __builtin_bit_cast(v8h, v4i{(int)wa[0], (int)wa[1], (int)wa[2], (int)wa[3]});
            const v8h fb = __builtin_bit_cast(v8h, v4i{(int)wb[0], (int)wb[1], (int)wb[2], (int)wb[3]});
            y = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, fb, y, 0, 0, 0);
          }
        }
        if (vec_store) {   // uniform
          const float bv = sBias[wn + j * 32 + l32];   // 0 past N
#pragma unroll
          for (int r = 0; r < 16; ++r) sT[d_row(r, lane) * kTS + l32] = f2h(y[r] + bv);
          // the wave's LDS writes before its reads of other lanes' values
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          const int row = lane >> 1, c0 = (lane & 1) * 16;
          const v4i p0 = *reinterpret_cast<const v4i*>(&sT[row * kTS + c0]);
          const v4i p1 = *reinterpret_cast<const v4i*>(&sT[row * kTS + c0 + 8]);
          const int m = m0 + wm + i * 32 + row;
          const int nb = n0 + wn + j * 32 + c0;
          if (m < M) {
            if (nb < N) *reinterpret_cast<v4i*>(&a.Y[(size_t)m * N + nb]) = p0;
            if (nb + 8 < N) *reinterpret_cast<v4i*>(&a.Y[(size_t)m * N + nb + 8]) = p1;
          }
          // the reads done before the next block overwrites the wave's rows
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        } else if (n < N) {
          const float bv = sBias[wn + j * 32 + l32];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm + i * 32 + d_row(r, lane);
            if (m < M) a.Y[(size_t)m * N + n] = f2h(y[r] + bv);
          }
        }
        __builtin_amdgcn_sched_barrier(0);   // one block at a time: bounded live ranges
      }
    }
  }
}

GemmSplit gemm_split_plan(int M, int N, int K, int cus) {
  const int nTm = (M + kBM - 1) / kBM, nTn = (N + kBN - 1) / kBN;
  const int T = nTm * nTn, nk = (K + kBK - 1) / kBK;
  GemmSplit p{T, 0, 1};
  if (cus <= 0 || T <= 0) return p;
  const int rem = T % cus;
  // Any partial last round is split (when at least two splits fit): with the
  // fix-up launch, splitting QKV's quarter-full last round (64 tiles, 4 ways)
  // measured 1.22 -> 1.17 ms per call.
  if (rem == 0) return p;
  // each split keeps at least 1024 bytes of K (8 k-steps), so the fix-up
  // stays a small part
  const int S = std::min(cus / rem, nk / 8);
  if (S < 2) return p;
  return GemmSplit{T - rem, rem, S};
}

namespace {
// Per-device compute-unit count, queried once (0: not yet, -1: unknown).
// Atomic, since callers may launch from several host threads.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    c = n > 0 ? n : -1;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c > 0 ? std::min(c, kGemmMaxSlices) : 0;
}
}  // namespace

hipError_t launch_gemm(const GemmArgs& in, hipStream_t stream) {
  GemmArgs a = in;
  const int nTm = (a.M + kBM - 1) / kBM, nTn = (a.N + kBN - 1) / kBN;
  GemmSplit p{nTm * nTn, 0, 1};
  if (a.part && a.part_slices > 0) {
    const GemmSplit q = gemm_split_plan(a.M, a.N, a.K, device_cus());
    if (q.split_tiles > 0 && q.split_tiles * q.S <= a.part_slices) p = q;
  }
  a.full_tiles = p.full_tiles;
  a.split_S = p.S;
  if (a.acc) {   // int32 output: the same tiles, splits and fix-up sums as for Y
    if (p.full_tiles > 0)
      hipLaunchKernelGGL((gemm_i8_kernel<true, false, false>), dim3(p.full_tiles),
                         dim3(kGemmThreads), 0, stream, a);
    if (p.split_tiles > 0) {
      hipLaunchKernelGGL((gemm_i8_kernel<true, true, false>), dim3(p.split_tiles * p.S),
                         dim3(kGemmThreads), 0, stream, a);
      hipLaunchKernelGGL((gemm_i8_kernel<true, true, false, true>), dim3(p.split_tiles),
                         dim3(kGemmThreads), 0, stream, a);
    }
    return hipGetLastError();
  }
  // whole tiles, then the split tail (both launches fill the chip)
  const bool zp = a.zp != nullptr;
  if (p.full_tiles > 0) {
    if (zp)
      hipLaunchKernelGGL((gemm_i8_kernel<false, false, true>), dim3(p.full_tiles),
                         dim3(kGemmThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_i8_kernel<false, false, false>), dim3(p.full_tiles),
                         dim3(kGemmThreads), 0, stream, a);
  }
  if (p.split_tiles > 0) {   // the split tiles' partials, then their fix-up
    if (zp) {
      hipLaunchKernelGGL((gemm_i8_kernel<false, true, true>), dim3(p.split_tiles * p.S),
                         dim3(kGemmThreads), 0, stream, a);
      hipLaunchKernelGGL((gemm_i8_kernel<false, true, true, true>), dim3(p.split_tiles),
                         dim3(kGemmThreads), 0, stream, a);
    } else {
      hipLaunchKernelGGL((gemm_i8_kernel<false, true, false>), dim3(p.split_tiles * p.S),
                         dim3(kGemmThreads), 0, stream, a);
      hipLaunchKernelGGL((gemm_i8_kernel<false, true, false, true>), dim3(p.split_tiles),
                         dim3(kGemmThreads), 0, stream, a);
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemm_f16(const uint16_t* A, const uint16_t* B, int M, int N, int K,
                           uint16_t* C, hipStream_t stream) {
  GemmArgs a{};
  a.Xq = reinterpret_cast<const int8_t*>(A);
  a.Wq = reinterpret_cast<const int8_t*>(B);
  a.M = M;
  a.N = N;
  a.K = 2 * K;   // bytes per row
  a.Y = C;
  const int tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  a.full_tiles = tiles;
  a.split_S = 1;
  hipLaunchKernelGGL((gemm_i8_kernel<false, false, false, false, true>), dim3(tiles),
                     dim3(kGemmThreads), 0, stream, a);
  return hipGetLastError();
}

const char* gemm_tile_info() {
  return "gemm: 256x256x128 tile, 5-slot LDS-DMA ring, 8 waves of 128x64, "
         "v_mfma_i32_16x16x64_i8, v_mfma_f32_32x32x16_f16 outlier tail";
}

}  // namespace i8l
