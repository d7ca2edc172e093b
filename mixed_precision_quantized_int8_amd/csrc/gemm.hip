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
// Tiling (256 threads = 4 waves of 64, one workgroup per CU):
//   workgroup tile 256 x 256, K step 64 bytes; a 4-stage LDS ring (128 KB) fed
//   by direct global->LDS loads (global_load_lds_dwordx4), three stages ahead;
//   each wave owns a 128 x 128 sub-tile = 8 x 8 blocks of v_mfma_i32_16x16x64_i8
//   whose 256 int32 accumulators per lane live in the accumulation registers.
//   LDS rows are 64 bytes = four 16-byte chunks; chunk c of row r is stored at
//   c ^ (((r >> 1) ^ (r >> 3)) & 3), so the 16-byte fragment reads of 8 or 16
//   consecutive rows fall into distinct banks.
//   Tiles are handed out XCD by XCD: workgroup b runs on XCD b % 8, and each
//   XCD takes a contiguous range of tiles ordered in groups of 8 tile-rows so
//   that concurrently running tiles share operand panels in that XCD's L2.
// Epilogue, one 16-column block of the wave tile at a time: the int32
// accumulators of the block are dequantized to fp32 (acc * sx * sw / 127^2),
// then the outlier product is accumulated onto them with
// v_mfma_f32_16x16x32_f16 from X_O[256 x 32] and the matching 32 weight rows
// (transposed to [256 x 32]) staged in LDS, and the block is stored as fp16.
// With at most 32 outlier columns the staging happens once per tile.  The
// outlier count is read from device memory, so no host synchronization is
// needed.
#include "common.h"
#include "launch.h"

namespace i8l {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kGemmThreads = 256;
constexpr int kGroupM = 8;
constexpr int kStages = 4;   // LDS ring depth (32 KB per stage)

__device__ __forceinline__ int lds_swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

// Tile assignment: contiguous tile ranges per XCD, grouped order inside.
__device__ __forceinline__ void tile_coords(int bid, int nTm, int nTn, int& tm, int& tn) {
  const int T = nTm * nTn;
  const int q = T >> 3, r = T & 7;
  const int xcd = bid & 7, local = bid >> 3;
  const int tile = xcd * q + min(xcd, r) + local;
  const int per_group = kGroupM * nTn;
  const int g = tile / per_group;
  const int first_m = g * kGroupM;
  const int gm = min(nTm - first_m, kGroupM);
  const int in = tile - g * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

#define I8L_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}
// Workgroup barrier without a memory fence (outstanding LDS-DMA loads stay in
// flight); the memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <bool OUT_I32>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_i8_kernel(GemmArgs a) {
  // kStages ring buffers of [A 256 x 64 | B 256 x 64] bytes
  __shared__ __attribute__((aligned(1024))) int8_t smem[kStages][2][kBM * kBK];

  const int M = a.M, N = a.N, K = a.K;
  const int nTm = (M + kBM - 1) / kBM, nTn = (N + kBN - 1) / kBN;
  int tm, tn;
  tile_coords(blockIdx.x, nTm, nTn, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  const int l16 = lane & 15, lg = lane >> 4;

  // Direct global -> LDS loads.  One instruction moves 64 lanes x 16 bytes into
  // 1 KB of LDS (16 rows of 64 bytes); lane l lands at row 16*blk + l/4,
  // physical chunk l%4, so it fetches the logical chunk (l%4) ^ swz(row).
  // Wave w fills blocks 4w .. 4w+3 of A and of B: 8 loads per stage.
  // Rows past M (or N) are clamped to the last row: they only feed outputs
  // that are never stored.  K-tail chunks are zeroed in LDS (zero_k_tail).
  // Every address stays inside the operand.
  uint32_t rowA[4], rowB[4];   // byte offset of the (clamped) row inside the tile
  int cofs[4];                 // byte offset of the lane's logical 16-byte chunk
  const int lastA = min(M - m0, kBM) - 1, lastB = min(N - n0, kBN) - 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wave * 4 + i) * 16 + (lane >> 2);
    cofs[i] = ((lane & 3) ^ lds_swz(row)) * 16;
    rowA[i] = (uint32_t)(min(row, lastA) * K);
    rowB[i] = (uint32_t)(min(row, lastB) * K);
  }
  const int8_t* tileA = a.Xq + (size_t)m0 * K;
  const int8_t* tileB = a.Wq + (size_t)n0 * K;
  auto issue = [&](int stage, int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // a chunk past K reads the row's first chunk instead (stays inside the
      // operand); zero_k_tail overwrites it in LDS
      const int kk = k0 + cofs[i] < K ? k0 + cofs[i] : 0;
      __builtin_amdgcn_global_load_lds((const void*)(tileA + rowA[i] + kk),
                                       I8L_LDS(&smem[stage][0][(wave * 4 + i) * 1024]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(tileB + rowB[i] + kk),
                                       I8L_LDS(&smem[stage][1][(wave * 4 + i) * 1024]), 16, 0, 0);
    }
  };
  // Last stage when K % 64 != 0: the chunks at k >= K hold a copy of the
  // row's first chunk; replace them by zeros.
  const int ktail = K % kBK;
  auto zero_k_tail = [&](int stage) {
    for (int q = t; q < 2 * kBM * 4; q += kGemmThreads) {
      const int op = q / (kBM * 4), row = (q / 4) % kBM, c = q & 3;
      if (c * 16 >= ktail)
        *reinterpret_cast<v4i*>(&smem[stage][op][row * kBK + ((c ^ lds_swz(row)) << 4)]) =
            v4i{0, 0, 0, 0};
    }
  };

  v4i acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int nk = (K + kBK - 1) / kBK;
  // Fragment reads of one stage: 8 A blocks and 8 B blocks of 16 rows x 64 bytes.
  auto read_frags = [&](int kt, v4i (&fa)[8], v4i (&fb)[8]) {
    const int8_t* sA = smem[kt % kStages][0];
    const int8_t* sB = smem[kt % kStages][1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = wm + i * 16 + l16;
      fa[i] = *reinterpret_cast<const v4i*>(&sA[row * kBK + ((lg ^ lds_swz(row)) << 4)]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = wn + j * 16 + l16;
      fb[j] = *reinterpret_cast<const v4i*>(&sB[row * kBK + ((lg ^ lds_swz(row)) << 4)]);
    }
  };
  // Make stage `kt` visible to every wave.  Stages after it stay in flight:
  // at this point stages kt .. min(kt + kStages - 3, nk - 1) are outstanding.
  auto wait_stage = [&](int kt) {
    const int ahead = min(kStages - 3, nk - 1 - kt);
    if (ahead >= 1) wait_vmcnt<8>();
    else wait_vmcnt<0>();
    lds_barrier();
  };
  // One k-step: 64 MFMAs on fragments already in registers (stage kt), while
  // the fragments of stage kt + 1 are read from LDS.
  auto step = [&](int kt, v4i (&ca)[8], v4i (&cb)[8], v4i (&na)[8], v4i (&nb)[8]) {
    if (kt + 1 < nk) {
      wait_stage(kt + 1);
      if (ktail && kt + 2 == nk) {
        zero_k_tail((kt + 1) % kStages);
        lds_barrier();
      }
      // the buffer refilled here was last read for stage kt - 1, whose
      // fragments every wave consumed before the barrier above
      if (kt + kStages - 1 < nk) issue((kt + kStages - 1) % kStages, kt + kStages - 1);
      read_frags(kt + 1, na, nb);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ca[i], cb[j], acc[i][j], 0, 0, 0);
  };

#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nk) issue(s, s);
  v4i a0[8], b0[8], a1[8], b1[8];
  // stage 0 must land; the other stages issued above may stay in flight
  static_assert(kStages == 4, "wait counts below assume a 4-stage ring");
  if (nk >= 3) wait_vmcnt<16>();
  else if (nk == 2) wait_vmcnt<8>();
  else wait_vmcnt<0>();
  lds_barrier();
  if (ktail && nk == 1) {
    zero_k_tail(0);
    lds_barrier();
  }
  read_frags(0, a0, b0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, a0, b0, a1, b1);
    step(kt + 1, a1, b1, a0, b0);
  }
  if (kt < nk) step(kt, a0, b0, a1, b1);
  __syncthreads();   // all waves done with the ring before the epilogue reuses it

  // D layout of a 16x16 block: lane holds rows 4*(lane/16) + r, column lane % 16.
  if constexpr (OUT_I32) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm + i * 16 + lg * 4 + r;
          const int n = n0 + wn + j * 16 + l16;
          if (m < M && n < N) a.acc[(size_t)m * N + n] = acc[i][j][r];
        }
    return;
  } else {
    // ---- epilogue, one 16-column block of the wave tile at a time -----------
    // (bounds the live fp32 values to 8 blocks; the int32 accumulators stay in
    // the accumulation registers until their block is converted)
    const int n_out = *a.n_out;
    uint16_t* sAo = reinterpret_cast<uint16_t*>(&smem[0][0][0]);   // [256 rows][32 halves]
    uint16_t* sBo = reinterpret_cast<uint16_t*>(&smem[0][1][0]);   // [256 cols][32 halves]
    // Stage outlier columns j0 .. j0+31 of X_O and the matching weight rows
    // (transposed to [column][outlier]); zero past n_out.
    auto stage_outliers = [&](int j0) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int q = t + kGemmThreads * s;
        const int row = q >> 2, c = q & 3;
        const int gm = m0 + row;
        const int jj = j0 + c * 8;
        v4i v = {0, 0, 0, 0};
        if (gm < M && jj < n_out) {
          const uint16_t* src = a.X_O + (size_t)gm * K + jj;
          if (jj + 8 <= n_out) {
            v = *reinterpret_cast<const v4i*>(src);
          } else {
            uint32_t w[4] = {0, 0, 0, 0};
            for (int e = 0; jj + e < n_out; ++e) w[e >> 1] |= (uint32_t)src[e] << ((e & 1) * 16);
            v = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
          }
        }
        *reinterpret_cast<v4i*>(&sAo[row * 32 + ((c ^ lds_swz(row)) << 3)]) = v;
      }
      const int col = t;   // 256 threads = 256 columns
      const int gn = n0 + col;
      uint32_t w[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) w[e] = 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int j = j0 + e;
        uint32_t h = 0;
        if (j < n_out && gn < N) h = a.W_rows[(size_t)a.idx[j] * N + gn];
        w[e >> 1] |= h << ((e & 1) * 16);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v4i v = {(int)w[4 * c], (int)w[4 * c + 1], (int)w[4 * c + 2], (int)w[4 * c + 3]};
        *reinterpret_cast<v4i*>(&sBo[col * 32 + ((c ^ lds_swz(col)) << 3)]) = v;
      }
    };
    auto load_ao = [&](v8h (&fa)[8]) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = wm + i * 16 + l16;
        fa[i] = *reinterpret_cast<const v8h*>(&sAo[row * 32 + ((lg ^ lds_swz(row)) << 3)]);
      }
    };
    auto load_bo = [&](int j) {
      const int col = wn + j * 16 + l16;
      return *reinterpret_cast<const v8h*>(&sBo[col * 32 + ((lg ^ lds_swz(col)) << 3)]);
    };

    const bool one_chunk = n_out <= 32;
    v8h fo[8];
    if (n_out > 0 && one_chunk) {
      stage_outliers(0);
      __syncthreads();
      load_ao(fo);
    }
    float sxv[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + i * 16 + lg * 4 + r;
        sxv[i][r] = m < M ? a.sx[m] : 0.0f;
      }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = n0 + wn + j * 16 + l16;
      const float swj = n < N ? a.sw[n] * (1.0f / 16129.0f) : 0.0f;
      v4f y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) y[i][r] = (float)acc[i][j][r] * (sxv[i][r] * swj);
      if (n_out > 0) {
        if (one_chunk) {
          const v8h fb = load_bo(j);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            y[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fo[i], fb, y[i], 0, 0, 0);
        } else {
          for (int j0 = 0; j0 < n_out; j0 += 32) {
            __syncthreads();
            stage_outliers(j0);
            __syncthreads();
            v8h fa[8];
            load_ao(fa);
            const v8h fb = load_bo(j);
#pragma unroll
            for (int i = 0; i < 8; ++i)
              y[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb, y[i], 0, 0, 0);
          }
        }
      }
      if (n < N) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm + i * 16 + lg * 4 + r;
            if (m < M) a.Y[(size_t)m * N + n] = f2h(y[i][r]);
          }
      }
    }
  }
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  const int nTm = (a.M + kBM - 1) / kBM, nTn = (a.N + kBN - 1) / kBN;
  const dim3 grid(nTm * nTn);
  if (a.acc)
    hipLaunchKernelGGL(gemm_i8_kernel<true>, grid, dim3(kGemmThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(gemm_i8_kernel<false>, grid, dim3(kGemmThreads), 0, stream, a);
  return hipGetLastError();
}

const char* gemm_tile_info() {
  return "gemm: 256x256x64 tile, 4 waves of 128x128, v_mfma_i32_16x16x64_i8, "
         "v_mfma_f32_16x16x32_f16 outlier tail";
}

}  // namespace i8l
