// The LLM.int8() layer for batches of 65 to 256 rows: the int8 GEMM with
// narrow 256 x 64 output tiles, dequantization, fp16 outlier product and
// bias fused into its epilogue.
//
// [blog, "Introduction to model quantization"] and [blog, "A gentle summary
// of LLM.int8()"], steps 2-3: the same product and epilogue as gemm.hip.
//
// At these sizes the layer is bound by the read of the int8 weight (an
// 8-row to 256-row batch against a 64 MB weight does about 2*M ops per weight
// byte, at most 512, below the chip's 629 ops/byte ridge), yet 256 x 256
// tiles give only N / 256 workgroups (64 for N = 16384): a quarter of the
// compute units, which then needs a split along K and int32 partials that
// move twice the weight's bytes.  Tiles of 256 rows x 64 output features give
// N / 64 workgroups (256 for N = 16384), each streaming its own 64 weight
// rows once while the activation codes, read by every workgroup, come from
// the L2.
//
// Tiles of BM = 256 rows (M > 128) or 128 rows (M <= 128: the activation codes,
// which every workgroup reads, are then half the bytes).  512 threads = 8
// waves; with BM = 256 wave w owns rows 32w .. 32w+31 of the tile and all 64
// features (two 32x32 blocks of v_mfma_i32_32x32x32_i8), with BM = 128 rows
// 32 (w % 4) .. +31 and features 32 (w / 4) .. +31 (one block).  K steps of
// 128 bytes; the LDS holds a ring of 4 steps (A panel BM x 128 bytes + B panel
// 8 KB each), filled by direct global -> LDS loads three steps ahead of the
// step being multiplied (BM / 64 + 1 loads of 1 KB per wave per step, a fixed
// count: past the last step the loads re-read the last step into a consumed
// slot).  LDS rows are 128 bytes with the same chunk swizzle as gemm.hip.
// Epilogue: the int32 accumulators (zero-point mode: plus (128 - zp) * wsum)
// are dequantized to fp32; the outlier columns are staged 32 at a time in LDS
// (X_O rows of the tile and the matching weight rows, from the fp16 weight or
// rebuilt from the codes) and added with v_mfma_f32_32x32x16_f16; the bias is
// added; the block is stored as fp16 in 16-byte row pieces through LDS.
#include "common.h"
#include "launch.h"

namespace i8l {

typedef int v16i_s __attribute__((ext_vector_type(16)));
typedef float v16f_s __attribute__((ext_vector_type(16)));

constexpr int kSBM = 256, kSBN = 64, kSBK = 128;   // kSBM: the largest tile height
constexpr int kSStages = 4;
constexpr int kSSlotA = kSBM * kSBK;   // 32 KB (ring slots sized for BM = 256)
constexpr int kSSlotB = kSBN * kSBK;   // 8 KB
constexpr int kSThreads = 512;
constexpr int kSOutC = 32;             // outlier columns staged per round
constexpr int kSOutS = kSOutC + 8;     // staged row stride in halves (80 bytes)

__device__ __attribute__((aligned(64))) int8_t g_skinny_zero[64];

__device__ __forceinline__ int sk_swz(int row) { return ((row >> 1) & 3) | (((row >> 4) & 1) << 2); }
__device__ __forceinline__ int sk_drow(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int N>
__device__ __forceinline__ void sk_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

#define I8L_SK_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// BM: tile height (256 or 128).  OUT_I32: store the int32 accumulators to
// a.acc instead of the layer's Y.  ZP: zero-point epilogue (see gemm.hip).
template <int BM, bool OUT_I32, bool ZP>
__global__ __launch_bounds__(kSThreads, 1) void gemm_skinny_kernel(GemmArgs a) {
  constexpr int NB = BM == 256 ? 2 : 1;   // 32-feature blocks per wave
  constexpr int LA = BM / 64;             // A loads per wave per step
  static_assert(BM == 256 || BM == 128, "tile height");
  __shared__ __attribute__((aligned(1024))) int8_t smem[kSStages * (kSSlotA + kSSlotB)];
  int8_t* const sA = smem;
  int8_t* const sB = smem + kSStages * kSSlotA;

  const int M = a.M, N = a.N, K = a.K;
  const int nk = (K + kSBK - 1) / kSBK;
  // tiles: 1 row of tiles for M <= 256, more rows (rare) in row-major order
  const int nTn = (N + kSBN - 1) / kSBN;
  const int tm = blockIdx.x / nTn, tn = blockIdx.x % nTn;
  const int m0 = tm * BM, n0 = tn * kSBN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  const int wm = BM == 256 ? wave * 32 : (wave & 3) * 32;
  const int wn = BM == 256 ? 0 : (wave >> 2) * 32;

  // loads: A blocks LA*w .. LA*w+LA-1 (8 rows of 128 bytes each), B block w
  const int lastA = min(M - m0, BM) - 1, lastB = min(N - n0, kSBN) - 1;
  uint32_t rowA[LA];
  int cofA[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int row = (wave * LA + i) * 8 + (lane >> 3);
    cofA[i] = ((lane & 7) ^ sk_swz(row)) * 16;
    rowA[i] = (uint32_t)(min(row, lastA) * K);
  }
  const int rowb = wave * 8 + (lane >> 3);
  const int cofB = ((lane & 7) ^ sk_swz(rowb)) * 16;
  const uint32_t rowB = (uint32_t)(min(rowb, lastB) * K);
  const int8_t* tileA = a.Xq + (size_t)m0 * K;
  const int8_t* tileB = a.Wq + (size_t)n0 * K;
  // The K loop starts at a step rotated by the workgroup's place on its XCD
  // (workgroup b runs on XCD b % 8): the XCD's compute units then read
  // different steps of the activation codes at any time instead of the same
  // lines at once.  Integer sums: the order does not change the result.
  const int rot = (int)((long long)(blockIdx.x >> 3) * nk / 32 % nk);
  auto load_step = [&](int kt) {   // kt may run past the end: clamped to the last step
    const int kc = min(kt, nk - 1) + rot, sl = kt % kSStages;
    const int ks = kc < nk ? kc : kc - nk;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int kk = ks * kSBK + cofA[i];
      const int8_t* g = kk < K ? tileA + rowA[i] + kk : g_skinny_zero;
      __builtin_amdgcn_global_load_lds((const void*)g,
                                       I8L_SK_LDS(&sA[sl * kSSlotA + (wave * LA + i) * 1024]),
                                       16, 0, 0);
    }
    const int kk = ks * kSBK + cofB;
    const int8_t* g = kk < K ? tileB + rowB + kk : g_skinny_zero;
    __builtin_amdgcn_global_load_lds((const void*)g, I8L_SK_LDS(&sB[sl * kSSlotB + wave * 1024]),
                                     16, 0, 0);
  };
  auto read_q = [&](int kt, int q, v4i& fa, v4i (&fb)[NB]) {
    const int sl = kt % kSStages, c = 2 * q + lh;
    const int row = wm + l32;
    fa = *reinterpret_cast<const v4i*>(&sA[sl * kSSlotA + row * kSBK + ((c ^ sk_swz(row)) << 4)]);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int rb = wn + j * 32 + l32;
      fb[j] = *reinterpret_cast<const v4i*>(&sB[sl * kSSlotB + rb * kSBK + ((c ^ sk_swz(rb)) << 4)]);
    }
  };

  v16i_s acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = v16i_s{};
  load_step(0);
  load_step(1);
  load_step(2);
  for (int kt = 0; kt < nk; ++kt) {
    sk_wait_vmcnt<2 * (LA + 1)>();                  // step kt landed (steps kt+1, kt+2 may fly)
    asm volatile("s_barrier" ::: "memory");         // ... for every wave; step kt-1 consumed
    load_step(kt + 3);                              // into step kt-1's slot
    v4i fa[2], fb[2][NB];
    read_q(kt, 0, fa[0], fb[0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < 3) read_q(kt, q + 1, fa[(q + 1) & 1], fb[(q + 1) & 1]);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[q & 1], fb[q & 1][j], acc[j], 0, 0, 0);
    }
  }
  sk_wait_vmcnt<0>();
  __syncthreads();   // the ring is free for the epilogue

  if constexpr (OUT_I32) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = n0 + wn + j * 32 + l32;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm + sk_drow(r, lane);
        if (m < M) a.acc[(size_t)m * N + n] = acc[j][r];
      }
    }
    return;
  } else {
    // ---- epilogue ----
    uint16_t* sXo = reinterpret_cast<uint16_t*>(smem);              // [256][kSOutS]
    uint16_t* sWo = sXo + kSBM * kSOutS;                             // [64][kSOutS]
    float* sSx = reinterpret_cast<float*>(sWo + kSBN * kSOutS);      // [256]
    float* sSw = sSx + kSBM;                                         // [64], includes 1/127^2
    float* sBias = sSw + kSBN;                                       // [64]
    int* sZc = reinterpret_cast<int*>(sBias + kSBN);                 // [256] 128 - zp
    int* sWs = sZc + kSBM;                                           // [64] wsum
    uint16_t* sT = reinterpret_cast<uint16_t*>(sWs + kSBN) + wave * 32 * 40;   // [32][40] per wave
    if (t < kSBM) {
      sSx[t] = t < BM && m0 + t < M ? a.sx[m0 + t] : 0.0f;
      if (ZP) sZc[t] = t < BM && m0 + t < M ? 128 - a.zp[m0 + t] : 0;
    } else if (t < kSBM + kSBN) {
      const int u = t - kSBM, n = n0 + u;
      sSw[u] = n < N ? a.sw[n] * (ZP ? 1.0f / 127.0f : 1.0f / 16129.0f) : 0.0f;
      sBias[u] = a.bias && n < N ? h2f(a.bias[n]) : 0.0f;
      if (ZP) sWs[u] = n < N ? a.wsum[n] : 0;
    }
    __syncthreads();
    v16f_s y[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float swv = sSw[wn + j * 32 + l32];
      const uint32_t wsv = ZP ? (uint32_t)sWs[wn + j * 32 + l32] : 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mr = wm + sk_drow(r, lane);
        int tot = acc[j][r];
        if (ZP) tot = (int)((uint32_t)tot + (uint32_t)sZc[mr] * wsv);   // mod 2^32, exact result
        y[j][r] = (float)tot * (sSx[mr] * swv);
      }
    }
    // outlier product, kSOutC staged columns per round
    const int n_out = *a.n_out;
    const int rows = min(M - m0, BM);
    const buf_rsrc rxo = make_rsrc(a.X_O + (size_t)m0 * K, (uint32_t)rows * (uint32_t)K * 2u);
    for (int j0 = 0; j0 < n_out; j0 += kSOutC) {   // uniform
      __syncthreads();   // the previous round's fragments are read
      // X_O rows of the tile, columns j0 .. j0+31: BM rows x 4 chunks of 8
#pragma unroll
      for (int i = 0; i < BM / 128; ++i) {
        const int q = t + i * kSThreads, row = q >> 2, ch = q & 3;
        v4i v = buf_load16(rxo, (uint32_t)(row * K + j0 + ch * 8) * 2u);
        const int nv = n_out - (j0 + ch * 8);   // valid halves of this chunk
#pragma unroll
        for (int d = 0; d < 4; ++d)
          v[d] &= (int)((2 * d < nv ? 0xffffu : 0u) | (2 * d + 1 < nv ? 0xffff0000u : 0u));
        *reinterpret_cast<v4i*>(&sXo[row * kSOutS + ch * 8]) = v;
      }
      // weight rows idx[j0 .. j0+31] at the tile's 64 features, transposed to
      // [feature][outlier]: thread (feature f, group g) takes outliers 4g .. 4g+3
      {
        const int f = t & 63, g4 = (t >> 6) * 4, n = n0 + f;
        const int nc = n < N ? n : N - 1;
        const float sn = a.W_rows ? 0.0f : a.sw[nc];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + g4 + e;
          uint16_t h = 0;
          if (j < n_out && n < N) {
            const int k = a.idx[j];
            h = a.W_rows ? a.W_rows[(size_t)k * N + n] : dequant_w16(a.Wq[(size_t)n * K + k], sn);
          }
          sWo[f * kSOutS + g4 + e] = h;
        }
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < 2; ++h) {   // 16 outlier columns per MFMA
        const v8h fa = *reinterpret_cast<const v8h*>(&sXo[(wm + l32) * kSOutS + h * 16 + lh * 8]);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const v8h fb =
              *reinterpret_cast<const v8h*>(&sWo[(wn + j * 32 + l32) * kSOutS + h * 16 + lh * 8]);
          y[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, fb, y[j], 0, 0, 0);
        }
      }
    }
    // bias, fp16, stores: through LDS in row order when N % 8 == 0
    const bool vec_store = (N & 7) == 0;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float bv = sBias[wn + j * 32 + l32];
      const int n = n0 + wn + j * 32 + l32;
      if (vec_store) {   // uniform
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[sk_drow(r, lane) * 40 + l32] = f2h(y[j][r] + bv);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int row = lane >> 1, c0 = (lane & 1) * 16;
        const v4i p0 = *reinterpret_cast<const v4i*>(&sT[row * 40 + c0]);
        const v4i p1 = *reinterpret_cast<const v4i*>(&sT[row * 40 + c0 + 8]);
        const int m = m0 + wm + row, nb = n0 + wn + j * 32 + c0;
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
          const int m = m0 + wm + sk_drow(r, lane);
          if (m < M) a.Y[(size_t)m * N + n] = f2h(y[j][r] + bv);
        }
      }
    }
  }
}

static_assert(kSBM * kSOutS * 2 + kSBN * kSOutS * 2 + (kSBM + 3 * kSBN) * 4 + kSBM * 4 +
                      kSThreads / 64 * 32 * 40 * 2 <=
                  kSStages * (kSSlotA + kSSlotB),
              "skinny epilogue staging must fit the ring");

template <int BM>
hipError_t launch_skinny_bm(const GemmArgs& a, hipStream_t stream) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + kSBN - 1) / kSBN);
  if (a.acc)
    hipLaunchKernelGGL((gemm_skinny_kernel<BM, true, false>), dim3(tiles), dim3(kSThreads), 0,
                       stream, a);
  else if (a.zp)
    hipLaunchKernelGGL((gemm_skinny_kernel<BM, false, true>), dim3(tiles), dim3(kSThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<BM, false, false>), dim3(tiles), dim3(kSThreads), 0,
                       stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  return a.M <= 128 ? launch_skinny_bm<128>(a, stream) : launch_skinny_bm<256>(a, stream);
}

}  // namespace i8l
