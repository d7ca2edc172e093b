// Small-M ("decode") LLM.int8() linear layer: the whole layer in one launch.
//
// Same method as the prefill path ([blog, "A gentle summary of LLM.int8()"],
// [blog, "A closer look at the MatMul"]), shaped for M <= 16 rows, where the
// time is the single read of the int8 weight from HBM.
//
// Each workgroup (8 waves) owns 64 output features (4 blocks of 16) and
// streams their int8 weight rows once; the 8 waves split K.
//   1. The first batch of weight loads is issued before anything else, so the
//      HBM latency overlaps the activation stage.
//   2. Fused variant (M*K small): every workgroup redundantly runs the
//      activation stage on the tiny X (L2-resident): each thread owns whole
//      8-column chunks over all M rows, so it decides their outlier flags
//      locally; row absmax over the regular columns is reduced across the
//      workgroup; codes go to LDS [M][K].  Workgroup 0 also writes the
//      intermediates (Xq, sx, outlier list, X_O) to the workspace.
//      Unfused variant: reads those intermediates, written by the activation
//      kernels, from the workspace.
//   3. v_mfma_i32_16x16x64_i8 with the activations as the 16-row operand
//      (rows >= M are zero) and 16 weight rows as the other; int32 partials of
//      the 8 waves are summed through LDS (exact, order-free).
//   4. Epilogue: dequantize with sx * sw / 127^2, add the fp32 outlier
//      products accumulated from the fp16 values, store fp16.
#include "common.h"
#include "launch.h"

namespace i8l {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kDecP = 4;                      // 16-feature blocks per workgroup
constexpr int kDecCols = 16 * kDecP;
constexpr int kDecU = 4;                      // k-steps of 64 per load batch
constexpr int kDecMaxK = 8192;                // fused variant
constexpr int kDecLdsXq = 65536;              // fused variant: M * Kpad <= this
constexpr int kDecRedBytes = kDecWaves * kDecP * 64 * 16;

struct DecodeArgs {
  const uint16_t* X;
  int M, K, N;
  const int8_t* Wq;
  const float* sw;
  const uint16_t* W_rows;
  float threshold;
  int enabled;
  uint16_t* Y;
  int32_t* n_out;
  int32_t* idx;
  float* sx;
  int8_t* Xq;
  uint16_t* X_O;
};

bool decode_fits(int M, int K) {
  const int kpad = (K + 63) / 64 * 64;
  if (M < 1 || M > 16 || K > kDecMaxK || M * kpad > kDecLdsXq) return false;
  return M <= 8 || K <= kDecThreads * 8;   // rows x chunks held per thread <= 16
}

template <int BS>
__device__ __forceinline__ int dec_block_excl_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = wave_incl_scan(v);
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < BS / 64 ? s_tmp[lane] : 0;
    int wi = wave_incl_scan(w);
    if (lane < BS / 64) s_tmp[lane] = wi - w;
    if (lane == 63) s_tmp[BS / 64] = wi;
  }
  __syncthreads();
  int r = s_tmp[wave] + incl - v;
  *total = s_tmp[BS / 64];
  __syncthreads();
  return r;
}

// MR: rows of X held per thread in the fused prologue (8 or 16, >= M);
// QC: 8-column chunks per thread (K <= kDecThreads * 8 * QC).
template <bool FUSED, int MR, int QC>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeArgs d) {
  constexpr int kUnion = (FUSED ? kDecLdsXq : 0) > kDecRedBytes ? kDecLdsXq : kDecRedBytes;
  __shared__ __attribute__((aligned(16))) int8_t sU[kUnion];   // Xq [M][Kpad], later partials
  __shared__ int sIdx[FUSED ? kDecMaxK : 1];
  __shared__ uint32_t sFlags[FUSED ? kDecMaxK / 32 : 1];
  __shared__ int sRank[FUSED ? kDecMaxK / 32 : 1];
  __shared__ int sTmp[kDecWaves + 1];
  __shared__ uint32_t sRowMax[kDecWaves][16];
  __shared__ float sSx[16];
  __shared__ int sNout;

  const int M = d.M, K = d.K, N = d.N;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n0 = blockIdx.x * kDecCols;
  const int kpad = (K + 63) & ~63;
  const int nsteps = kpad >> 6;
  const int s0 = wave * nsteps / kDecWaves, s1 = (wave + 1) * nsteps / kDecWaves;
  const int lr = lane & 15;             // operand row inside a 16-block
  const int kl = (lane >> 4) * 16;      // 16-byte k chunk of this lane

  auto load_b = [&](int s, v4i (&fb)[kDecU][kDecP]) {
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      const int k = (s + u) * 64 + kl;
#pragma unroll
      for (int c = 0; c < kDecP; ++c) {
        const int n = n0 + c * 16 + lr;
        fb[u][c] = (s + u < s1 && n < N && k < K)
                       ? __builtin_nontemporal_load(
                             reinterpret_cast<const v4i*>(d.Wq + (size_t)n * K + k))
                       : v4i{0, 0, 0, 0};
      }
    }
  };

  v4i fb[kDecU][kDecP];
  load_b(s0, fb);

  // ---- activation stage ------------------------------------------------------
  if constexpr (FUSED) {
    const int nq = K >> 3;              // 8-column chunks; nq <= kDecThreads * 2
    uint32_t um[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) um[m] = 0;
    v4i xv[QC][MR];
#pragma unroll
    for (int h = 0; h < QC; ++h) {
      const int q = t + h * kDecThreads;
#pragma unroll
      for (int m = 0; m < MR; ++m)
        xv[h][m] = (q < nq && m < M) ? *reinterpret_cast<const v4i*>(d.X + (size_t)m * K + q * 8)
                                     : v4i{0, 0, 0, 0};
      uint32_t cm[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cm[e] = 0;
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t b = ((uint32_t)xv[h][m][e >> 1] >> ((e & 1) * 16)) & 0x7fffu;
          cm[e] = b > cm[e] ? b : cm[e];
        }
      uint32_t ob = 0;
      if (d.enabled) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (h2f((uint16_t)cm[e]) >= d.threshold) ob |= 1u << e;
      }
      // bytes past the last chunk (K % 32 == 16) complete the last word with zeros
      if (q < 4 * ((K + 31) >> 5)) reinterpret_cast<uint8_t*>(sFlags)[q] = q < nq ? (uint8_t)ob : 0;
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t b = ((uint32_t)xv[h][m][e >> 1] >> ((e & 1) * 16)) & 0x7fffu;
          if (!((ob >> e) & 1u)) um[m] = b > um[m] ? b : um[m];
        }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const uint32_t w = wave_max_u32(um[m]);
      if (lane == 0) sRowMax[wave][m] = w;
    }
    __syncthreads();
    if (t < MR) {
      uint32_t mm = 0;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) mm = sRowMax[w][t] > mm ? sRowMax[w][t] : mm;
      sSx[t] = h2f((uint16_t)mm);
    }
    // outlier list: prefix popcount over the flag words
    const int nw = (K + 31) >> 5;
    const uint32_t fw = t < nw ? sFlags[t] : 0u;   // nw <= 256 < kDecThreads
    int total;
    int rank = dec_block_excl_scan<kDecThreads>(__builtin_popcount(fw), sTmp, &total);
    if (t < nw) sRank[t] = rank;
    {
      uint32_t f = fw;
      int r = rank;
      while (f) {
        sIdx[r++] = t * 32 + __builtin_ctz(f);
        f &= f - 1u;
      }
    }
    if (t == 0) sNout = total;
    __syncthreads();   // sSx, sIdx, sNout visible
    // codes -> LDS (and, in workgroup 0, to the workspace)
#pragma unroll
    for (int h = 0; h < QC; ++h) {
      const int q = t + h * kDecThreads;
      if (q < nq) {
        const uint32_t ob = reinterpret_cast<const uint8_t*>(sFlags)[q];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          if (m < M) {
            const float inv = quant_scale(sSx[m]);
            int code[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint16_t hb = (uint16_t)(((uint32_t)xv[h][m][e >> 1] >> ((e & 1) * 16)) & 0xffffu);
              code[e] = ((ob >> e) & 1u) ? 0 : quant_code(h2f(hb), inv);
            }
            v2i packed = {(int)pack4_i8(code[0], code[1], code[2], code[3]),
                          (int)pack4_i8(code[4], code[5], code[6], code[7])};
            *reinterpret_cast<v2i*>(&sU[m * kpad + q * 8]) = packed;
            if (blockIdx.x == 0) {
              *reinterpret_cast<v2i*>(d.Xq + (size_t)m * K + q * 8) = packed;
              if (ob) {
                // rank of this chunk's first column among the outliers
                const int word = q >> 2, sh = (q & 3) * 8;
                int rb = sRank[word] + __builtin_popcount(sFlags[word] & ((1u << sh) - 1u));
#pragma unroll
                for (int e = 0; e < 8; ++e)
                  if ((ob >> e) & 1u) {
                    const uint16_t hb =
                        (uint16_t)(((uint32_t)xv[h][m][e >> 1] >> ((e & 1) * 16)) & 0xffffu);
                    d.X_O[(size_t)m * K + rb] = hb;
                    ++rb;
                  }
              }
            }
          }
        }
      }
    }
    // zero the K padding of each row so partial k-steps read zeros
    if (kpad > K) {
      for (int i = t; i < M * (kpad - K); i += kDecThreads) {
        const int m = i / (kpad - K), k = K + i % (kpad - K);
        sU[m * kpad + k] = 0;
      }
    }
    if (blockIdx.x == 0) {
      if (t < M) d.sx[t] = sSx[t];
      for (int j = t; j < sNout; j += kDecThreads) d.idx[j] = sIdx[j];
      if (t == 0) *d.n_out = sNout;
    }
    __syncthreads();
  }

  // ---- int8 product --------------------------------------------------------------
  v4i acc[kDecP];
#pragma unroll
  for (int c = 0; c < kDecP; ++c) acc[c] = v4i{0, 0, 0, 0};
  for (int s = s0; s < s1; s += kDecU) {
    v4i fa[kDecU];
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      const int k = (s + u) * 64 + kl;
      if constexpr (FUSED) {
        fa[u] = (s + u < s1 && lr < M) ? *reinterpret_cast<const v4i*>(&sU[lr * kpad + k])
                                        : v4i{0, 0, 0, 0};
      } else {
        fa[u] = (s + u < s1 && lr < M && k < K)
                    ? *reinterpret_cast<const v4i*>(d.Xq + (size_t)lr * K + k)
                    : v4i{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < kDecU; ++u)
#pragma unroll
      for (int c = 0; c < kDecP; ++c)
        acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[u], fb[u][c], acc[c], 0, 0, 0);
    if (s + kDecU < s1) load_b(s + kDecU, fb);
  }

  // ---- sum the partials of the 8 waves -----------------------------------------
  __syncthreads();   // everyone is done reading the LDS codes
  v4i* red = reinterpret_cast<v4i*>(sU);
#pragma unroll
  for (int c = 0; c < kDecP; ++c) red[(wave * kDecP + c) * 64 + lane] = acc[c];
  __syncthreads();
  if (wave >= kDecP) return;
  const int c = wave;
  v4i tot = {0, 0, 0, 0};
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    const v4i p = red[(w * kDecP + c) * 64 + lane];
    tot[0] += p[0]; tot[1] += p[1]; tot[2] += p[2]; tot[3] += p[3];
  }

  // ---- epilogue --------------------------------------------------------------------
  const int n = n0 + c * 16 + lr;
  const int mb = (lane >> 4) * 4;       // D rows of this lane: mb .. mb + 3
  if (n >= N || mb >= M) return;
  const float swn = d.sw[n] * (1.0f / 16129.0f);
  float y[4];
  int nout;
  if constexpr (FUSED) nout = sNout; else nout = *d.n_out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = mb + r;
    const float sxm = (m < M) ? (FUSED ? sSx[m] : d.sx[m]) : 0.0f;
    y[r] = (float)tot[r] * (sxm * swn);
  }
  for (int j = 0; j < nout; ++j) {
    const int k = FUSED ? sIdx[j] : d.idx[j];
    const float w = h2f(d.W_rows[(size_t)k * N + n]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mb + r;
      if (m < M) {
        const float x = FUSED ? h2f(d.X[(size_t)m * K + k]) : h2f(d.X_O[(size_t)m * K + j]);
        y[r] += x * w;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = mb + r;
    if (m < M) d.Y[(size_t)m * N + n] = f2h(y[r]);
  }
}

hipError_t launch_decode(const uint16_t* X, int M, int K, const int8_t* Wq, const float* sw,
                         int N, const uint16_t* W_rows, float threshold, bool enabled,
                         uint16_t* Y, const Workspace& ws, hipStream_t stream) {
  DecodeArgs d{X, M, K, N, Wq, sw, W_rows, threshold, enabled ? 1 : 0, Y,
               ws.n_out, ws.idx, ws.sx, ws.Xq, ws.X_O};
  const dim3 grid((N + kDecCols - 1) / kDecCols);
  if (decode_fits(M, K)) {
    // decode_fits bounds M * K, so rows held per thread times chunks is <= 16
    if (M <= 8 && K <= kDecThreads * 8)
      hipLaunchKernelGGL((decode_kernel<true, 8, 1>), grid, dim3(kDecThreads), 0, stream, d);
    else if (M <= 8)
      hipLaunchKernelGGL((decode_kernel<true, 8, 2>), grid, dim3(kDecThreads), 0, stream, d);
    else
      hipLaunchKernelGGL((decode_kernel<true, 16, 1>), grid, dim3(kDecThreads), 0, stream, d);
  } else {
    hipError_t e = launch_quantize_activation(X, M, K, threshold, enabled, ws, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_kernel<false, 8, 1>), grid, dim3(kDecThreads), 0, stream, d);
  }
  return hipGetLastError();
}

}  // namespace i8l
