// Small-M ("decode") LLM.int8() linear layer: the whole layer in one launch.
//
// Same method as the prefill path ([blog, "A gentle summary of LLM.int8()"],
// [blog, "A closer look at the MatMul"]), shaped for M <= 16 rows, where the
// time is the single read of the int8 weight from HBM.
//
// Each workgroup (8 waves) owns 64 output features (4 blocks of 16) and
// streams their int8 weight rows once; the 8 waves split K.
//   1. A wave's weight loads (8 k-steps x 4 blocks = 128 VGPRs at a time)
//      are issued right after the few activation loads, so the HBM latency
//      overlaps the whole activation stage; the K chunk a wave streams is
//      rotated by the workgroup index to spread concurrent requests.
//   2. Fused variant (M*K small): every workgroup redundantly runs the
//      activation stage on the tiny X (L2-resident): each thread owns whole
//      8-column chunks over all M rows, so it decides their outlier flags
//      locally; row absmax over the regular columns is reduced across the
//      workgroup; codes go to LDS [M][K].  Workgroup 0 also writes the
//      intermediates (Xq, sx, outlier list, X_O) to the workspace.
//      Unfused variant: reads those intermediates, written by the activation
//      kernels, from the workspace.
//   3. The outlier values of X are gathered into LDS during the prologue (up
//      to 64), and each epilogue lane loads its outlier weight values (up to 8)
//      into registers as soon as the outlier list is known, so the epilogue
//      issues no dependent global loads in the common case; more outliers
//      take slower loops over global memory.
//   4. v_mfma_i32_16x16x64_i8 with the activations as the 16-row operand
//      (rows >= M are zero) and 16 weight rows as the other; int32 partials of
//      the 8 waves are summed through LDS (exact, order-free).
//   5. Epilogue: dequantize with sx * sw / 127^2, add the fp32 outlier
//      products, store fp16.
#include "common.h"
#include "launch.h"

namespace i8l {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kDecP = 4;                      // 16-feature blocks per workgroup
constexpr int kDecCols = 16 * kDecP;
constexpr int kDecMaxK = 8192;                // fused variant
constexpr int kDecLdsXq = 65536;              // fused variant: M * Kpad <= this
constexpr int kDecRedBytes = kDecWaves * kDecP * 64 * 16;
constexpr int kDecMaxOutLds = 64;             // outlier values of X gathered into LDS
constexpr int kDecOutReg = 8;                 // outlier weight values held per lane

// 16 zero bytes for lanes whose load is out of range (loads stay unconditional).
__device__ __attribute__((aligned(64))) int8_t g_dec_zero[64];

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
  lds_sync();
  if (wave == 0) {
    int w = lane < BS / 64 ? s_tmp[lane] : 0;
    int wi = wave_incl_scan(w);
    if (lane < BS / 64) s_tmp[lane] = wi - w;
    if (lane == 63) s_tmp[BS / 64] = wi;
  }
  lds_sync();
  int r = s_tmp[wave] + incl - v;
  *total = s_tmp[BS / 64];
  lds_sync();
  return r;
}

// MR: rows of X held per thread in the fused prologue (8 or 16, >= M);
// QC: 8-column chunks per thread (K <= kDecThreads * 8 * QC);
// kDecU: k-steps of 64 bytes per weight load batch (register budget).
template <bool FUSED, int MR, int QC, int kDecU, int kDecPre = 2>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeArgs d) {
  constexpr int kUnion = (FUSED ? kDecLdsXq : 0) > kDecRedBytes ? kDecLdsXq : kDecRedBytes;
  __shared__ __attribute__((aligned(16))) int8_t sU[kUnion];   // Xq [M][Kpad], later partials
  __shared__ int sIdx[FUSED ? kDecMaxK : 1];
  __shared__ uint32_t sFlags[FUSED ? kDecMaxK / 32 : 1];
  __shared__ int sRank[FUSED ? kDecMaxK / 32 : 1];
  __shared__ float sXO[16][kDecMaxOutLds];        // X at the outlier columns
  __shared__ int sTmp[kDecWaves + 1];
  __shared__ uint32_t sRowMax[kDecWaves][16];
  __shared__ float sSx[16];
  __shared__ int sNout;

  const int M = d.M, K = d.K, N = d.N;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n0 = blockIdx.x * kDecCols;
  const int kpad = (K + 63) & ~63;
  const int nsteps = kpad >> 6;
  // K chunk of this wave, rotated by the workgroup index so that concurrently
  // running workgroups start their weight streams at different offsets
  // (measured ~15% more HBM bandwidth than all starting at chunk 0).
  const int kc = (wave + blockIdx.x) % kDecWaves;
  const int s0 = kc * nsteps / kDecWaves, s1 = (kc + 1) * nsteps / kDecWaves;
  const int lr = lane & 15;             // operand row inside a 16-block
  const int kl = (lane >> 4) * 16;      // 16-byte k chunk of this lane

  // Weight loads are unconditional (out-of-range lanes read the zero page):
  // with a fixed number of loads in flight the compiler can wait for the
  // activation loads issued before them without waiting for the whole stream.
  auto load_b = [&](int s, v4i (&fb)[kDecU][kDecP], int u0, int u1) {
#pragma unroll
    for (int u = u0; u < u1; ++u) {
      const int k = (s + u) * 64 + kl;
#pragma unroll
      for (int c = 0; c < kDecP; ++c) {
        const int n = n0 + c * 16 + lr;
        const bool in = s + u < s1 && n < N && k < K;
        const int8_t* p = in ? d.Wq + (size_t)n * K + k : g_dec_zero;
        fb[u][c] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
      }
    }
  };

  // Fused variant: the activation rows this thread owns are loaded before the
  // weight stream, so the activation stage only waits for them (loads retire
  // in order) and runs while the weight is in flight.
  constexpr int kXR = FUSED ? MR : 1, kXC = FUSED ? QC : 1;
  v4i xv[kXC][kXR];
  if constexpr (FUSED) {
    const int nq = K >> 3;
#pragma unroll
    for (int h = 0; h < QC; ++h) {
      const int q = t + h * kDecThreads;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const bool in = q < nq && m < M;
        const void* p = in ? (const void*)(d.X + (size_t)m * K + q * 8) : (const void*)g_dec_zero;
        xv[h][m] = *reinterpret_cast<const v4i*>(p);
      }
    }
  }
  // Only the first kDecPre k-steps go out before the activation stage: with a
  // full memory queue, waves stall on issue and the stage's barriers would wait
  // for the whole stream; the rest is issued right after the stage.
  v4i fb[kDecU][kDecP];
  load_b(s0, fb, 0, kDecPre);

  // Outlier weight values of this lane's output feature (epilogue lanes of
  // waves 0..kDecP-1), loaded into registers as soon as the outlier list is
  // known and used only in the epilogue: loads retire in order, so nothing
  // waits for them before the weight stream has arrived anyway.
  // Unconditional raw fp16 loads (out-of-range lanes read the zero page),
  // converted only in the epilogue, so nothing waits for them here.
  uint16_t wo[kDecOutReg];
  auto load_wo = [&](int nout, const int* idx_src) {
    const int n = n0 + (wave & (kDecP - 1)) * 16 + lr;
#pragma unroll
    for (int j = 0; j < kDecOutReg; ++j) {
      const bool in = wave < kDecP && j < nout && n < N;
      const int k = in ? idx_src[j] : 0;
      const uint16_t* p = in ? d.W_rows + (size_t)k * N + n
                             : reinterpret_cast<const uint16_t*>(g_dec_zero);
      wo[j] = *p;
    }
  };

  int nout;
  // ---- activation stage ------------------------------------------------------
  if constexpr (FUSED) {
    const int nq = K >> 3;              // 8-column chunks; nq <= kDecThreads * QC
    uint32_t um[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) um[m] = 0;
#pragma unroll
    for (int h = 0; h < QC; ++h) {
      const int q = t + h * kDecThreads;
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
    lds_sync();
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
    const int rank = dec_block_excl_scan<kDecThreads>(__builtin_popcount(fw), sTmp, &total);
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
    lds_sync();   // sSx, sIdx, sRank, sNout visible
    nout = sNout;
    load_wo(nout, sIdx);
    // codes -> LDS; outlier values -> LDS (and, in workgroup 0, all of it to
    // the workspace)
#pragma unroll
    for (int h = 0; h < QC; ++h) {
      const int q = t + h * kDecThreads;
      if (q < nq) {
        const uint32_t ob = reinterpret_cast<const uint8_t*>(sFlags)[q];
        const int word = q >> 2, sh = (q & 3) * 8;
        const int rb0 = sRank[word] + __builtin_popcount(sFlags[word] & ((1u << sh) - 1u));
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          if (m < M) {
            const float inv = quant_scale(sSx[m]);
            int code[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint16_t hb =
                  (uint16_t)(((uint32_t)xv[h][m][e >> 1] >> ((e & 1) * 16)) & 0xffffu);
              code[e] = ((ob >> e) & 1u) ? 0 : quant_code(h2f(hb), inv);
            }
            v2i packed = {(int)pack4_i8(code[0], code[1], code[2], code[3]),
                          (int)pack4_i8(code[4], code[5], code[6], code[7])};
            *reinterpret_cast<v2i*>(&sU[m * kpad + q * 8]) = packed;
            if (blockIdx.x == 0) *reinterpret_cast<v2i*>(d.Xq + (size_t)m * K + q * 8) = packed;
            if (ob) {
              int rb = rb0;   // rank of this chunk's first outlier column
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if ((ob >> e) & 1u) {
                  const uint16_t hb =
                      (uint16_t)(((uint32_t)xv[h][m][e >> 1] >> ((e & 1) * 16)) & 0xffffu);
                  if (rb < kDecMaxOutLds) sXO[m][rb] = h2f(hb);
                  if (blockIdx.x == 0) d.X_O[(size_t)m * K + rb] = hb;
                  ++rb;
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
      for (int j = t; j < nout; j += kDecThreads) d.idx[j] = sIdx[j];
      if (t == 0) *d.n_out = nout;
    }
    lds_sync();
  } else {
    nout = 0;   // read after the main loop (see below)
  }

  load_b(s0, fb, kDecPre, kDecU);

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
    if (s + kDecU < s1) load_b(s + kDecU, fb, 0, kDecU);
  }

  if constexpr (!FUSED) {
    // The activation kernels wrote the outlier list and values; read them now
    // that the weight stream has been consumed.
    nout = *d.n_out;
    load_wo(nout, d.idx);
    const int nl = min(nout, kDecMaxOutLds);
    for (int e = t; e < nl * M; e += kDecThreads) {
      const int m = e / nl, j = e % nl;
      sXO[m][j] = h2f(d.X_O[(size_t)m * K + j]);
    }
  }

  // ---- sum the partials of the 8 waves -----------------------------------------
  lds_sync();   // everyone is done reading the LDS codes
  v4i* red = reinterpret_cast<v4i*>(sU);
#pragma unroll
  for (int c = 0; c < kDecP; ++c) red[(wave * kDecP + c) * 64 + lane] = acc[c];
  lds_sync();
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
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = mb + r;
    const float sxm = (m < M) ? (FUSED ? sSx[m] : d.sx[m]) : 0.0f;
    y[r] = (float)tot[r] * (sxm * swn);
  }
#pragma unroll
  for (int j = 0; j < kDecOutReg; ++j) {
    if (j < nout) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (mb + r < M) y[r] += sXO[mb + r][j] * h2f(wo[j]);
    }
  }
  const int nl = min(nout, kDecMaxOutLds);
  for (int j = kDecOutReg; j < nl; ++j) {   // weight values beyond the registers
    const int k = FUSED ? sIdx[j] : d.idx[j];
    const float w = h2f(d.W_rows[(size_t)k * N + n]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (mb + r < M) y[r] += sXO[mb + r][j] * w;
  }
  for (int j = nl; j < nout; ++j) {   // beyond the LDS gather: straight from memory
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
      hipLaunchKernelGGL((decode_kernel<true, 8, 1, 8>), grid, dim3(kDecThreads), 0, stream, d);
    else if (M <= 8)
      hipLaunchKernelGGL((decode_kernel<true, 8, 2, 4>), grid, dim3(kDecThreads), 0, stream, d);
    else
      hipLaunchKernelGGL((decode_kernel<true, 16, 1, 4>), grid, dim3(kDecThreads), 0, stream, d);
  } else {
    hipError_t e = launch_quantize_activation(X, M, K, threshold, enabled, ws, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_kernel<false, 8, 1, 8>), grid, dim3(kDecThreads), 0, stream, d);
  }
  return hipGetLastError();
}

hipError_t launch_decode_unfused(const uint16_t* X, int M, int K, const int8_t* Wq,
                                 const float* sw, int N, const uint16_t* W_rows, uint16_t* Y,
                                 const Workspace& ws, hipStream_t stream) {
  DecodeArgs d{X, M, K, N, Wq, sw, W_rows, 0.0f, 0, Y, ws.n_out, ws.idx, ws.sx, ws.Xq, ws.X_O};
  const dim3 grid((N + kDecCols - 1) / kDecCols);
  hipLaunchKernelGGL((decode_kernel<false, 8, 1, 8>), grid, dim3(kDecThreads), 0, stream, d);
  return hipGetLastError();
}

}  // namespace i8l
