// Weight quantization: per-output-feature absmax codes of an fp16 weight.
//
// [blog, "A closer look at the MatMul"]: the weight matrix is quantized column
// by column (one absmax per output feature of Y = X @ W).  [blog, "Usage"]:
// the quantization runs once when the layer is placed on the GPU and the int8
// weight keeps nn.Linear's [out][in] layout, here Wq[N][K] (K contiguous),
// which is also the layout the int8 matrix cores read.
//
// One workgroup owns a strip of 64 output features over all of K:
//   pass 1 reads the strip and reduces |W| down K (sw),
//   pass 2 re-reads it in 64x64 tiles, transposes through LDS and writes
//   16-byte runs of codes along K.
// The strip is re-read from L2/MALL, not HBM, on the second pass for the
// weight sizes used here.  Runs once per layer, off the timed path.
#include "common.h"
#include "launch.h"

namespace i8l {

constexpr int kWqStrip = 64;   // output features per workgroup
constexpr int kWqTileK = 64;   // K rows per transpose tile
constexpr int kWqThreads = 256;

template <bool VEC>
__global__ __launch_bounds__(kWqThreads) void wquant_kernel(const uint16_t* __restrict__ W, int K,
                                                           int N, int8_t* __restrict__ Wq,
                                                           float* __restrict__ sw) {
  __shared__ uint32_t red[32][kWqStrip + 1];
  __shared__ float inv_s[kWqStrip];
  __shared__ float tile[kWqTileK][kWqStrip + 1];

  const int t = threadIdx.x;
  const int n0 = blockIdx.x * kWqStrip;
  const int rg = t >> 3;         // 0..31: row group
  const int cc = (t & 7) * 8;    // first of 8 columns owned by this thread

  // ---- pass 1: column absmax ------------------------------------------------
  uint32_t mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mx[e] = 0;
  for (int k = rg; k < K; k += 32) {
    const uint16_t* row = W + (size_t)k * N + n0 + cc;
    if (VEC && n0 + cc + 8 <= N) {
      v4i raw = *reinterpret_cast<const v4i*>(row);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t b = habs_bits(((uint32_t)raw[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
        mx[e] = b > mx[e] ? b : mx[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (n0 + cc + e < N) {
          uint32_t b = habs_bits(row[e]);
          mx[e] = b > mx[e] ? b : mx[e];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][cc + e] = mx[e];
  __syncthreads();
  if (t < kWqStrip) {
    uint32_t m = 0;
    for (int r = 0; r < 32; ++r) m = red[r][t] > m ? red[r][t] : m;
    const float a = h2f((uint16_t)m);
    inv_s[t] = quant_scale(a);
    if (n0 + t < N) sw[n0 + t] = a;
  }
  __syncthreads();

  // ---- pass 2: codes, transposed through LDS ----------------------------------
  const int nl = t >> 2;          // output feature inside the strip
  const int kc = (t & 3) * 16;    // 16 consecutive k of that feature
  for (int k0 = 0; k0 < K; k0 += kWqTileK) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kr = rg + 32 * h;
      const int k = k0 + kr;
      const uint16_t* row = W + (size_t)k * N + n0 + cc;
      if (k < K && VEC && n0 + cc + 8 <= N) {
        v4i raw = *reinterpret_cast<const v4i*>(row);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          tile[kr][cc + e] = h2f((uint16_t)(((uint32_t)raw[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          tile[kr][cc + e] = (k < K && n0 + cc + e < N) ? h2f(row[e]) : 0.0f;
      }
    }
    __syncthreads();
    const int n = n0 + nl;
    const int k = k0 + kc;
    if (n < N && k < K) {
      const float inv = inv_s[nl];
      uint32_t w[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        w[g] = pack4_i8(quant_code(tile[kc + 4 * g + 0][nl], inv),
                        quant_code(tile[kc + 4 * g + 1][nl], inv),
                        quant_code(tile[kc + 4 * g + 2][nl], inv),
                        quant_code(tile[kc + 4 * g + 3][nl], inv));
      v4i out = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      *reinterpret_cast<v4i*>(Wq + (size_t)n * K + k) = out;
    }
    __syncthreads();
  }
}

hipError_t launch_quantize_weight(const uint16_t* W, int K, int N, int8_t* Wq, float* sw,
                                  hipStream_t stream) {
  const dim3 grid((N + kWqStrip - 1) / kWqStrip);
  const bool vec = (N % 8 == 0) && ((uintptr_t)W % 16 == 0);
  if (vec)
    hipLaunchKernelGGL(wquant_kernel<true>, grid, dim3(kWqThreads), 0, stream, W, K, N, Wq, sw);
  else
    hipLaunchKernelGGL(wquant_kernel<false>, grid, dim3(kWqThreads), 0, stream, W, K, N, Wq, sw);
  return hipGetLastError();
}

// Code sums S[n] = sum_k Wq[n][k] for the zero-point mode: with activation
// codes q stored as q - 128, sum_k (q - zp) w = sum_k (q - 128) w + (128 - zp) S[n]
// ([blog, "Introduction to model quantization"], the unsigned scheme).
// One wave per row of Wq, 16-byte loads along K (K % 16 == 0).  Runs once per
// layer, next to the weight quantization.
constexpr int kWsThreads = 256;
__global__ __launch_bounds__(kWsThreads) void wsum_kernel(const int8_t* __restrict__ Wq, int N,
                                                         int K, int32_t* __restrict__ S) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * (kWsThreads / 64) + (threadIdx.x >> 6);
  if (n >= N) return;   // whole wave
  const int8_t* row = Wq + (size_t)n * K;
  int sum = 0;
  for (int k = lane * 16; k < K; k += 64 * 16) {
    const v4i v = *reinterpret_cast<const v4i*>(row + k);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x = v[e];
      sum += (int)(int8_t)x + (int)(int8_t)(x >> 8) + (int)(int8_t)(x >> 16) + (x >> 24);
    }
  }
  sum = wave_sum(sum);
  if (lane == 0) S[n] = sum;
}

hipError_t launch_weight_code_sums(const int8_t* Wq, int N, int K, int32_t* S,
                                   hipStream_t stream) {
  const int per = kWsThreads / 64;
  hipLaunchKernelGGL(wsum_kernel, dim3((N + per - 1) / per), dim3(kWsThreads), 0, stream, Wq, N,
                     K, S);
  return hipGetLastError();
}

}  // namespace i8l
