// Weight quantization: per-output-feature absmax codes of an fp16 weight.
//
// [blog, "A closer look at the MatMul"]: the weight matrix is quantized column
// by column (one absmax per output feature of Y = X @ W).  [blog, "Usage"]:
// the quantization runs once when the layer is placed on the GPU and the int8
// weight keeps nn.Linear's [out][in] layout, here Wq[N][K] (K contiguous),
// which is also the layout the int8 matrix cores read.
//
// Two launches after clearing sw (a fill kernel, safe under graph capture):
//   wabsmax  the column maxima: each workgroup reduces |W| over a chunk of
//            1024 rows of a strip of 512 output features (16-byte loads,
//            whole 128-byte lines per 8 lanes) and merges its maxima into sw
//            with an integer atomicMax on the fp32 bits (the order of
//            non-negative floats is that of their bit patterns);
//   wcode    the codes: each workgroup takes a tile of 128 rows (k) x 64
//            output features, reads it once (128-byte row pieces), holds it
//            in LDS and writes Wq[n][k0 .. k0+128) as whole 128-byte runs.
// The weight is read twice (every code needs its column's absmax over all K)
// and the codes written once: 2.5 bytes of traffic per weight element.
#include "common.h"
#include "launch.h"

namespace i8l {

constexpr int kWaStrip = 512;    // wabsmax: output features per workgroup (8 per lane)
constexpr int kWaRows = 1024;    // wabsmax: rows per workgroup
constexpr int kWaThreads = 256;
constexpr int kWcK = 128;        // wcode: rows (k) per tile
constexpr int kWcN = 64;         // wcode: output features per tile
constexpr int kWcThreads = 256;

// grid = (ceil(N / 512), ceil(K / 1024)); sw cleared beforehand.
// VEC: N % 8 == 0 and W 16-byte aligned (whole 16-byte pieces per lane).
template <bool VEC>
__global__ __launch_bounds__(kWaThreads) void wabsmax_kernel(const uint16_t* __restrict__ W,
                                                            int K, int N,
                                                            float* __restrict__ sw) {
  __shared__ uint32_t red[kWaThreads / 64][kWaStrip];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * kWaStrip + lane * 8;
  const int k0 = blockIdx.y * kWaRows;
  const int k1 = min(K, k0 + kWaRows);
  uint32_t mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mx[e] = 0;
  if (VEC && c < N) {
    // four rows in flight per lane
    int k = k0 + wave;
    for (; k + 12 < k1; k += 16) {
      v4i r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        r[u] = *reinterpret_cast<const v4i*>(W + (size_t)(k + 4 * u) * N + c);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t b = habs_bits(((uint32_t)r[u][e >> 1] >> ((e & 1) * 16)) & 0xffffu);
          mx[e] = b > mx[e] ? b : mx[e];
        }
    }
    for (; k < k1; k += 4) {
      const v4i r = *reinterpret_cast<const v4i*>(W + (size_t)k * N + c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t b = habs_bits(((uint32_t)r[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
        mx[e] = b > mx[e] ? b : mx[e];
      }
    }
  } else if (!VEC) {
    for (int k = k0 + wave; k < k1; k += 4) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c + e < N) {
          const uint32_t b = habs_bits(W[(size_t)k * N + c + e]);
          mx[e] = b > mx[e] ? b : mx[e];
        }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = mx[e];
  __syncthreads();
  for (int j = threadIdx.x; j < kWaStrip; j += kWaThreads) {
    uint32_t m = red[0][j];
#pragma unroll
    for (int w = 1; w < kWaThreads / 64; ++w) m = red[w][j] > m ? red[w][j] : m;
    const int n = blockIdx.x * kWaStrip + j;
    if (n < N && m != 0)
      atomicMax(reinterpret_cast<unsigned int*>(sw) + n, __float_as_uint(h2f((uint16_t)m)));
  }
}

// grid = (ceil(N / 64), ceil(K / 128)).  Tile: rows k0 .. k0+127 (K % 16 == 0,
// so a row is either wholly inside or past K in 16-code pieces) x output
// features n0 .. n0+63.
template <bool VEC>
__global__ __launch_bounds__(kWcThreads) void wcode_kernel(const uint16_t* __restrict__ W, int K,
                                                          int N, const float* __restrict__ sw,
                                                          int8_t* __restrict__ Wq) {
  __shared__ uint16_t tile[kWcK][kWcN + 2];   // 33 dwords per row: column reads spread banks
  __shared__ float inv_s[kWcN];
  const int t = threadIdx.x;
  const int n0 = blockIdx.x * kWcN, k0 = blockIdx.y * kWcK;
  if (t < kWcN) inv_s[t] = n0 + t < N ? quant_scale(sw[n0 + t]) : 0.0f;
  // load: 128 rows x 8 pieces of 8 values, four pieces per thread
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = t + i * kWcThreads, row = q >> 3, ch = q & 7;
    const int k = k0 + row, c = n0 + ch * 8;
    uint32_t v[4] = {0, 0, 0, 0};
    if (VEC) {
      if (k < K && c < N) {
        const v4i r = *reinterpret_cast<const v4i*>(W + (size_t)k * N + c);
#pragma unroll
        for (int d = 0; d < 4; ++d) v[d] = (uint32_t)r[d];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k < K && c + e < N) v[e >> 1] |= (uint32_t)W[(size_t)k * N + c + e] << ((e & 1) * 16);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      tile[row][ch * 8 + 2 * d] = (uint16_t)(v[d] & 0xffffu);
      tile[row][ch * 8 + 2 * d + 1] = (uint16_t)(v[d] >> 16);
    }
  }
  __syncthreads();
  // store: 64 output features x 8 pieces of 16 codes, two pieces per thread
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = t + i * kWcThreads, nl = q >> 3, ch = q & 7;
    const int n = n0 + nl, k = k0 + ch * 16;
    if (n < N && k < K) {
      const float inv = inv_s[nl];
      uint32_t w[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        w[g] = pack4_i8(quant_code(h2f(tile[ch * 16 + 4 * g + 0][nl]), inv),
                        quant_code(h2f(tile[ch * 16 + 4 * g + 1][nl]), inv),
                        quant_code(h2f(tile[ch * 16 + 4 * g + 2][nl]), inv),
                        quant_code(h2f(tile[ch * 16 + 4 * g + 3][nl]), inv));
      *reinterpret_cast<v4i*>(Wq + (size_t)n * K + k) =
          v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
  }
}

hipError_t launch_quantize_weight(const uint16_t* W, int K, int N, int8_t* Wq, float* sw,
                                  hipStream_t stream) {
  hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(sw), N, 0u, stream);
  if (e != hipSuccess) return e;
  const bool vec = (N % 8 == 0) && ((uintptr_t)W % 16 == 0);
  const dim3 ga((N + kWaStrip - 1) / kWaStrip, (K + kWaRows - 1) / kWaRows);
  const dim3 gc((N + kWcN - 1) / kWcN, (K + kWcK - 1) / kWcK);
  if (vec) {
    hipLaunchKernelGGL(wabsmax_kernel<true>, ga, dim3(kWaThreads), 0, stream, W, K, N, sw);
    hipLaunchKernelGGL(wcode_kernel<true>, gc, dim3(kWcThreads), 0, stream, W, K, N,
                       (const float*)sw, Wq);
  } else {
    hipLaunchKernelGGL(wabsmax_kernel<false>, ga, dim3(kWaThreads), 0, stream, W, K, N, sw);
    hipLaunchKernelGGL(wcode_kernel<false>, gc, dim3(kWcThreads), 0, stream, W, K, N,
                       (const float*)sw, Wq);
  }
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
