// Backward pass of the mixed int8/fp16 training mode.
//
// [blog, "Usage"]: with has_fp16_weights=True (the default) the layer keeps
// its fp16 weight for training in mixed int8/fp16 precision.  The pages give
// no gradient path; the one implemented here treats the quantization as the
// identity, so the gradients are those of the product X . W:
//   dX = dY . W^T           (fp16 operands, fp32 accumulation, fp16 result)
//   dW = X^T . dY           (the same, in the weight's math layout [K][N])
//   dbias[n] = sum_i dY[i][n]
// Both products run on the fp16 matrix cores through the GEMM of gemm.hip,
// which wants both operands contiguous along the summed dimension.  dX's
// operands already are (dY [M][N], W [K][N] both run along N).  dW sums over
// the rows i, so X and dY are first transposed into the workspace (rows
// padded with zeros to a multiple of 8, whole 16-byte chunks); the transpose
// of dY also forms the per-tile column sums of the bias gradient, which a
// last small kernel adds up in a fixed order (deterministic).
#include "common.h"
#include "launch.h"

namespace i8l {

constexpr int kTr = 64;            // transpose tile: 64 x 64 fp16
constexpr int kTrThreads = 256;
constexpr int kTrPad = kTr + 2;    // LDS row: 33 dwords, so a column read hits 64 banks

// out[c][r] = in[r][c] for r < R, c < C; out rows have stride Rp (a multiple of
// 8, >= R) and hold 0 for r in [R, Rp).  C % 8 == 0 (whole 16-byte chunks).
// colsum (optional): colsum[blockIdx.y][c] = sum of the tile's 64 rows of
// column c, in fp32, rows in ascending order.
// grid = (ceil(C / 64), ceil(Rp / 64)).
__global__ __launch_bounds__(kTrThreads) void transpose_f16_kernel(
    const uint16_t* __restrict__ in, int R, int C, int Rp, uint16_t* __restrict__ out,
    float* __restrict__ colsum) {
  __shared__ uint16_t tile[kTr][kTrPad];
  const int t = threadIdx.x;
  const int c0 = blockIdx.x * kTr, r0 = blockIdx.y * kTr;
  // load: 64 rows x 8 chunks of 8 values, two chunks per thread
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = t + i * kTrThreads, row = q >> 3, ch = q & 7;
    const int r = r0 + row, c = c0 + ch * 8;
    v4i v = v4i{0, 0, 0, 0};
    if (r < R && c < C) v = *reinterpret_cast<const v4i*>(in + (size_t)r * C + c);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      tile[row][ch * 8 + 2 * d] = (uint16_t)((uint32_t)v[d] & 0xffffu);
      tile[row][ch * 8 + 2 * d + 1] = (uint16_t)((uint32_t)v[d] >> 16);
    }
  }
  __syncthreads();
  if (colsum && t < kTr && c0 + t < C) {
    float s = 0.0f;
    for (int row = 0; row < kTr; ++row) s += h2f(tile[row][t]);
    colsum[(size_t)blockIdx.y * C + c0 + t] = s;
  }
  // store: 64 output rows (columns c) x 8 chunks of 8 values (rows r)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = t + i * kTrThreads, orow = q >> 3, ch = q & 7;
    const int c = c0 + orow, r = r0 + ch * 8;
    if (c < C && r < Rp) {
      uint32_t w[4];
#pragma unroll
      for (int d = 0; d < 4; ++d)
        w[d] = (uint32_t)tile[ch * 8 + 2 * d][orow] | ((uint32_t)tile[ch * 8 + 2 * d + 1][orow] << 16);
      *reinterpret_cast<v4i*>(out + (size_t)c * Rp + r) =
          v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
  }
}

// db[c] = fp16(sum over t < T of colsum[t][c]), t ascending.
__global__ void bias_grad_kernel(const float* __restrict__ colsum, int T, int C,
                                 uint16_t* __restrict__ db) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  float s = 0.0f;
  for (int t = 0; t < T; ++t) s += colsum[(size_t)t * C + c];
  db[c] = f2h(s);
}

int train_pad_rows(int M) { return (M + 7) / 8 * 8; }

size_t backward_weight_workspace(int M, int K, int N, size_t* off_xt, size_t* off_dyt,
                                 size_t* off_part) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t Mp = (size_t)train_pad_rows(M);
  size_t off = 0;
  *off_xt = off;
  off += up((size_t)K * Mp * 2);
  *off_dyt = off;
  off += up((size_t)N * Mp * 2);
  *off_part = off;
  off += up((Mp + kTr - 1) / kTr * (size_t)N * 4);
  return off;
}

hipError_t launch_backward_input(const uint16_t* dY, const uint16_t* W, int M, int K, int N,
                                 uint16_t* dX, hipStream_t stream) {
  // dX [M][K] = dY [M][N] . (W [K][N])^T: the sum runs along N in both
  return launch_gemm_f16(dY, W, M, K, N, dX, stream);
}

hipError_t launch_backward_weight(const uint16_t* X, const uint16_t* dY, int M, int K, int N,
                                  uint16_t* dW, uint16_t* dbias, void* workspace,
                                  hipStream_t stream) {
  if (M == 0) {   // no rows: every gradient entry is an empty sum
    // K % 16 == 0, so dW holds K * N / 2 whole words; cleared in pieces below 2^30
    const size_t words = (size_t)K * N / 2;
    for (size_t w0 = 0; w0 < words; w0 += (size_t)1 << 30) {
      const size_t n = words - w0 < ((size_t)1 << 30) ? words - w0 : ((size_t)1 << 30);
      hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(dW) + w0, (int)n, 0u, stream);
      if (e != hipSuccess) return e;
    }
    if (!dbias) return hipSuccess;
    return launch_fill_u32(reinterpret_cast<uint32_t*>(dbias), N / 2, 0u, stream);   // N % 8 == 0
  }
  size_t oxt, odyt, opart;
  backward_weight_workspace(M, K, N, &oxt, &odyt, &opart);
  char* ws = static_cast<char*>(workspace);
  uint16_t* XT = reinterpret_cast<uint16_t*>(ws + oxt);
  uint16_t* dYT = reinterpret_cast<uint16_t*>(ws + odyt);
  float* part = reinterpret_cast<float*>(ws + opart);
  const int Mp = train_pad_rows(M);
  const int T = (Mp + kTr - 1) / kTr;
  hipLaunchKernelGGL(transpose_f16_kernel, dim3((K + kTr - 1) / kTr, T), dim3(kTrThreads), 0,
                     stream, X, M, K, Mp, XT, (float*)nullptr);
  hipLaunchKernelGGL(transpose_f16_kernel, dim3((N + kTr - 1) / kTr, T), dim3(kTrThreads), 0,
                     stream, dY, M, N, Mp, dYT, dbias ? part : (float*)nullptr);
  // dW [K][N] = XT [K][Mp] . (dYT [N][Mp])^T
  hipError_t e = launch_gemm_f16(XT, dYT, K, N, Mp, dW, stream);
  if (e != hipSuccess || !dbias) return e;
  hipLaunchKernelGGL(bias_grad_kernel, dim3((N + 255) / 256), dim3(256), 0, stream,
                     (const float*)part, T, N, dbias);
  return hipGetLastError();
}

}  // namespace i8l
