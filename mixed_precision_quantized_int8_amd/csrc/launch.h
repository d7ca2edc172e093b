// Internal launchers of the gfx950 kernels; the C ABI (int8lin_abi.hip) calls
// these after validating its arguments on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace i8l {

// Workspace carving shared by int8_linear and int8_quantize_activation.
struct Workspace {
  int32_t* n_out;      // [1]
  int32_t* idx;        // [K]
  float* sx;           // [M] absmax, or range / 255 in zero-point mode
  int32_t* zp;         // [M] zero points (zero-point mode only)
  int8_t* Xq;          // [M][K]
  uint16_t* X_O;       // [M][K] capacity, row stride K
  uint32_t* flags;     // [ceil(K/32)]
  int32_t* gemm_cnt;   // [kGemmMaxSlices] reserved (unused)
  int32_t* gemm_part;  // [gemm_slices][256][256] int32 partial tiles
  int gemm_slices;     // partial tiles the workspace holds
  uint32_t* act_part;  // M <= 16: per 512-column slice, the outlier count, then
                       // the row partials (see launch_quantize_activation)
};

// Split-K tail of the GEMM: the tiles of the last, partial round over the
// compute units are split along K so that the round fills the chip.
constexpr int kGemmMaxSlices = 256;
struct GemmSplit {
  int full_tiles;    // tiles computed whole (a multiple of the CU count)
  int split_tiles;   // tiles after them, each split into S K ranges
  int S;
};
GemmSplit gemm_split_plan(int M, int N, int K, int cus);

// p[0 .. n) = v, as a kernel (a fill kernel rather than a memset node keeps the
// sequence safe to capture in a HIP graph).
hipError_t launch_fill_u32(uint32_t* p, int n, uint32_t v, hipStream_t stream);

hipError_t launch_quantize_weight(const uint16_t* W, int K, int N, int8_t* Wq, float* sw,
                                  hipStream_t stream);

// Outlier column scan + row quantization: for M > 16 two kernels after a flag
// clear; for 1 <= M <= 16 two kernels over 512-column slices that pass
// per-slice outlier counts and row partials through ws.act_part
// ([act_slices(K)] counts, then [act_slices(K)][16] row maxima, then, in
// zero-point mode, [act_slices(K)][16] row minima).
// `enabled` false skips the scan: no column is an outlier.  `zp`: zero-point
// codes (stored minus 128), range / 255 in ws.sx and the zero points in ws.zp.
constexpr int kActSlice = 512;
constexpr int kActSmallRows = 16;
inline int act_slices(int K) { return (K + kActSlice - 1) / kActSlice; }
hipError_t launch_quantize_activation(const uint16_t* X, int M, int K, float threshold,
                                      bool enabled, const Workspace& ws, hipStream_t stream,
                                      bool zp = false);

// S[n] = sum_k Wq[n][k] (the zero-point correction of the int8 product).
hipError_t launch_weight_code_sums(const int8_t* Wq, int N, int K, int32_t* S,
                                   hipStream_t stream);

// int8 GEMM on the matrix cores.  With Y != nullptr: dequantize with sx/sw, add
// the fp16 outlier product (X_O against rows idx of W_rows) and store fp16 Y.
// With acc != nullptr: store the raw int32 accumulators instead.  Either way,
// given partial-tile space (part, part_slices) the tiles of a partial last
// round are split along K and summed by a fix-up launch.
struct GemmArgs {
  const int8_t* Xq;
  const int8_t* Wq;
  int M, N, K;
  const float* sx;
  const float* sw;
  const int32_t* n_out;
  const int32_t* idx;
  const uint16_t* X_O;      // row stride K
  const uint16_t* W_rows;   // [K][N]
  uint16_t* Y;
  int32_t* acc;
  const uint16_t* bias;   // fp16 [N] added before the final rounding, or NULL
  // zero-point mode (zp != NULL): Xq holds q - 128 and sx the row's range / 255;
  // the accumulator becomes acc + (128 - zp[m]) * wsum[n] (exact in int32) and
  // is dequantized with sx * sw / 127
  const int32_t* zp;
  const int32_t* wsum;
  int32_t* cnt;      // split-K tail: reserved (unused) / partials
  int32_t* part;
  int part_slices;   // 0: never split
  // set by launch_gemm
  int full_tiles, split_S;
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);

// The same product and epilogue with 256 x 64 tiles and no split along K
// (skinny.hip), for kStreamMaxM < M <= kSkinnyMaxM: weight-bound batches,
// where 256 x 256 tiles would leave most compute units idle.
constexpr int kSkinnyMaxM = 256;
hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream);

// Small-M (decode) path, M <= kStreamMaxM: when decode_fits(M, K) (M <= 16,
// K <= 4096) one fused kernel does the activation stage, the int8 product,
// the outlier product and the epilogue; otherwise the activation kernels run
// first and a weight-streaming kernel does the rest.
constexpr int kStreamMaxM = 64;
bool decode_fits(int M, int K);
hipError_t launch_decode(const uint16_t* X, int M, int K, const int8_t* Wq, const float* sw,
                         int N, const uint16_t* W_rows, const uint16_t* bias, float threshold,
                         bool enabled, uint16_t* Y, const Workspace& ws, hipStream_t stream);
// Zero-point mode for M <= kStreamMaxM: the fused kernel when decode_fits(M, K), else the
// activation kernels (zero-point codes), then the streaming kernel with the
// corrected epilogue.
hipError_t launch_decode_zp(const uint16_t* X, int M, int K, const int8_t* Wq, const float* sw,
                            const int32_t* wsum, int N, const uint16_t* W_rows,
                            const uint16_t* bias, float threshold, bool enabled, uint16_t* Y,
                            const Workspace& ws, hipStream_t stream);

// C [M][N] = A [M][K] . B [N][K]^T, fp16 operands (K-contiguous, K % 8 == 0,
// 16-byte aligned rows), fp32 accumulation, fp16 result (round to nearest
// even); the int8 GEMM's tiles and pipeline on the fp16 matrix cores.
hipError_t launch_gemm_f16(const uint16_t* A, const uint16_t* B, int M, int N, int K,
                           uint16_t* C, hipStream_t stream);

// Training-mode backward (train.hip).  N % 8 == 0; 16-byte aligned operands.
// dX [M][K] = dY [M][N] . W^T  (W [K][N]).
hipError_t launch_backward_input(const uint16_t* dY, const uint16_t* W, int M, int K, int N,
                                 uint16_t* dX, hipStream_t stream);
// dW [K][N] = X^T . dY, dbias [N] = column sums of dY (optional); the
// workspace holds X^T, dY^T (rows padded to a multiple of 8) and the bias
// partial sums, laid out by backward_weight_workspace.
size_t backward_weight_workspace(int M, int K, int N, size_t* off_xt, size_t* off_dyt,
                                 size_t* off_part);
hipError_t launch_backward_weight(const uint16_t* X, const uint16_t* dY, int M, int K, int N,
                                  uint16_t* dW, uint16_t* dbias, void* workspace,
                                  hipStream_t stream);

const char* gemm_tile_info();

}  // namespace i8l
