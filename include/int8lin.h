/*
 * int8lin.h -- C ABI of the LLM.int8() quantized linear layer for AMD MI355X
 * (gfx950).  Implemented by libint8lin.so (hand-written HIP kernels).
 *
 * The method is the one described in the blog "A Gentle Introduction to 8-bit
 * Matrix Multiplication for transformers at scale using Hugging Face
 * Transformers, Accelerate and bitsandbytes" (cited as [blog] below):
 *   - vector-wise absmax quantization: one scale per row of the fp16 hidden
 *     states X and one per output column of the weight W
 *     ([blog, "Introduction to model quantization"]);
 *   - mixed-precision decomposition: a column of X holding any value of
 *     magnitude >= threshold (6 in the blog) is an outlier column; outlier
 *     columns are multiplied in fp16 against the matching fp16 rows of W, the
 *     rest in int8 x int8 -> int32; the int8 result is dequantized with the
 *     outer product of the scales over 127^2 and added to the fp16 outlier
 *     product ([blog, "A gentle summary of LLM.int8()"] and
 *     [blog, "A closer look at the MatMul"]).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers (HBM of the current HIP device) and
 *     are row-major.  fp16 tensors are passed as raw IEEE binary16 bits
 *     (uint16_t).  The caller owns and allocates every buffer; the library
 *     allocates no device memory and keeps no state besides a thread-local
 *     error message.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL means the
 *     default stream) and returns without synchronizing.  Device-side faults
 *     surface at the caller's next synchronization.
 *   - All argument checks run on the host before any HIP call; on a non-OK
 *     status nothing has been enqueued and i8l_last_error() tells why.
 *   - Shapes: M (rows of X) >= 0, N (output features) >= 0; M == 0 or N == 0
 *     is a valid no-op.  K (input features) must satisfy 16 <= K <= 133136 and
 *     K % 16 == 0 (K * 127^2 must fit in int32).
 *   - Alignment: X, Y, Wq, Xq, acc, X_outliers and workspace pointers must be
 *     16-byte aligned; sw, sx, outlier_idx and n_outliers 4-byte aligned; W and
 *     W_outlier_rows 2-byte aligned.
 *   - Rounding: quantized codes are clamp(round_half_away_from_zero(
 *     fp32(x) * fl32(127 / absmax)), -127, 127), with 127 / absmax an IEEE fp32
 *     division; absmax == 0 gives code 0.
 *   - Functions are reentrant; calls that share a workspace must not overlap.
 */
#ifndef INT8LIN_H
#define INT8LIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  I8L_OK = 0,
  I8L_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad shape, NaN threshold */
  I8L_ERR_K_TOO_LARGE = 2, /* K > 133136: int32 accumulators could overflow */
  I8L_ERR_WORKSPACE = 3,   /* workspace smaller than required */
  I8L_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} i8l_status;

/* Largest supported K (K * 127 * 127 < 2^31, rounded down to a multiple of 16). */
#define I8L_MAX_K 133136

/* Largest K of the zero-point entry points (K * 255 * 127 < 2^31, a multiple
 * of 16): every sum_k (q - zp) * w then fits in int32. */
#define I8L_MAX_K_ZP 66304

/* Byte offsets, inside the int8_linear / int8_quantize_activation workspace, of
 * the intermediates that the call leaves there.  After an int8_linear call
 * (once the stream has reached it) the workspace holds, for that call:
 *   n_outliers   int32 [1]        number of outlier columns n_out
 *   outlier_idx  int32 [K] cap    ascending outlier column indices, first n_out
 *   sx           fp32  [M]        row absmax of X over the regular columns
 *   Xq           int8  [M][K]     row-quantized X, 0 in outlier columns
 *   X_outliers   fp16  [M][K] cap outlier values, element (i, j) at i*K + j,
 *                                 j < n_out, j-th outlier column in ascending order
 *   flags        uint32 [ceil(K/32)] internal: outlier column bitmask
 *   zero_points  int32 [M]        int8_linear_zp only: the row zero points;
 *                                 sx then holds range / 255 and Xq the codes
 *                                 minus 128 (see int8_quantize_activation_zp);
 *                                 internal for absmax codes
 *   act_partials uint32           internal (1 <= M <= 16): per 512-column
 *                                 slice of K, its outlier count and per-row
 *                                 partial maxima / minima of the activation
 *                                 stage (0 bytes for other M)
 *   gemm_counters, gemm_partials   internal (M > 64): a reserved region and
 *                                 int32 partial tiles of the GEMM's split-K
 *                                 tail; gemm_slices partial tiles of 256x256
 * `total` is the size the call requires; it depends on M, K and N. */
typedef struct {
  size_t total;
  size_t n_outliers;
  size_t outlier_idx;
  size_t sx;
  size_t Xq;
  size_t X_outliers;
  size_t flags;
  size_t gemm_counters;
  size_t gemm_partials;
  size_t gemm_slices;
  size_t zero_points;
  size_t act_partials;
} i8l_workspace_layout;

/* Fills *layout for an int8_linear call of this shape.
 * Returns I8L_ERR_INVALID_ARG / I8L_ERR_K_TOO_LARGE on a bad shape. */
i8l_status i8l_linear_workspace(int64_t M, int64_t K, int64_t N, i8l_workspace_layout *layout);

/* Workspace bytes int8_linear needs for this shape (0 on a bad shape). */
size_t i8l_linear_workspace_bytes(int64_t M, int64_t K, int64_t N);

/* Weight quantization ([blog, "A closer look at the MatMul"]: the weight is
 * quantized per column; [blog, "Usage"]: it happens once, when the layer is
 * placed on the GPU, and keeps the int8 weight in nn.Linear's [out][in] layout
 * next to one absmax per output feature).
 *   W   fp16 [K][N]  math layout (Y = X @ W), read only
 *   Wq  int8 [N][K]  out: Wq[n][k] = code(W[k][n], sw[n])
 *   sw  fp32 [N]     out: sw[n] = max_k |W[k][n]| */
i8l_status int8_quantize_weight(const uint16_t *W, int64_t K, int64_t N,
                                int8_t *Wq, float *sw, void *stream);

/* The LLM.int8() linear layer: Y = dequant(int8 part) + fp16 outlier part.
 *   X               fp16 [M][K]  hidden states, read only
 *   Wq, sw          from int8_quantize_weight for the same K, N
 *   W_outlier_rows  fp16 [K][N]  the fp16 weight in math layout; only rows
 *                   that are outlier columns of X are read.  NULL: no fp16
 *                   weight is kept, and each outlier weight value is rebuilt
 *                   from its code as fp16(fl32(Wq[n][k] * sw[n]) / 127)
 *                   ([blog, "Usage"]: the int8 weight times its per-output
 *                   scale over 127 gives the weight back).
 *   threshold       finite > 0: columns of X with any |x| >= threshold are
 *                   outliers; <= 0 or +inf: no decomposition (pure int8);
 *                   NaN: I8L_ERR_INVALID_ARG.
 *   Y               fp16 [M][N]  out: fp16(acc*sx[i]*sw[n]/127^2 + outlier
 *                   product), accumulated in fp32, round-to-nearest-even,
 *                   overflow to +/-inf.
 *   workspace       device scratch of i8l_linear_workspace_bytes(M, K, N)
 *                   bytes; it holds the call's intermediates afterwards (see
 *                   i8l_workspace_layout). */
i8l_status int8_linear(const uint16_t *X, int64_t M, int64_t K,
                       const int8_t *Wq, const float *sw, int64_t N,
                       const uint16_t *W_outlier_rows, float threshold,
                       uint16_t *Y, void *workspace, size_t workspace_bytes,
                       void *stream);

/* int8_linear with a bias, for a linear layer that has one ([blog, "Usage"]:
 * the 8-bit layer takes nn.Linear's bias argument).
 *   bias   fp16 [N], 2-byte aligned, or NULL (then identical to int8_linear);
 *          Y = fp16(acc*sx[i]*sw[n]/127^2 + outlier product + bias[n]), the sum
 *          formed in fp32 and rounded once.
 * Every other argument, and every error, as for int8_linear. */
i8l_status int8_linear_bias(const uint16_t *X, int64_t M, int64_t K,
                            const int8_t *Wq, const float *sw, int64_t N,
                            const uint16_t *W_outlier_rows, const uint16_t *bias,
                            float threshold, uint16_t *Y, void *workspace,
                            size_t workspace_bytes, void *stream);

/* int8_linear_bias without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The intermediates go to a static scratch
 * array of I8L_STATIC_SCRATCH_BYTES inside the library, one copy per GPU,
 * allocated when the library's code is loaded on that GPU and held until the
 * process ends; the call itself allocates nothing.  Every call on a GPU uses
 * that GPU's one array, so calls that overlap on one GPU (other streams, other
 * host threads) race and must be serialized by the caller; the array keeps the
 * last call's intermediates, and nothing in it needs to start at zero.
 * Arguments, results and errors as for int8_linear_bias, except: a shape
 * whose workspace (i8l_linear_workspace_bytes, less the GEMM's split-K partial
 * tiles if only that makes it fit, in which case every output tile is
 * computed whole) exceeds I8L_STATIC_SCRATCH_BYTES gives I8L_ERR_WORKSPACE
 * with nothing enqueued.  Fits, for example: every M <= 64 with K <= 133136,
 * and M = 2048 with K = 4096. */
#define I8L_STATIC_SCRATCH_BYTES (32u << 20)
i8l_status int8_linear_static(const uint16_t *X, int64_t M, int64_t K,
                              const int8_t *Wq, const float *sw, int64_t N,
                              const uint16_t *W_outlier_rows, const uint16_t *bias,
                              float threshold, uint16_t *Y, void *stream);

/* Activation stage on its own ([blog, "A gentle summary of LLM.int8()"],
 * step 1, and the row-wise quantization of [blog, "A closer look at the
 * MatMul"]); the same kernels int8_linear runs for M > 16.
 *   Xq          int8 [M][K]      out, 0 in outlier columns
 *   sx          fp32 [M]         out
 *   outlier_idx int32 [K] cap    out, ascending, first n_out entries valid
 *   n_outliers  int32 [1]        out
 *   X_outliers  fp16 [M][K] cap  out, element (i, j) at i*K + j for j < n_out
 *   workspace   at least i8l_linear_workspace_bytes(M, K, 0) bytes */
i8l_status int8_quantize_activation(const uint16_t *X, int64_t M, int64_t K, float threshold,
                                    int8_t *Xq, float *sx, int32_t *outlier_idx,
                                    int32_t *n_outliers, uint16_t *X_outliers,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* Exact int8 GEMM on its own ([blog, "Introduction to model quantization"]:
 * the normalised int8 matrices are multiplied), the kernel int8_linear uses
 * for M > 64 with its int32 result written out instead of dequantized.
 *   Xq         int8 [M][K]
 *   Wq         int8 [N][K]
 *   acc        int32 [M][N]  out: acc[i][n] = sum_k Xq[i][k] * Wq[n][k]
 *   workspace  NULL: every 256x256 output tile is computed whole.  Otherwise
 *              at least i8l_linear_workspace_bytes(M, K, N) bytes, 16-byte
 *              aligned: the tiles of a partial last round over the compute
 *              units are then split along K, their int32 partials stored in
 *              the workspace and summed by a fix-up launch, exactly as in
 *              int8_linear (too small: I8L_ERR_WORKSPACE).  The result is the
 *              same exact integer either way. */
i8l_status int8_gemm_i32(const int8_t *Xq, const int8_t *Wq, int64_t M, int64_t N, int64_t K,
                         int32_t *acc, void *workspace, size_t workspace_bytes, void *stream);

/* ---- Zero-point variant ----------------------------------------------------
 * [blog, "Introduction to model quantization"] describes, next to absmax, the
 * unsigned int8 scheme: subtract the minimum, scale the range onto [0, 255],
 * and round the image of 0 to an integer, the zero point.  Here X is quantized
 * that way per row (over the regular columns; the outlier decomposition is the
 * same as in int8_linear) and the weight keeps its absmax codes per output
 * feature:
 *   lo = min(0, min_k x), hi = max(0, max_k x) over the row's regular columns,
 *   inv = fl32(255 / fl32(hi - lo))  (0 when hi == lo),
 *   zp = round_half_away(fl32(-lo * inv)),
 *   q = clamp(round_half_away(fl32(x * inv)) + zp, 0, 255),
 *   xscale = fl32(fl32(hi - lo) / 255);
 * outlier columns take q = zp (the code of 0).  Codes are stored as q - 128
 * (int8) so the int8 matrix cores multiply them; the layer uses
 *   sum_k (q - zp) w = sum_k (q - 128) w + (128 - zp) S[n],  S[n] = sum_k Wq[n][k],
 * exact in int32 for K <= I8L_MAX_K_ZP, and
 *   Y = fp16(acc * xscale[i] * sw[n] / 127 + outlier product + bias[n]).
 * X must be finite in its regular columns (a non-finite value there makes the
 * codes of that row unspecified; with the decomposition on, +-inf is always an
 * outlier). */

/* S[n] = sum_k Wq[n][k] (int32), the per-output correction term of the
 * zero-point variant; computed once per layer, like the weight codes.
 *   Wq  int8 [N][K]  16-byte aligned, read only
 *   S   int32 [N]    out, 4-byte aligned
 * Shape rules as for int8_quantize_weight. */
i8l_status int8_weight_code_sums(const int8_t *Wq, int64_t N, int64_t K, int32_t *S,
                                 void *stream);

/* The layer with zero-point activation codes (see above).
 *   wsum   int32 [N] from int8_weight_code_sums for this Wq, 4-byte aligned
 * Every other argument, the workspace size and the errors as for
 * int8_linear_bias; in addition K > I8L_MAX_K_ZP gives I8L_ERR_K_TOO_LARGE.
 * Afterwards the workspace holds Xq (q - 128), sx (xscale), zero_points, the
 * outlier list and X_outliers of this call. */
i8l_status int8_linear_zp(const uint16_t *X, int64_t M, int64_t K,
                          const int8_t *Wq, const float *sw, const int32_t *wsum, int64_t N,
                          const uint16_t *W_outlier_rows, const uint16_t *bias,
                          float threshold, uint16_t *Y, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Activation stage of the zero-point variant on its own.
 *   Xq      int8 [M][K]  out: q - 128, zp - 128 in outlier columns
 *   zp      int32 [M]    out: zero points in [0, 255]
 *   xscale  fp32 [M]     out: fl32(range / 255)
 * Other arguments, alignment, workspace and errors as for
 * int8_quantize_activation; K > I8L_MAX_K_ZP gives I8L_ERR_K_TOO_LARGE. */
i8l_status int8_quantize_activation_zp(const uint16_t *X, int64_t M, int64_t K, float threshold,
                                       int8_t *Xq, int32_t *zp, float *xscale,
                                       int32_t *outlier_idx, int32_t *n_outliers,
                                       uint16_t *X_outliers, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* ---- Mixed int8/fp16 training mode -----------------------------------------
 * [blog, "Usage"]: has_fp16_weights=True (the default) keeps the fp16 weight
 * for training in mixed int8/fp16 precision.  The pages describe no gradient
 * path; the one provided here treats the quantization as the identity: the
 * forward pass is int8_quantize_weight on the current fp16 weight followed by
 * int8_linear_bias with that weight as W_outlier_rows, and the gradients are
 * those of Y = X . W + bias, formed from fp16 operands with fp32 accumulation
 * and rounded once to fp16 (round to nearest even, overflow to +/-inf).
 * Shapes: M >= 0, K as for int8_linear, N >= 0 with N % 8 == 0. */

/* Workspace bytes int8_linear_backward_weight needs (0 on a bad shape):
 * X^T and dY^T with their rows padded to a multiple of 8, and the bias
 * gradient's partial sums. */
size_t i8l_backward_weight_workspace_bytes(int64_t M, int64_t K, int64_t N);

/* dX = dY . W^T.
 *   dY  fp16 [M][N]  gradient of the layer's output, 16-byte aligned
 *   W   fp16 [K][N]  the fp16 weight in math layout, 16-byte aligned
 *   dX  fp16 [M][K]  out, 16-byte aligned
 * M == 0: no-op.  N == 0: dX = 0 (dY and W may then be NULL). */
i8l_status int8_linear_backward_input(const uint16_t *dY, const uint16_t *W, int64_t M,
                                      int64_t K, int64_t N, uint16_t *dX, void *stream);

/* dW = X^T . dY and dbias[n] = sum_i dY[i][n].
 *   X       fp16 [M][K]  the layer's input, 16-byte aligned
 *   dY      fp16 [M][N]  16-byte aligned
 *   dW      fp16 [K][N]  out (the weight's math layout), 16-byte aligned
 *   dbias   fp16 [N]     out, 4-byte aligned, or NULL (not computed)
 *   workspace  at least i8l_backward_weight_workspace_bytes(M, K, N) bytes,
 *              16-byte aligned (may be NULL when M == 0)
 * M == 0: dW = 0 and dbias = 0.  N == 0: no-op. */
i8l_status int8_linear_backward_weight(const uint16_t *X, const uint16_t *dY, int64_t M,
                                       int64_t K, int64_t N, uint16_t *dW, uint16_t *dbias,
                                       void *workspace, size_t workspace_bytes, void *stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *i8l_last_error(void);

/* Static build description: target architecture and kernel tile sizes. */
const char *i8l_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* INT8LIN_H */
