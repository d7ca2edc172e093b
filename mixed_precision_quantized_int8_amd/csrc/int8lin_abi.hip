// C ABI of the LLM.int8() linear layer (declared in include/int8lin.h).
//
// Every entry point validates its arguments on the host before making any HIP
// call, so a bad call returns an error code with nothing enqueued.  Then it
// carves the caller's workspace and enqueues the kernels on the caller's
// stream; it never synchronizes and never allocates device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>

#include "../../include/int8lin.h"
#include "launch.h"

#define I8L_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

i8l_status fail(i8l_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

i8l_status ok() {
  g_err[0] = 0;
  return I8L_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Shape rules shared by all entry points.
i8l_status check_shape(const char* fn, int64_t M, int64_t K, int64_t N) {
  if (M < 0 || N < 0) return fail(I8L_ERR_INVALID_ARG, "%s: M=%lld and N=%lld must be >= 0", fn,
                                  (long long)M, (long long)N);
  if (K > I8L_MAX_K)
    return fail(I8L_ERR_K_TOO_LARGE, "%s: K=%lld exceeds %d (K*127^2 must fit in int32)", fn,
                (long long)K, I8L_MAX_K);
  if (K < 16 || K % 16 != 0)
    return fail(I8L_ERR_INVALID_ARG, "%s: K=%lld must be a positive multiple of 16", fn,
                (long long)K);
  if (M > INT32_MAX || N > INT32_MAX)
    return fail(I8L_ERR_INVALID_ARG, "%s: M and N must be < 2^31", fn);
  if ((M > 0 && (uint64_t)M * (uint64_t)K > (1ull << 40)) ||
      (N > 0 && (uint64_t)N * (uint64_t)K > (1ull << 40)) ||
      (uint64_t)M * (uint64_t)N > (1ull << 40))
    return fail(I8L_ERR_INVALID_ARG, "%s: tensor sizes exceed 2^40 elements", fn);
  return I8L_OK;
}

i8l_status check_zp_k(const char* fn, int64_t K) {
  if (K > I8L_MAX_K_ZP)
    return fail(I8L_ERR_K_TOO_LARGE,
                "%s: K=%lld exceeds %d for zero-point codes (K*255*127 must fit in int32)", fn,
                (long long)K, I8L_MAX_K_ZP);
  return I8L_OK;
}

// The GEMM's split-K tail (M > 256, the only shapes that reach it) needs
// int32 partial tiles, sized for a device with up to kGemmMaxSlices compute
// units; the counters region before them is reserved.  split == false lays out
// no partial tiles (the GEMM then computes every tile whole).
i8l_workspace_layout layout_of(int64_t M, int64_t K, int64_t N, bool split = true) {
  i8l_workspace_layout L;
  size_t off = 0;
  L.n_outliers = off; off += up(sizeof(int32_t));
  L.outlier_idx = off; off += up((size_t)K * sizeof(int32_t));
  L.sx = off; off += up((size_t)M * sizeof(float));
  L.flags = off; off += up((size_t)((K + 31) / 32) * sizeof(uint32_t));
  L.Xq = off; off += up((size_t)M * (size_t)K);
  L.X_outliers = off; off += up((size_t)M * (size_t)K * sizeof(uint16_t));
  // before the GEMM's part, so that its offset does not depend on N
  L.zero_points = off; off += up((size_t)M * sizeof(int32_t));
  // small M: per 512-column slice an outlier count and 16 row maxima and minima
  const size_t act_words =
      (M >= 1 && M <= i8l::kActSmallRows) ? (size_t)i8l::act_slices((int)K) * (1 + 2 * i8l::kActSmallRows) : 0;
  L.act_partials = off; off += up(act_words * sizeof(uint32_t));
  int slices = 0;
  if (split && M > i8l::kSkinnyMaxM && N > 0) {
    const i8l::GemmSplit p = i8l::gemm_split_plan((int)M, (int)N, (int)K, i8l::kGemmMaxSlices);
    slices = p.split_tiles * p.S;
  }
  L.gemm_counters = off; off += up(slices > 0 ? i8l::kGemmMaxSlices * sizeof(int32_t) : 0);
  L.gemm_partials = off; off += up((size_t)slices * 256 * 256 * sizeof(int32_t));
  L.gemm_slices = (size_t)slices;
  L.total = off;
  return L;
}

i8l::Workspace carve(void* ws, const i8l_workspace_layout& L) {
  char* b = static_cast<char*>(ws);
  i8l::Workspace w;
  w.n_out = reinterpret_cast<int32_t*>(b + L.n_outliers);
  w.idx = reinterpret_cast<int32_t*>(b + L.outlier_idx);
  w.sx = reinterpret_cast<float*>(b + L.sx);
  w.Xq = reinterpret_cast<int8_t*>(b + L.Xq);
  w.X_O = reinterpret_cast<uint16_t*>(b + L.X_outliers);
  w.flags = reinterpret_cast<uint32_t*>(b + L.flags);
  w.gemm_cnt = reinterpret_cast<int32_t*>(b + L.gemm_counters);
  w.gemm_part = reinterpret_cast<int32_t*>(b + L.gemm_partials);
  w.gemm_slices = (int)L.gemm_slices;
  w.zp = reinterpret_cast<int32_t*>(b + L.zero_points);
  w.act_part = reinterpret_cast<uint32_t*>(b + L.act_partials);
  return w;
}

#define REQUIRE_PTR(fn, p, al)                                                                   \
  do {                                                                                           \
    if (!(p)) return fail(I8L_ERR_INVALID_ARG, "%s: " #p " is NULL", fn);                        \
    if (!aligned((p), (al)))                                                                     \
      return fail(I8L_ERR_INVALID_ARG, "%s: " #p " must be %d-byte aligned", fn, (int)(al));    \
  } while (0)

i8l_status hip_status(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(I8L_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

I8L_API i8l_status i8l_linear_workspace(int64_t M, int64_t K, int64_t N,
                                        i8l_workspace_layout* layout) {
  i8l_status s = check_shape("i8l_linear_workspace", M, K, N);
  if (s != I8L_OK) return s;
  if (!layout) return fail(I8L_ERR_INVALID_ARG, "i8l_linear_workspace: layout is NULL");
  *layout = layout_of(M, K, N);
  return ok();
}

I8L_API size_t i8l_linear_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (check_shape("i8l_linear_workspace_bytes", M, K, N) != I8L_OK) return 0;
  return layout_of(M, K, N).total;
}

I8L_API i8l_status int8_quantize_weight(const uint16_t* W, int64_t K, int64_t N, int8_t* Wq,
                                        float* sw, void* stream) {
  const char* fn = "int8_quantize_weight";
  i8l_status s = check_shape(fn, 0, K, N);
  if (s != I8L_OK) return s;
  if (N == 0) return ok();
  REQUIRE_PTR(fn, W, 2);
  REQUIRE_PTR(fn, Wq, 16);
  REQUIRE_PTR(fn, sw, 4);
  (void)hipGetLastError();
  return hip_status(fn, i8l::launch_quantize_weight(W, (int)K, (int)N, Wq, sw,
                                                    static_cast<hipStream_t>(stream)));
}

I8L_API i8l_status int8_weight_code_sums(const int8_t* Wq, int64_t N, int64_t K, int32_t* S,
                                        void* stream) {
  const char* fn = "int8_weight_code_sums";
  i8l_status s = check_shape(fn, 0, K, N);
  if (s != I8L_OK) return s;
  if (N == 0) return ok();
  REQUIRE_PTR(fn, Wq, 16);
  REQUIRE_PTR(fn, S, 4);
  (void)hipGetLastError();
  return hip_status(fn, i8l::launch_weight_code_sums(Wq, (int)N, (int)K, S,
                                                     static_cast<hipStream_t>(stream)));
}

// ---- Static scratch of int8_linear_static ----------------------------------
// The workspace of callers that cannot allocate device memory: a file-scope
// device array, one copy per GPU the library runs on, held until the process
// ends.  Its host-side name is not a device address: host code uses only the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[I8L_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
// Device address of `scratch` per device, looked up on the first call made
// with that device current (0: not yet).
std::atomic<uintptr_t> g_scratch_addr[kMaxDevices];

i8l_status scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(I8L_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(I8L_ERR_INVALID_ARG, "%s: device %d outside the %d the library tracks", fn, dev,
                kMaxDevices);
  uintptr_t a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (a == 0) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(I8L_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    a = reinterpret_cast<uintptr_t>(p);
    g_scratch_addr[dev].store(a, std::memory_order_release);   // the same value on every race
  }
  *out = reinterpret_cast<void*>(a);
  return I8L_OK;
}
}  // namespace

namespace {
// zp: zero-point codes for X and the corrected epilogue (wsum required).
// use_scratch: the workspace is the static scratch array (workspace and
// workspace_bytes are ignored); shapes whose workspace does not fit it are
// rejected, after dropping the GEMM's split-K partials if that makes it fit.
i8l_status linear_impl(const char* fn, const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq,
                       const float* sw, const int32_t* wsum, int64_t N,
                       const uint16_t* W_outlier_rows, const uint16_t* bias, float threshold,
                       uint16_t* Y, void* workspace, size_t workspace_bytes, void* stream,
                       bool zp, bool use_scratch = false) {
  i8l_status s = check_shape(fn, M, K, N);
  if (s != I8L_OK) return s;
  if (zp && (s = check_zp_k(fn, K)) != I8L_OK) return s;
  if (isnan(threshold)) return fail(I8L_ERR_INVALID_ARG, "%s: threshold is NaN", fn);
  const bool enabled = threshold > 0.0f && isfinite(threshold);
  if (M == 0 || N == 0) return ok();   // nothing to read or write
  REQUIRE_PTR(fn, X, 16);
  REQUIRE_PTR(fn, Wq, 16);
  REQUIRE_PTR(fn, sw, 4);
  if (zp) REQUIRE_PTR(fn, wsum, 4);
  REQUIRE_PTR(fn, Y, 16);
  if (!use_scratch) REQUIRE_PTR(fn, workspace, 16);
  // NULL W_outlier_rows: the outlier rows are rebuilt from Wq and sw
  if (W_outlier_rows && !aligned(W_outlier_rows, 2))
    return fail(I8L_ERR_INVALID_ARG, "%s: W_outlier_rows must be 2-byte aligned", fn);
  if (bias && !aligned(bias, 2))
    return fail(I8L_ERR_INVALID_ARG, "%s: bias must be 2-byte aligned", fn);
  i8l_workspace_layout L = layout_of(M, K, N);
  if (use_scratch) {
    if (L.total > (size_t)I8L_STATIC_SCRATCH_BYTES) L = layout_of(M, K, N, false);
    if (L.total > (size_t)I8L_STATIC_SCRATCH_BYTES)
      return fail(I8L_ERR_WORKSPACE,
                  "%s: M=%lld K=%lld N=%lld needs %zu bytes of scratch; the static scratch "
                  "holds %zu (use int8_linear_bias with a workspace)",
                  fn, (long long)M, (long long)K, (long long)N, L.total,
                  (size_t)I8L_STATIC_SCRATCH_BYTES);
    if ((s = scratch_address(fn, &workspace)) != I8L_OK) return s;
    workspace_bytes = I8L_STATIC_SCRATCH_BYTES;
  }
  if (workspace_bytes < L.total)
    return fail(I8L_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu required", fn,
                workspace_bytes, L.total);
  (void)hipGetLastError();
  const i8l::Workspace w = carve(workspace, L);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int m = (int)M, k = (int)K, n = (int)N;
  if (m <= i8l::kStreamMaxM) {   // weight-bound: the fused or the streaming kernel
    if (zp)
      return hip_status(fn, i8l::launch_decode_zp(X, m, k, Wq, sw, wsum, n, W_outlier_rows, bias,
                                                  threshold, enabled, Y, w, st));
    return hip_status(fn, i8l::launch_decode(X, m, k, Wq, sw, n, W_outlier_rows, bias, threshold,
                                             enabled, Y, w, st));
  }
  hipError_t e = i8l::launch_quantize_activation(X, m, k, threshold, enabled, w, st, zp);
  if (e != hipSuccess) return hip_status(fn, e);
  i8l::GemmArgs g{w.Xq, Wq, m, n, k, w.sx, sw, w.n_out, w.idx, w.X_O, W_outlier_rows, Y, nullptr,
                  bias, zp ? w.zp : nullptr, zp ? wsum : nullptr, w.gemm_cnt, w.gemm_part,
                  w.gemm_slices, 0, 1};
  if (m <= i8l::kSkinnyMaxM) return hip_status(fn, i8l::launch_gemm_skinny(g, st));
  return hip_status(fn, i8l::launch_gemm(g, st));
}
}  // namespace

I8L_API i8l_status int8_linear(const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq,
                               const float* sw, int64_t N, const uint16_t* W_outlier_rows,
                               float threshold, uint16_t* Y, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return linear_impl("int8_linear", X, M, K, Wq, sw, nullptr, N, W_outlier_rows, nullptr,
                     threshold, Y, workspace, workspace_bytes, stream, false);
}

I8L_API i8l_status int8_linear_bias(const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq,
                                    const float* sw, int64_t N, const uint16_t* W_outlier_rows,
                                    const uint16_t* bias, float threshold, uint16_t* Y,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return linear_impl("int8_linear_bias", X, M, K, Wq, sw, nullptr, N, W_outlier_rows, bias,
                     threshold, Y, workspace, workspace_bytes, stream, false);
}

I8L_API i8l_status int8_linear_static(const uint16_t* X, int64_t M, int64_t K,
                                      const int8_t* Wq, const float* sw, int64_t N,
                                      const uint16_t* W_outlier_rows, const uint16_t* bias,
                                      float threshold, uint16_t* Y, void* stream) {
  return linear_impl("int8_linear_static", X, M, K, Wq, sw, nullptr, N, W_outlier_rows, bias,
                     threshold, Y, nullptr, 0, stream, false, true);
}

I8L_API i8l_status int8_linear_zp(const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq,
                                  const float* sw, const int32_t* wsum, int64_t N,
                                  const uint16_t* W_outlier_rows, const uint16_t* bias,
                                  float threshold, uint16_t* Y, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return linear_impl("int8_linear_zp", X, M, K, Wq, sw, wsum, N, W_outlier_rows, bias, threshold,
                     Y, workspace, workspace_bytes, stream, true);
}

namespace {
// use_zp: zero-point codes (sx then receives range / 255, zp the zero points).
i8l_status quantize_activation_impl(const char* fn, const uint16_t* X, int64_t M, int64_t K,
                                    float threshold, int8_t* Xq, float* sx, int32_t* zp,
                                    int32_t* outlier_idx, int32_t* n_outliers,
                                    uint16_t* X_outliers, void* workspace,
                                    size_t workspace_bytes, void* stream, bool use_zp) {
  i8l_status s = check_shape(fn, M, K, 0);
  if (s != I8L_OK) return s;
  if (use_zp && (s = check_zp_k(fn, K)) != I8L_OK) return s;
  if (isnan(threshold)) return fail(I8L_ERR_INVALID_ARG, "%s: threshold is NaN", fn);
  const bool enabled = threshold > 0.0f && isfinite(threshold);
  if (M == 0) {
    // no rows: no outliers; only the count (0) is written, so only it is required
    REQUIRE_PTR(fn, n_outliers, 4);
    (void)hipGetLastError();
    return hip_status(fn, i8l::launch_fill_u32(reinterpret_cast<uint32_t*>(n_outliers), 1, 0u,
                                               static_cast<hipStream_t>(stream)));
  }
  REQUIRE_PTR(fn, X, 16);
  REQUIRE_PTR(fn, Xq, 16);
  REQUIRE_PTR(fn, sx, 4);
  if (use_zp) REQUIRE_PTR(fn, zp, 4);
  REQUIRE_PTR(fn, outlier_idx, 4);
  REQUIRE_PTR(fn, n_outliers, 4);
  REQUIRE_PTR(fn, X_outliers, 16);
  REQUIRE_PTR(fn, workspace, 16);
  const i8l_workspace_layout L = layout_of(M, K, 0);
  if (workspace_bytes < L.total)
    return fail(I8L_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu required", fn,
                workspace_bytes, L.total);
  (void)hipGetLastError();
  i8l::Workspace w = carve(workspace, L);
  w.n_out = n_outliers;
  w.idx = outlier_idx;
  w.sx = sx;
  w.Xq = Xq;
  w.X_O = X_outliers;
  if (use_zp) w.zp = zp;
  return hip_status(fn, i8l::launch_quantize_activation(X, (int)M, (int)K, threshold, enabled, w,
                                                        static_cast<hipStream_t>(stream),
                                                        use_zp));
}
}  // namespace

I8L_API i8l_status int8_quantize_activation(const uint16_t* X, int64_t M, int64_t K,
                                            float threshold, int8_t* Xq, float* sx,
                                            int32_t* outlier_idx, int32_t* n_outliers,
                                            uint16_t* X_outliers, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  return quantize_activation_impl("int8_quantize_activation", X, M, K, threshold, Xq, sx, nullptr,
                                  outlier_idx, n_outliers, X_outliers, workspace,
                                  workspace_bytes, stream, false);
}

I8L_API i8l_status int8_quantize_activation_zp(const uint16_t* X, int64_t M, int64_t K,
                                               float threshold, int8_t* Xq, int32_t* zp,
                                               float* xscale, int32_t* outlier_idx,
                                               int32_t* n_outliers, uint16_t* X_outliers,
                                               void* workspace, size_t workspace_bytes,
                                               void* stream) {
  return quantize_activation_impl("int8_quantize_activation_zp", X, M, K, threshold, Xq, xscale,
                                  zp, outlier_idx, n_outliers, X_outliers, workspace,
                                  workspace_bytes, stream, true);
}

I8L_API i8l_status int8_gemm_i32(const int8_t* Xq, const int8_t* Wq, int64_t M, int64_t N,
                                 int64_t K, int32_t* acc, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const char* fn = "int8_gemm_i32";
  i8l_status s = check_shape(fn, M, K, N);
  if (s != I8L_OK) return s;
  if (M == 0 || N == 0) return ok();
  REQUIRE_PTR(fn, Xq, 16);
  REQUIRE_PTR(fn, Wq, 16);
  REQUIRE_PTR(fn, acc, 16);
  // with a workspace the tiles are split along K exactly as int8_linear splits
  // them; without one every tile is computed whole
  int32_t* part = nullptr;
  int slices = 0;
  if (workspace) {
    if (!aligned(workspace, 16))
      return fail(I8L_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
    const i8l_workspace_layout L = layout_of(M, K, N);
    if (workspace_bytes < L.total)
      return fail(I8L_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu required", fn,
                  workspace_bytes, L.total);
    const i8l::Workspace w = carve(workspace, L);
    part = w.gemm_part;
    slices = w.gemm_slices;
  }
  (void)hipGetLastError();
  i8l::GemmArgs g{Xq, Wq, (int)M, (int)N, (int)K, nullptr, nullptr, nullptr, nullptr, nullptr,
                  nullptr, nullptr, acc, nullptr, nullptr, nullptr, nullptr, part, slices, 0, 1};
  // the kernel int8_linear runs for this M: 256 x 64 tiles up to 256 rows
  if (M <= i8l::kSkinnyMaxM)
    return hip_status(fn, i8l::launch_gemm_skinny(g, static_cast<hipStream_t>(stream)));
  return hip_status(fn, i8l::launch_gemm(g, static_cast<hipStream_t>(stream)));
}

// ---- Training mode: backward pass ------------------------------------------------

namespace {
// Shape rules of the backward entry points: the layer's rules for M, K, plus
// N % 8 == 0 (the products run along N and along rows padded to 8, in whole
// 16-byte chunks).
i8l_status check_backward_shape(const char* fn, int64_t M, int64_t K, int64_t N) {
  i8l_status s = check_shape(fn, M, K, N);
  if (s != I8L_OK) return s;
  if (N % 8 != 0)
    return fail(I8L_ERR_INVALID_ARG, "%s: N=%lld must be a multiple of 8", fn, (long long)N);
  if ((uint64_t)K * (uint64_t)N > (1ull << 40) || (uint64_t)M + 8 > (uint64_t)INT32_MAX)
    return fail(I8L_ERR_INVALID_ARG, "%s: tensor sizes exceed the supported range", fn);
  return I8L_OK;
}
}  // namespace

I8L_API size_t i8l_backward_weight_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (check_backward_shape("i8l_backward_weight_workspace_bytes", M, K, N) != I8L_OK) return 0;
  size_t a, b, c;
  return i8l::backward_weight_workspace((int)M, (int)K, (int)N, &a, &b, &c);
}

I8L_API i8l_status int8_linear_backward_input(const uint16_t* dY, const uint16_t* W, int64_t M,
                                              int64_t K, int64_t N, uint16_t* dX,
                                              void* stream) {
  const char* fn = "int8_linear_backward_input";
  i8l_status s = check_backward_shape(fn, M, K, N);
  if (s != I8L_OK) return s;
  if (M == 0) return ok();
  REQUIRE_PTR(fn, dX, 16);
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (N == 0)   // empty sums: dX = 0 (K % 16 == 0: whole words)
    return hip_status(fn, i8l::launch_fill_u32(reinterpret_cast<uint32_t*>(dX),
                                               (int)((uint64_t)M * K / 2), 0u, st));
  REQUIRE_PTR(fn, dY, 16);
  REQUIRE_PTR(fn, W, 16);
  return hip_status(fn, i8l::launch_backward_input(dY, W, (int)M, (int)K, (int)N, dX, st));
}

I8L_API i8l_status int8_linear_backward_weight(const uint16_t* X, const uint16_t* dY, int64_t M,
                                               int64_t K, int64_t N, uint16_t* dW,
                                               uint16_t* dbias, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  const char* fn = "int8_linear_backward_weight";
  i8l_status s = check_backward_shape(fn, M, K, N);
  if (s != I8L_OK) return s;
  if (N == 0) return ok();
  REQUIRE_PTR(fn, dW, 16);
  if (dbias && !aligned(dbias, 4))
    return fail(I8L_ERR_INVALID_ARG, "%s: dbias must be 4-byte aligned", fn);
  if (M > 0) {
    REQUIRE_PTR(fn, X, 16);
    REQUIRE_PTR(fn, dY, 16);
    REQUIRE_PTR(fn, workspace, 16);
    size_t a, b, c;
    const size_t need = i8l::backward_weight_workspace((int)M, (int)K, (int)N, &a, &b, &c);
    if (workspace_bytes < need)
      return fail(I8L_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu required", fn,
                  workspace_bytes, need);
  }
  (void)hipGetLastError();
  return hip_status(fn, i8l::launch_backward_weight(X, dY, (int)M, (int)K, (int)N, dW, dbias,
                                                    workspace, static_cast<hipStream_t>(stream)));
}

I8L_API const char* i8l_last_error(void) { return g_err; }

I8L_API const char* i8l_build_info(void) {
  // built once (thread-safe static initialization), read-only afterwards
  static const std::string info =
      std::string("int8lin gfx950; ") + i8l::gemm_tile_info() +
      "; M <= 64: fused kernel (M <= 16, K <= 4096) or activation kernels + weight-streaming "
      "kernel";
  return info.c_str();
}
