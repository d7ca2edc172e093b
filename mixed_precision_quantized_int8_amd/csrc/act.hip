// Activation stage of LLM.int8(): outlier column scan, row absmax over the
// regular columns, row-wise int8 codes and the gather of the outlier values.
//
// [blog, "A gentle summary of LLM.int8()"], step 1: outliers are taken out of
// the hidden states column by column.  [blog, "A closer look at the MatMul"]:
// an outlier has magnitude 6 or more (the threshold), and the remaining hidden
// states are quantized row by row.  [blog, "Introduction to model
// quantization"]: absmax codes are round(x * 127 / absmax) in [-127, 127].
//
// For M > 16, launches on the caller's stream (more than 256 rows with the
// decomposition on: clear, rowpass, rowfix instead; see below):
//   clear     zero the column bitmask (a fill kernel, safe under graph capture);
//             only where several workgroups share a column (M > 256)
//   colflags  one pass over X: per thread 16-byte loads, 8 running column
//             maxima (NaN entries count as 0: a NaN never reaches the
//             threshold); a set bit for every column whose maximum reaches the
//             threshold (atomicOr, issued only for the rare outlier columns;
//             with the threshold off, one workgroup holds every row of its
//             columns and stores its flag words outright).  For M <= 256 the
//             same test runs in colscan_strip_kernel: 64-column strips, each
//             workgroup over every row, every flag word stored.
//   rowquant  one workgroup per row: the bitmask and its prefix popcounts go
//             to LDS, the row is held in registers while its absmax over the
//             regular columns is reduced, then codes are written (8 bytes per
//             thread, coalesced) and outlier values are scattered to X_O at
//             their rank; workgroup 0 also writes the ascending index list.
// Zero-point mode of rowquant ([blog, "Introduction to model quantization"],
// the unsigned scheme): the row's minimum and maximum over the regular columns,
// widened to contain 0, give inv = fl32(255 / range) and the zero point
// zp = round_half_away(-min * inv); codes are clamp(round_half_away(x * inv) +
// zp, 0, 255), stored as code - 128 so the int8 matrix cores can take them;
// outlier columns store zp - 128 (the code of 0).  The row writes
// fl32(range / 255) to sx and zp to the zero-point array.
// The column dependency (every row must be seen before any row scale) would
// have X read twice.  For more than 256 rows it is read once: rowpass_kernel
// codes each row with a provisional scale (its largest entry below the
// threshold; zero-point codes: its smallest and largest) and sets the outlier
// flags, and rowfix_kernel then zeroes (zero-point codes: sets to the code of
// 0) and gathers the outlier columns, recomputing only the rows whose
// provisional scale came from an outlier column.  17-256 rows, and the
// threshold off, keep the scan + row pass (two reads; for small M the reads
// are latency, not bytes).
// For 1 <= M <= 16 (the small-M path with K > 4096, and the stage export) two
// launches over 512-column slices do the same work with many workgroups
// instead of one per row (see the kernels below).
#include "common.h"
#include "launch.h"

namespace i8l {

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int n, uint32_t v) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, int n, uint32_t v, hipStream_t stream) {
  const int blocks = n > 0 ? (n + 255) / 256 : 1;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks < 1024 ? blocks : 1024), dim3(256), 0, stream, p,
                     n, v);
  return hipGetLastError();
}

constexpr int kColThreads = 256;
constexpr int kColStrip = kWave * 8;   // columns per workgroup: 8 fp16 per lane

// grid = (ceil(K / 512), ceil(M / rows_per_block)); waves of a block stride over rows.
// STORE: grid.y == 1 (the block scans every row of its columns), so it stores
// all of its flag words, zeros included, and no clear is needed; scan == 0
// then stores zeros without reading X (decomposition off).
template <bool STORE>
__global__ __launch_bounds__(kColThreads) void colflags_kernel(const uint16_t* __restrict__ X, int M,
                                                              int K, int rows_per_block,
                                                              float threshold, int scan,
                                                              uint32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  __shared__ uint32_t s_bits[kColThreads / 64][kColStrip / 32];
  const int c = blockIdx.x * kColStrip + lane * 8;
  // K % 16 == 0, so c < K means all 8 columns are in range; lanes past K scan
  // no rows (they stay in for the block-wide combine below)
  const int r0 = blockIdx.y * rows_per_block;
  const int r1 = (c < K && scan) ? min(M, r0 + rows_per_block) : r0;
  const uint16_t* base = X + c;
  uint32_t mx[4] = {0, 0, 0, 0};   // packed pairs of |fp16| bit patterns
  int r = r0 + wave;
  // four independent 16-byte loads in flight per thread
  for (; r + 12 < r1; r += 16) {
    v4i a = *reinterpret_cast<const v4i*>(base + (size_t)r * K);
    v4i b = *reinterpret_cast<const v4i*>(base + (size_t)(r + 4) * K);
    v4i d = *reinterpret_cast<const v4i*>(base + (size_t)(r + 8) * K);
    v4i e = *reinterpret_cast<const v4i*>(base + (size_t)(r + 12) * K);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t x0 = habs2_nonan((uint32_t)a[j]), x1 = habs2_nonan((uint32_t)b[j]);
      uint32_t x2 = habs2_nonan((uint32_t)d[j]), x3 = habs2_nonan((uint32_t)e[j]);
      // per-halfword unsigned max
      uint32_t lo = max(max(x0 & 0xffffu, x1 & 0xffffu), max(x2 & 0xffffu, x3 & 0xffffu));
      uint32_t hi = max(max(x0 >> 16, x1 >> 16), max(x2 >> 16, x3 >> 16));
      lo = max(lo, mx[j] & 0xffffu);
      hi = max(hi, mx[j] >> 16);
      mx[j] = lo | (hi << 16);
    }
  }
  for (; r < r1; r += 4) {
    v4i a = *reinterpret_cast<const v4i*>(base + (size_t)r * K);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t x0 = habs2_nonan((uint32_t)a[j]);
      uint32_t lo = max(x0 & 0xffffu, mx[j] & 0xffffu);
      uint32_t hi = max(x0 >> 16, mx[j] >> 16);
      mx[j] = lo | (hi << 16);
    }
  }
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t h = (mx[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
    if (scan && h2f((uint16_t)h) >= threshold) bits |= 1u << e;
  }
  // one atomic per flag word and block: the 4 lanes of a word, then the 4
  // waves (which scanned other rows of the same columns), are combined first
  uint32_t wbits = bits << (c & 31);
  wbits |= __shfl_xor(wbits, 1, 64);
  wbits |= __shfl_xor(wbits, 2, 64);
  if ((lane & 3) == 0) s_bits[wave][lane >> 2] = wbits;
  __syncthreads();
  const int t = threadIdx.x;
  if (t < kColStrip / 32) {
    uint32_t v = 0;
#pragma unroll
    for (int w = 0; w < kColThreads / 64; ++w) v |= s_bits[w][t];
    const int word = blockIdx.x * (kColStrip / 32) + t;
    if constexpr (STORE) {
      if (word < (K + 31) / 32) flags[word] = v;
    } else if (v) {
      atomicOr(flags + word, v);
    }
  }
}

// Column scan for batches of up to 32 * RPT rows: one workgroup per strip of
// 64 columns holds every row of it, so the strip's two flag words are complete
// there and are stored outright (zeros included: no clear launch).  Thread t
// reads columns 8 (t % 8) .. +7 of rows t / 8 + 32 i, i < RPT, all loads in
// flight at once; rows past M and columns past K read 0 from the buffer
// resource.  Narrow strips give K / 64 workgroups (64 for K = 4096), where the
// 512-column strips of colflags_kernel give K / 512 with several round trips
// each.  scan == 0 stores zeros without reading X.
constexpr int kStripCols = 64;
template <int RPT>
__global__ __launch_bounds__(kColThreads) void colscan_strip_kernel(const uint16_t* __restrict__ X,
                                                                    int M, int K, float threshold,
                                                                    int scan,
                                                                    uint32_t* __restrict__ flags) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = t & 7;
  const int c = blockIdx.x * kStripCols + g * 8;
  uint32_t mx[4] = {0, 0, 0, 0};   // packed pairs of |fp16| bit patterns
  if (scan) {   // uniform
    const buf_rsrc rx = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
    v4i x[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = (t >> 3) + 32 * i;
      x[i] = buf_load16(rx, r < M && c < K ? (uint32_t)(r * K + c) * 2u : kBufOff);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t v = habs2_nonan((uint32_t)x[i][j]);
        const uint32_t lo = max(v & 0xffffu, mx[j] & 0xffffu);
        const uint32_t hi = max(v >> 16, mx[j] >> 16);
        mx[j] = lo | (hi << 16);
      }
    // the 8 row groups of the wave that share a column chunk (lane bits 3-5)
#pragma unroll
    for (int off = 8; off < 64; off <<= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t o = (uint32_t)__shfl_xor((int)mx[j], off, 64);
        const uint32_t lo = max(o & 0xffffu, mx[j] & 0xffffu);
        const uint32_t hi = max(o >> 16, mx[j] >> 16);
        mx[j] = lo | (hi << 16);
      }
  }
  __shared__ uint32_t s_mx[kColThreads / 64][8][4];
  __shared__ uint32_t s_byte[8];
  if (lane < 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) s_mx[wave][lane][j] = mx[j];
  }
  __syncthreads();
  if (t < 8) {
    uint32_t bits = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t h = 0;
#pragma unroll
      for (int w = 0; w < kColThreads / 64; ++w) {
        const uint32_t v = (s_mx[w][t][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        h = v > h ? v : h;
      }
      if (scan && h2f((uint16_t)h) >= threshold) bits |= 1u << e;
    }
    s_byte[t] = bits;
  }
  __syncthreads();
  if (t < kStripCols / 32) {
    const uint32_t v = s_byte[4 * t] | (s_byte[4 * t + 1] << 8) | (s_byte[4 * t + 2] << 16) |
                       (s_byte[4 * t + 3] << 24);
    const int word = blockIdx.x * (kStripCols / 32) + t;
    if (word < (K + 31) / 32) flags[word] = v;
  }
}

// Exclusive block-wide prefix sum (blockDim.x threads, multiple of 64).
template <int BS>
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int* total) {
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

constexpr int kMaxFlagWords = (I8L_MAX_K_DEV + 31) / 32;

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off, 64);
    v = o < v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
  for (int off = 32; off > 0; off >>= 1) v = __builtin_fminf(v, __shfl_xor(v, off, 64));
  return v;
}

// One workgroup per row of X.  NCH 16-byte chunks per thread: K <= BS * 8 * NCH.
// ZP: zero-point codes (zp != nullptr) instead of absmax codes.
template <int BS, int NCH, bool ZP>
__global__ __launch_bounds__(BS) void rowquant_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                     const uint32_t* __restrict__ flags,
                                                     int8_t* __restrict__ Xq, float* __restrict__ sx,
                                                     int32_t* __restrict__ zp,
                                                     int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ n_out,
                                                     uint16_t* __restrict__ X_O) {
  __shared__ uint32_t s_flags[kMaxFlagWords];
  __shared__ int s_rank[kMaxFlagWords];
  __shared__ int s_tmp[BS / 64 + 1];
  __shared__ uint32_t s_max[BS / 64];
  __shared__ float s_lo[ZP ? BS / 64 : 1], s_hi[ZP ? BS / 64 : 1];

  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const int nw = (K + 31) >> 5;

  // Loads first, all branch-free buffer loads (past the end they read 0): the
  // flag words w = t + i*BS, then the row; writing the flags to LDS waits only
  // for the flag loads, and the row stays in flight while the flags are
  // scanned (the barriers below order LDS only).
  constexpr int FW = (NCH + 3) / 4;   // BS*NCH*8 >= K, so FW*BS >= ceil(K/32)
  const buf_rsrc rf = make_rsrc(flags, (uint32_t)nw * 4u);
  uint32_t fl[FW];
#pragma unroll
  for (int i = 0; i < FW; ++i) fl[i] = buf_load_u32(rf, (uint32_t)(t + i * BS) * 4u);
  const buf_rsrc rx = make_rsrc(X + (size_t)row * K, (uint32_t)K * 2u);
  const int nchunks = K >> 3;
  v4i raw[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) raw[j] = buf_load16(rx, (uint32_t)(t + j * BS) * 16u);
#pragma unroll
  for (int i = 0; i < FW; ++i)
    if (t + i * BS < nw) s_flags[t + i * BS] = fl[i];
  lds_sync();

  // exclusive prefix popcount per flag word, over contiguous word ranges
  const int w0 = t * ((nw + BS - 1) / BS);
  const int w1 = min(nw, w0 + (nw + BS - 1) / BS);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __builtin_popcount(s_flags[w]);
  int total;
  int base = block_excl_scan<BS>(cnt, s_tmp, &total);
  for (int w = w0; w < w1; ++w) {
    s_rank[w] = base;
    base += __builtin_popcount(s_flags[w]);
  }
  lds_sync();
  // workgroup 0 writes the ascending index list and the outlier count
  auto write_index = [&]() {
    if (row == 0) {
      for (int w = t; w < nw; w += BS) {
        uint32_t f = s_flags[w];
        int r = s_rank[w];
        while (f) {
          const int b = __builtin_ctz(f);
          idx[r++] = w * 32 + b;
          f &= f - 1u;
        }
      }
      if (t == 0) *n_out = total;
    }
  };
  uint32_t mx = 0;
  float lo = 0.0f, hi = 0.0f;   // zero-point mode: the range always contains 0
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int q = t + j * BS;
    if (q < nchunks) {
      const uint32_t ob = (s_flags[q >> 2] >> ((q & 3) * 8)) & 0xffu;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t hb = ((uint32_t)raw[j][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        if (!((ob >> e) & 1u)) {
          if constexpr (ZP) {
            const float x = h2f((uint16_t)hb);
            lo = __builtin_fminf(lo, x);
            hi = __builtin_fmaxf(hi, x);
          } else {
            const uint32_t h = hb & 0x7fffu;
            mx = h > mx ? h : mx;
          }
        }
      }
    }
  }
  float inv, scale;
  int zpv = 0;
  if constexpr (ZP) {
    lo = wave_min(lo);
    hi = wave_max(hi);
    if ((t & 63) == 0) {
      s_lo[t >> 6] = lo;
      s_hi[t >> 6] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < BS / 64; ++w) {
      lo = __builtin_fminf(lo, s_lo[w]);
      hi = __builtin_fmaxf(hi, s_hi[w]);
    }
    const float range = hi - lo;
    inv = range > 0.0f ? 255.0f / range : 0.0f;
    zpv = (int)__builtin_roundf(-lo * inv);
    scale = range / 255.0f;
  } else {
    mx = wave_max_u32(mx);
    if ((t & 63) == 0) s_max[t >> 6] = mx;
    __syncthreads();
    mx = 0;
#pragma unroll
    for (int w = 0; w < BS / 64; ++w) mx = s_max[w] > mx ? s_max[w] : mx;
    scale = h2f((uint16_t)mx);
    inv = quant_scale(scale);
  }

  int8_t* qr = Xq + (size_t)row * K;
  uint16_t* orow = X_O + (size_t)row * K;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int q = t + j * BS;
    if (q < nchunks) {
      const int word = q >> 2;
      const int sh = (q & 3) * 8;
      const uint32_t ob = (s_flags[word] >> sh) & 0xffu;
      int code[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t hb = (uint16_t)(((uint32_t)raw[j][e >> 1] >> ((e & 1) * 16)) & 0xffffu);
        if constexpr (ZP) {
          int c = ((ob >> e) & 1u) ? zpv : (int)__builtin_roundf(h2f(hb) * inv) + zpv;
          c = c < 0 ? 0 : (c > 255 ? 255 : c);
          code[e] = c - 128;
        } else {
          code[e] = ((ob >> e) & 1u) ? 0 : quant_code(h2f(hb), inv);
        }
      }
      v2i packed = {(int)pack4_i8(code[0], code[1], code[2], code[3]),
                    (int)pack4_i8(code[4], code[5], code[6], code[7])};
      *reinterpret_cast<v2i*>(qr + q * 8) = packed;
      if (ob) {
        const uint32_t fw = s_flags[word];
        const int rb = s_rank[word];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if ((ob >> e) & 1u) {
            const int bit = sh + e;
            const int rank = rb + __builtin_popcount(fw & ((1u << bit) - 1u));
            orow[rank] = (uint16_t)(((uint32_t)raw[j][e >> 1] >> ((e & 1) * 16)) & 0xffffu);
          }
        }
      }
    }
  }
  if (t == 0) {
    sx[row] = scale;
    if constexpr (ZP) zp[row] = zpv;
  }

  write_index();
}

// Row pass of the prefill path (absmax codes, more than 256 rows, decomposition
// on): one workgroup per row reads the row once.  Entries at or above the
// threshold (a NaN never is) get code 0 and set their column's flag
// (atomicOr; the flags were cleared before).  The other entries are coded with
// a provisional scale, the largest magnitude among them, and a column where it
// occurs is recorded in rowval (-1 when the scale is 0; rowval is the
// workspace's zero-point array, unused by absmax codes).  Every regular column
// lies wholly below the threshold, so the maximum over the regular columns,
// the scale the method asks for, is at most the provisional one, and equal to
// it when the recorded column is regular: the codes, sx and all are then
// final except in the outlier columns, which rowfix_kernel zeroes and
// gathers.  When the recorded column is an outlier column the fix-up
// recomputes the row.  X is read once instead of twice (column scan, then row
// quantization).
// ZP (zero-point codes): the provisional range is the smallest and largest
// entry below the threshold, widened to contain 0 (a NaN counts for neither),
// recorded with a column of each; the codes, xscale and zero point follow the
// rules of rowquant_kernel.  The two columns go to the last 8 bytes of the
// row's X_O capacity (the zero-point array is an output here); the fix-up
// reads them before it writes any X_O value of the row.
template <int BS, int NCH, bool ZP>
__global__ __launch_bounds__(BS) void rowpass_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                    float threshold, uint32_t* __restrict__ flags,
                                                    int8_t* __restrict__ Xq,
                                                    float* __restrict__ sx,
                                                    int32_t* __restrict__ rowval,
                                                    uint16_t* __restrict__ X_O) {
  __shared__ uint32_t s_h[BS / 64], s_c[BS / 64];
  __shared__ float s_lo[ZP ? BS / 64 : 1], s_hi[ZP ? BS / 64 : 1];
  __shared__ uint32_t s_cl[ZP ? BS / 64 : 1], s_ch[ZP ? BS / 64 : 1];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int row = blockIdx.x;
  const buf_rsrc rx = make_rsrc(X + (size_t)row * K, (uint32_t)K * 2u);
  const int nchunks = K >> 3;
  v4i raw[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) raw[j] = buf_load16(rx, (uint32_t)(t + j * BS) * 16u);
  // an entry at or above the threshold (a NaN never is)
  auto big = [&](uint32_t h) { return h <= 0x7c00u && h2f((uint16_t)h) >= threshold; };
  // the per-chunk masks are kept in registers up to 8 chunks per thread, and
  // recomputed when the codes are formed beyond (register budget of 1024 threads)
  constexpr bool kKeep = NCH <= 8;
  uint32_t bigm[kKeep ? NCH : 1];
  uint32_t mx = 0, mc = 0xffffffffu;   // largest magnitude bits below the threshold, its column
  float lo = 0.0f, hi = 0.0f;          // zero-point codes: the range, with its columns
  uint32_t cl = 0xffffffffu, ch = 0xffffffffu;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int q = t + j * BS;
    if constexpr (kKeep) bigm[j] = 0;
    if (q < nchunks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t hb = ((uint32_t)raw[j][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        const uint32_t h = hb & 0x7fffu;
        const bool b = big(h);
        if constexpr (kKeep) bigm[j] |= (uint32_t)b << e;
        if constexpr (ZP) {
          const float x = h2f((uint16_t)hb);
          if (!b && x < lo) {
            lo = x;
            cl = (uint32_t)(q * 8 + e);
          }
          if (!b && x > hi) {
            hi = x;
            ch = (uint32_t)(q * 8 + e);
          }
        } else if (!b && h > mx) {
          mx = h;
          mc = (uint32_t)(q * 8 + e);
        }
      }
    }
  }
  if constexpr (ZP) {
    // the workgroup's range, and the smallest column holding each end
    const float wl = wave_min(lo), wh = wave_max(hi);
    const uint32_t wcl = wave_min_u32(lo == wl ? cl : 0xffffffffu);
    const uint32_t wch = wave_min_u32(hi == wh ? ch : 0xffffffffu);
    if (lane == 0) {
      s_lo[wave] = wl;
      s_hi[wave] = wh;
      s_cl[wave] = wcl;
      s_ch[wave] = wch;
    }
    __syncthreads();
    float bl = 0.0f, bh = 0.0f;
    uint32_t bcl = 0xffffffffu, bch = 0xffffffffu;
#pragma unroll
    for (int w = 0; w < BS / 64; ++w) {
      if (s_lo[w] < bl) {
        bl = s_lo[w];
        bcl = s_cl[w];
      } else if (s_lo[w] == bl && s_cl[w] < bcl) {
        bcl = s_cl[w];
      }
      if (s_hi[w] > bh) {
        bh = s_hi[w];
        bch = s_ch[w];
      } else if (s_hi[w] == bh && s_ch[w] < bch) {
        bch = s_ch[w];
      }
    }
    const float range = bh - bl;
    const float inv = range > 0.0f ? 255.0f / range : 0.0f;
    const int zpv = (int)__builtin_roundf(-bl * inv);
    int8_t* qr = Xq + (size_t)row * K;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int q = t + j * BS;
      if (q < nchunks) {
        int code[8];
        uint32_t bm8 = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t hb = (uint16_t)(((uint32_t)raw[j][e >> 1] >> ((e & 1) * 16)) & 0xffffu);
          bool b;
          if constexpr (kKeep) b = (bigm[j] >> e) & 1u;
          else b = big(hb & 0x7fffu);
          bm8 |= (uint32_t)b << e;
          int c = b ? zpv : (int)__builtin_roundf(h2f(hb) * inv) + zpv;
          c = c < 0 ? 0 : (c > 255 ? 255 : c);
          code[e] = c - 128;
        }
        v2i packed = {(int)pack4_i8(code[0], code[1], code[2], code[3]),
                      (int)pack4_i8(code[4], code[5], code[6], code[7])};
        *reinterpret_cast<v2i*>(qr + q * 8) = packed;
        if (bm8) atomicOr(flags + (q >> 2), bm8 << ((q & 3) * 8));
      }
    }
    if (t == 0) {
      sx[row] = range / 255.0f;
      rowval[row] = zpv;   // the zero-point array
      int32_t* cols = reinterpret_cast<int32_t*>(X_O + (size_t)row * K + K - 4);
      cols[0] = bl < 0.0f ? (int)bcl : -1;
      cols[1] = bh > 0.0f ? (int)bch : -1;
    }
    return;
  }
  // the workgroup's largest magnitude, and the smallest column that holds it
  uint32_t wm = mx;
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)wm, off, 64);
    wm = o > wm ? o : wm;
  }
  uint32_t wc = mx == wm ? mc : 0xffffffffu;
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)wc, off, 64);
    wc = o < wc ? o : wc;
  }
  if (lane == 0) {
    s_h[wave] = wm;
    s_c[wave] = wc;
  }
  __syncthreads();
  uint32_t bm = 0, bc = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < BS / 64; ++w) {
    if (s_h[w] > bm) {
      bm = s_h[w];
      bc = s_c[w];
    } else if (s_h[w] == bm && s_c[w] < bc) {
      bc = s_c[w];
    }
  }
  const float scale = h2f((uint16_t)bm);
  const float inv = quant_scale(scale);
  int8_t* qr = Xq + (size_t)row * K;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int q = t + j * BS;
    if (q < nchunks) {
      int code[8];
      uint32_t bm8 = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t hb = (uint16_t)(((uint32_t)raw[j][e >> 1] >> ((e & 1) * 16)) & 0xffffu);
        bool b;
        if constexpr (kKeep) b = (bigm[j] >> e) & 1u;
        else b = big(hb & 0x7fffu);
        bm8 |= (uint32_t)b << e;
        code[e] = b ? 0 : quant_code(h2f(hb), inv);
      }
      v2i packed = {(int)pack4_i8(code[0], code[1], code[2], code[3]),
                    (int)pack4_i8(code[4], code[5], code[6], code[7])};
      *reinterpret_cast<v2i*>(qr + q * 8) = packed;
      if (bm8) atomicOr(flags + (q >> 2), bm8 << ((q & 3) * 8));
    }
  }
  if (t == 0) {
    sx[row] = scale;
    rowval[row] = bm > 0 ? (int)bc : -1;
  }
}

// Fix-up after rowpass_kernel, kFixRows rows per workgroup.  The flag words
// and their prefix counts (the rank of each outlier column) are loaded once per
// workgroup.  A row whose recorded column is regular only has the codes of the
// outlier columns zeroed and their values copied to X_O at their rank (the
// gathers of all the workgroup's rows in flight together); a row whose recorded
// column is an outlier column is recomputed by the whole workgroup in two
// passes over the row in 16-byte pieces (its maximum over the regular columns,
// then the codes), with the rules of rowquant_kernel.  Workgroup 0 writes the
// ascending index list and the outlier count.
// ZP: the row's two recorded columns (its range's ends) come from the end of
// its X_O capacity and its zero point from rowval; outlier columns get the
// zero point's code; the recompute follows rowquant_kernel's zero-point rules.
constexpr int kFixThreads = 256, kFixRows = 16;
template <bool ZP>
__global__ __launch_bounds__(kFixThreads) void rowfix_kernel(const uint16_t* __restrict__ X, int M,
                                                            int K,
                                                            const uint32_t* __restrict__ flags,
                                                            int32_t* __restrict__ rowval,
                                                            int8_t* __restrict__ Xq,
                                                            float* __restrict__ sx,
                                                            int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ n_out,
                                                            uint16_t* __restrict__ X_O) {
  constexpr int BS = kFixThreads;
  __shared__ uint32_t s_flags[kMaxFlagWords];
  __shared__ int s_rank[kMaxFlagWords];
  __shared__ int s_tmp[BS / 64 + 1];
  __shared__ int s_full[kFixRows];
  __shared__ int s_c0[kFixRows], s_c1[kFixRows], s_zq[kFixRows];
  __shared__ uint32_t s_max[BS / 64];
  __shared__ float s_lo[ZP ? BS / 64 : 1], s_hi[ZP ? BS / 64 : 1];
  const int t = threadIdx.x;
  const int nw = (K + 31) >> 5;
  const int r0 = blockIdx.x * kFixRows;
  const int nr = min(kFixRows, M - r0);
  for (int w = t; w < nw; w += BS) s_flags[w] = flags[w];
  // the rows' recorded columns (and zero points) into LDS before the barrier,
  // so that these loads are complete before any X_O store of the workgroup
  if (t < nr) {
    if constexpr (ZP) {
      const int32_t* cols = reinterpret_cast<const int32_t*>(X_O + (size_t)(r0 + t) * K + K - 4);
      s_c0[t] = cols[0];
      s_c1[t] = cols[1];
      s_zq[t] = rowval[r0 + t] - 128;   // the code of 0
    } else {
      s_c0[t] = rowval[r0 + t];
      s_c1[t] = -1;
      s_zq[t] = 0;
    }
  }
  lds_sync();
  const int per = (nw + BS - 1) / BS;
  const int w0 = t * per, w1 = min(nw, w0 + per);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __builtin_popcount(s_flags[w]);
  int total;
  int base = block_excl_scan<BS>(cnt, s_tmp, &total);
  for (int w = w0; w < w1; ++w) {
    s_rank[w] = base;
    base += __builtin_popcount(s_flags[w]);
  }
  if (t < nr) {
    const int c0 = s_c0[t], c1 = s_c1[t];
    s_full[t] = (c0 >= 0 && ((s_flags[c0 >> 5] >> (c0 & 31)) & 1u)) ||
                (c1 >= 0 && ((s_flags[c1 >> 5] >> (c1 & 31)) & 1u));
  }
  lds_sync();
  // regular recorded column: zero the outlier columns' codes, gather their
  // values; the loads of all the rows go out before any store (rows past M
  // re-read the last row and store nothing).  Offsets inside the workgroup's
  // kFixRows rows fit in 32 bits (16 * K).
  const uint16_t* xw = X + (size_t)r0 * K;
  uint16_t* ow = X_O + (size_t)r0 * K;
  int8_t* qw = Xq + (size_t)r0 * K;
  for (int w = w0; w < w1; ++w) {
    uint32_t f = s_flags[w];
    int r = s_rank[w];
    while (f) {
      const int j = w * 32 + __builtin_ctz(f);
      uint16_t v[kFixRows];
#pragma unroll
      for (int i = 0; i < kFixRows; ++i) v[i] = xw[min(i, nr - 1) * K + j];
#pragma unroll
      for (int i = 0; i < kFixRows; ++i) {
        if (i < nr && !s_full[i]) {
          ow[i * K + r] = v[i];
          qw[i * K + j] = (int8_t)s_zq[i];
        }
      }
      ++r;
      f &= f - 1u;
    }
  }
  // outlier recorded column: the row again, with the method's scale
  const int nchunks = K >> 3;
  for (int i = 0; i < nr; ++i) {
    if (!s_full[i]) continue;   // uniform
    const int row = r0 + i;
    const buf_rsrc rx = make_rsrc(X + (size_t)row * K, (uint32_t)K * 2u);
    uint32_t mx = 0;
    float lo = 0.0f, hi = 0.0f;   // zero-point codes: the range always contains 0
    for (int q = t; q < nchunks; q += BS) {
      const v4i x = buf_load16(rx, (uint32_t)q * 16u);
      const uint32_t ob = (s_flags[q >> 2] >> ((q & 3) * 8)) & 0xffu;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t hb = ((uint32_t)x[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        if (!((ob >> e) & 1u)) {
          if constexpr (ZP) {
            const float v = h2f((uint16_t)hb);
            lo = __builtin_fminf(lo, v);
            hi = __builtin_fmaxf(hi, v);
          } else {
            const uint32_t h = hb & 0x7fffu;
            mx = h > mx ? h : mx;
          }
        }
      }
    }
    float scale, inv;
    int zpv = 0;
    if constexpr (ZP) {
      lo = wave_min(lo);
      hi = wave_max(hi);
      if ((t & 63) == 0) {
        s_lo[t >> 6] = lo;
        s_hi[t >> 6] = hi;
      }
      __syncthreads();
#pragma unroll
      for (int w = 0; w < BS / 64; ++w) {
        lo = __builtin_fminf(lo, s_lo[w]);
        hi = __builtin_fmaxf(hi, s_hi[w]);
      }
      const float range = hi - lo;
      inv = range > 0.0f ? 255.0f / range : 0.0f;
      zpv = (int)__builtin_roundf(-lo * inv);
      scale = range / 255.0f;
    } else {
      mx = wave_max_u32(mx);
      if ((t & 63) == 0) s_max[t >> 6] = mx;
      __syncthreads();
      mx = 0;
#pragma unroll
      for (int w = 0; w < BS / 64; ++w) mx = s_max[w] > mx ? s_max[w] : mx;
      scale = h2f((uint16_t)mx);
      inv = quant_scale(scale);
    }
    int8_t* qr = Xq + (size_t)row * K;
    uint16_t* orow = X_O + (size_t)row * K;
    for (int q = t; q < nchunks; q += BS) {
      const v4i x = buf_load16(rx, (uint32_t)q * 16u);
      const int word = q >> 2, sh = (q & 3) * 8;
      const uint32_t ob = (s_flags[word] >> sh) & 0xffu;
      int code[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t hb = (uint16_t)(((uint32_t)x[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
        if constexpr (ZP) {
          int cz = ((ob >> e) & 1u) ? zpv : (int)__builtin_roundf(h2f(hb) * inv) + zpv;
          cz = cz < 0 ? 0 : (cz > 255 ? 255 : cz);
          code[e] = cz - 128;
        } else {
          code[e] = ((ob >> e) & 1u) ? 0 : quant_code(h2f(hb), inv);
        }
      }
      v2i packed = {(int)pack4_i8(code[0], code[1], code[2], code[3]),
                    (int)pack4_i8(code[4], code[5], code[6], code[7])};
      *reinterpret_cast<v2i*>(qr + q * 8) = packed;
      if (ob) {
        const uint32_t fw = s_flags[word];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if ((ob >> e) & 1u) {
            const int bit = sh + e;
            orow[s_rank[word] + __builtin_popcount(fw & ((1u << bit) - 1u))] =
                (uint16_t)(((uint32_t)x[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
          }
        }
      }
    }
    if (t == 0) {
      sx[row] = scale;
      if constexpr (ZP) rowval[row] = zpv;
    }
    __syncthreads();   // s_max, s_lo, s_hi are reused by the next recomputed row
  }
  if (blockIdx.x == 0) {
    for (int w = t; w < nw; w += BS) {
      uint32_t f = s_flags[w];
      int r = s_rank[w];
      while (f) {
        idx[r++] = w * 32 + __builtin_ctz(f);
        f &= f - 1u;
      }
    }
    if (t == 0) *n_out = total;
  }
}

// ---- small M (1 <= M <= 16): one workgroup per 512-column slice -------------------
// All rows of a slice sit in one workgroup, so its column maxima are complete
// there.  The scan kernel writes the slice's flag words (every word is written,
// so no clear is needed), its outlier count and, per row, the maximum over the
// regular columns: magnitude bits, or in zero-point mode the largest and
// smallest value keys (an outlier or out-of-range value counts as 0, which the
// range contains anyway).  The quantize kernel reduces the partials of all
// slices to the row scales, ranks its outlier columns after those of the
// slices before it, and writes the codes, outlier values and indices of its
// slice; slice 0 writes the row scales, zero points and the outlier count.
constexpr int kSmallThreads = 256;   // wave w holds rows w, w + 4, w + 8, w + 12


// X[r][c .. c+8) of the lane's rows as fp16 (zero past M or K).
__device__ __forceinline__ void small_load_rows(const uint16_t* X, int M, int K, int c,
                                                v4i (&x)[4]) {
  const int wave = threadIdx.x >> 6;
  const buf_rsrc rx = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave + 4 * i;
    x[i] = buf_load16(rx, r < M && c < K ? (uint32_t)(r * K + c) * 2u : kBufOff);
  }
}

template <bool ZP>
__global__ __launch_bounds__(kSmallThreads) void act_small_scan_kernel(
    const uint16_t* __restrict__ X, int M, int K, float threshold, int enabled,
    uint32_t* __restrict__ flags, uint32_t* __restrict__ part) {
  __shared__ uint32_t s_cm[kSmallThreads / 64][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sl = blockIdx.x, nsl = gridDim.x;
  const int c = sl * kActSlice + lane * 8;
  v4i x[4];
  small_load_rows(X, M, K, c, x);

  // column maxima of the lane's 8 columns: over the wave's rows, then the waves
  u16x2 cm[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cm[j] = u16x2{0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      cm[j] = __builtin_elementwise_max(cm[j],
                                        __builtin_bit_cast(u16x2, habs2_nonan((uint32_t)x[i][j])));
    s_cm[wave][lane][j] = __builtin_bit_cast(uint32_t, cm[j]);
  }
  lds_sync();
  uint32_t bits = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u16x2 v = {0, 0};
#pragma unroll
    for (int w = 0; w < kSmallThreads / 64; ++w)
      v = __builtin_elementwise_max(v, __builtin_bit_cast(u16x2, s_cm[w][lane][j]));
    if (enabled) {
      if (h2f(v[0]) >= threshold) bits |= 1u << (2 * j);
      if (h2f(v[1]) >= threshold) bits |= 2u << (2 * j);
    }
  }

  // the slice's flag words (4 lanes per word) and outlier count
  uint32_t wb = bits << ((lane & 3) * 8);
  wb |= __shfl_xor(wb, 1, 64);
  wb |= __shfl_xor(wb, 2, 64);
  const int word = sl * (kActSlice / 32) + (lane >> 2);
  if (wave == 0 && (lane & 3) == 0 && word < ((K + 31) >> 5)) flags[word] = wb;
  const int cnt = wave_sum(__builtin_popcount(bits));
  if (threadIdx.x == 0) part[sl] = (uint32_t)cnt;

  // per row: the maximum (and minimum key) over the regular columns
  uint32_t keep[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t b0 = (bits >> (2 * j)) & 1u, b1 = (bits >> (2 * j + 1)) & 1u;
    keep[j] = ((b0 - 1u) & 0xffffu) | ((b1 - 1u) << 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave + 4 * i;
    if (r >= M) break;   // uniform over the wave
    u16x2 hi2 = {0, 0}, lo2 = {0xffff, 0xffff};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = (uint32_t)x[i][j] & keep[j];
      if constexpr (ZP) {
        const u16x2 k2 = __builtin_bit_cast(u16x2, f16x2_keys(v));
        hi2 = __builtin_elementwise_max(hi2, k2);
        lo2 = __builtin_elementwise_min(lo2, k2);
      } else {
        hi2 = __builtin_elementwise_max(hi2, __builtin_bit_cast(u16x2, v & 0x7fff7fffu));
      }
    }
    const uint32_t hi = wave_max_u32(hi2[0] > hi2[1] ? hi2[0] : hi2[1]);
    if (lane == 0) part[nsl + sl * kActSmallRows + r] = hi;
    if constexpr (ZP) {
      const uint32_t lo = wave_min_u32(lo2[0] < lo2[1] ? lo2[0] : lo2[1]);
      if (lane == 0) part[nsl + (nsl + sl) * kActSmallRows + r] = lo;
    }
  }
}

template <bool ZP>
__global__ __launch_bounds__(kSmallThreads) void act_small_quant_kernel(
    const uint16_t* __restrict__ X, int M, int K, const uint32_t* __restrict__ flags,
    const uint32_t* __restrict__ part, int8_t* __restrict__ Xq, float* __restrict__ sx,
    int32_t* __restrict__ zp, int32_t* __restrict__ idx, int32_t* __restrict__ n_out,
    uint16_t* __restrict__ X_O) {
  constexpr int kGroups = kSmallThreads / kActSmallRows;   // 16 slice groups
  __shared__ uint32_t s_hi[kGroups][kActSmallRows];
  __shared__ uint32_t s_lo[ZP ? kGroups : 1][kActSmallRows];
  __shared__ int s_cnt[kSmallThreads / 64][2];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int sl = blockIdx.x, nsl = gridDim.x;
  const int c = sl * kActSlice + lane * 8;
  const int nw = (K + 31) >> 5;
  v4i x[4];
  small_load_rows(X, M, K, c, x);
  const int word = sl * (kActSlice / 32) + (lane >> 2);
  const uint32_t fw = buf_load_u32(make_rsrc(flags, (uint32_t)nw * 4u), (uint32_t)word * 4u);

  // row partials of all slices: thread (g, m) reduces slices g, g + 16, ...
  {
    const int m = t % kActSmallRows, g = t / kActSmallRows;
    uint32_t hi = 0, lo = 0xffffu;
    if (m < M) {
      for (int s = g; s < nsl; s += kGroups) {
        const uint32_t h = part[nsl + s * kActSmallRows + m];
        hi = h > hi ? h : hi;
        if constexpr (ZP) {
          const uint32_t l = part[nsl + (nsl + s) * kActSmallRows + m];
          lo = l < lo ? l : lo;
        }
      }
    }
    s_hi[g][m] = hi;
    if constexpr (ZP) s_lo[g][m] = lo;
  }
  // outliers of the slices before this one, and of all slices
  int before = 0, total = 0;
  for (int s = t; s < nsl; s += kSmallThreads) {
    const int v = (int)part[s];
    total += v;
    before += s < sl ? v : 0;
  }
  before = wave_sum(before);
  total = wave_sum(total);
  if (lane == 0) {
    s_cnt[wave][0] = before;
    s_cnt[wave][1] = total;
  }
  lds_sync();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kSmallThreads / 64; ++w) {
    base += s_cnt[w][0];
    total += s_cnt[w][1];
  }

  // ranks of the lane's outlier columns: after the slices before and the lanes before
  const uint32_t bits = (fw >> ((lane & 3) * 8)) & 0xffu;
  const int pc = __builtin_popcount(bits);
  const int rank0 = base + wave_incl_scan(pc) - pc;
  if (wave == 0 && bits) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((bits >> e) & 1u) idx[rank0 + __builtin_popcount(bits & ((1u << e) - 1u))] = c + e;
  }
  if (sl == 0 && t == 0) *n_out = total;

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave + 4 * i;
    if (r >= M) break;   // uniform over the wave
    uint32_t mh = 0, ml = 0xffffu;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      mh = s_hi[g][r] > mh ? s_hi[g][r] : mh;
      if constexpr (ZP) ml = s_lo[g][r] < ml ? s_lo[g][r] : ml;
    }
    float inv, scale;
    int zpv = 0;
    if constexpr (ZP) {
      // [blog, "Introduction to model quantization"], the unsigned scheme
      const float hi = __builtin_fmaxf(f16_of_key(mh), 0.0f);
      const float lo = __builtin_fminf(f16_of_key(ml), 0.0f);
      const float range = hi - lo;
      inv = range > 0.0f ? 255.0f / range : 0.0f;
      zpv = (int)__builtin_roundf(-lo * inv);
      scale = range / 255.0f;
    } else {
      scale = h2f((uint16_t)mh);
      inv = quant_scale(scale);
    }
    if (c < K) {
      int code[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t hb = (uint16_t)(((uint32_t)x[i][e >> 1] >> ((e & 1) * 16)) & 0xffffu);
        const bool out = (bits >> e) & 1u;
        if constexpr (ZP) {
          int cc = out ? zpv : (int)__builtin_roundf(h2f(hb) * inv) + zpv;
          cc = cc < 0 ? 0 : (cc > 255 ? 255 : cc);
          code[e] = cc - 128;
        } else {
          code[e] = out ? 0 : quant_code(h2f(hb), inv);
        }
      }
      const v2i packed = {(int)pack4_i8(code[0], code[1], code[2], code[3]),
                          (int)pack4_i8(code[4], code[5], code[6], code[7])};
      *reinterpret_cast<v2i*>(Xq + (size_t)r * K + c) = packed;
      if (bits) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((bits >> e) & 1u)
            X_O[(size_t)r * K + rank0 + __builtin_popcount(bits & ((1u << e) - 1u))] =
                (uint16_t)(((uint32_t)x[i][e >> 1] >> ((e & 1) * 16)) & 0xffffu);
      }
    }
    if (sl == 0 && lane == 0) {
      sx[r] = scale;
      if constexpr (ZP) zp[r] = zpv;
    }
  }
}

template <int BS, int NCH>
static void launch_rowquant(const uint16_t* X, int M, int K, bool zp, const Workspace& ws,
                            hipStream_t stream) {
  if (zp)
    hipLaunchKernelGGL((rowquant_kernel<BS, NCH, true>), dim3(M), dim3(BS), 0, stream, X, M, K,
                       (const uint32_t*)ws.flags, ws.Xq, ws.sx, ws.zp, ws.idx, ws.n_out, ws.X_O);
  else
    hipLaunchKernelGGL((rowquant_kernel<BS, NCH, false>), dim3(M), dim3(BS), 0, stream, X, M, K,
                       (const uint32_t*)ws.flags, ws.Xq, ws.sx, nullptr, ws.idx, ws.n_out,
                       ws.X_O);
}

// Row pass, then its fix-up (absmax codes, M > 256, decomposition on; the
// flags cleared first).  The zero-point array of the workspace, unused by
// absmax codes, carries each row's recorded column from one to the other.
template <int BS, int NCH>
static void launch_rowpass(const uint16_t* X, int M, int K, float threshold, bool zp,
                           const Workspace& ws, hipStream_t stream) {
  const dim3 fgrid((M + kFixRows - 1) / kFixRows), fblock(kFixThreads);
  if (zp) {
    hipLaunchKernelGGL((rowpass_kernel<BS, NCH, true>), dim3(M), dim3(BS), 0, stream, X, M, K,
                       threshold, ws.flags, ws.Xq, ws.sx, ws.zp, ws.X_O);
    hipLaunchKernelGGL(rowfix_kernel<true>, fgrid, fblock, 0, stream, X, M, K,
                       (const uint32_t*)ws.flags, ws.zp, ws.Xq, ws.sx, ws.idx, ws.n_out, ws.X_O);
  } else {
    hipLaunchKernelGGL((rowpass_kernel<BS, NCH, false>), dim3(M), dim3(BS), 0, stream, X, M, K,
                       threshold, ws.flags, ws.Xq, ws.sx, ws.zp, ws.X_O);
    hipLaunchKernelGGL(rowfix_kernel<false>, fgrid, fblock, 0, stream, X, M, K,
                       (const uint32_t*)ws.flags, ws.zp, ws.Xq, ws.sx, ws.idx, ws.n_out, ws.X_O);
  }
}

hipError_t launch_quantize_activation(const uint16_t* X, int M, int K, float threshold,
                                      bool enabled, const Workspace& ws, hipStream_t stream,
                                      bool zp) {
  if (M >= 1 && M <= kActSmallRows) {
    const dim3 grid(act_slices(K)), block(kSmallThreads);
    if (zp) {
      hipLaunchKernelGGL(act_small_scan_kernel<true>, grid, block, 0, stream, X, M, K, threshold,
                         (int)enabled, ws.flags, ws.act_part);
      hipLaunchKernelGGL(act_small_quant_kernel<true>, grid, block, 0, stream, X, M, K,
                         (const uint32_t*)ws.flags, (const uint32_t*)ws.act_part, ws.Xq, ws.sx,
                         ws.zp, ws.idx, ws.n_out, ws.X_O);
    } else {
      hipLaunchKernelGGL(act_small_scan_kernel<false>, grid, block, 0, stream, X, M, K, threshold,
                         (int)enabled, ws.flags, ws.act_part);
      hipLaunchKernelGGL(act_small_quant_kernel<false>, grid, block, 0, stream, X, M, K,
                         (const uint32_t*)ws.flags, (const uint32_t*)ws.act_part, ws.Xq, ws.sx,
                         nullptr, ws.idx, ws.n_out, ws.X_O);
    }
    return hipGetLastError();
  }
  const int bx = (K + kColStrip - 1) / kColStrip;
  if (M <= 32 * 8) {
    // narrow strips over every row: every flag word stored, so no clear launch
    const dim3 grid((K + kStripCols - 1) / kStripCols), block(kColThreads);
    const int sc = (int)enabled;
    if (M <= 32)
      hipLaunchKernelGGL(colscan_strip_kernel<1>, grid, block, 0, stream, X, M, K, threshold, sc,
                         ws.flags);
    else if (M <= 64)
      hipLaunchKernelGGL(colscan_strip_kernel<2>, grid, block, 0, stream, X, M, K, threshold, sc,
                         ws.flags);
    else if (M <= 128)
      hipLaunchKernelGGL(colscan_strip_kernel<4>, grid, block, 0, stream, X, M, K, threshold, sc,
                         ws.flags);
    else
      hipLaunchKernelGGL(colscan_strip_kernel<8>, grid, block, 0, stream, X, M, K, threshold, sc,
                         ws.flags);
  } else if (!enabled) {
    // one row block: every flag word is stored, so no clear launch
    hipLaunchKernelGGL(colflags_kernel<true>, dim3(bx, 1), dim3(kColThreads), 0, stream, X, M, K,
                       M, threshold, (int)enabled, ws.flags);
  } else {
    // one read of X (rowpass_kernel), then the fix-up
    const hipError_t e = launch_fill_u32(ws.flags, (K + 31) / 32, 0u, stream);
    if (e != hipSuccess) return e;
    const int nch = K / 8;
    if (nch <= 256) launch_rowpass<256, 1>(X, M, K, threshold, zp, ws, stream);
    else if (nch <= 512) launch_rowpass<256, 2>(X, M, K, threshold, zp, ws, stream);
    else if (nch <= 1024) launch_rowpass<256, 4>(X, M, K, threshold, zp, ws, stream);
    else if (nch <= 2048) launch_rowpass<512, 4>(X, M, K, threshold, zp, ws, stream);
    else if (nch <= 4096) launch_rowpass<1024, 4>(X, M, K, threshold, zp, ws, stream);
    else if (nch <= 7168) launch_rowpass<1024, 7>(X, M, K, threshold, zp, ws, stream);
    else if (nch <= 8192) launch_rowpass<1024, 8>(X, M, K, threshold, zp, ws, stream);
    else if (nch <= 16384) launch_rowpass<1024, 16>(X, M, K, threshold, zp, ws, stream);
    else launch_rowpass<1024, 17>(X, M, K, threshold, zp, ws, stream);
    return hipGetLastError();
  }
  if (M > 0) {
    // Few 16-byte chunks per thread and wide workgroups: the row's loads are
    // spread over many waves (measured on MI355X: 2048 x 14336 in 24.6 us with
    // 512 threads x 4 chunks against 43 us with 256 x 32; 4096 x 57344 in
    // 164 us with 1024 x 7 against 232 us with 256 x 32).
    const int nch = K / 8;
    if (nch <= 256) launch_rowquant<256, 1>(X, M, K, zp, ws, stream);
    else if (nch <= 512) launch_rowquant<256, 2>(X, M, K, zp, ws, stream);
    else if (nch <= 1024) launch_rowquant<256, 4>(X, M, K, zp, ws, stream);
    else if (nch <= 2048) launch_rowquant<512, 4>(X, M, K, zp, ws, stream);
    else if (nch <= 4096) launch_rowquant<1024, 4>(X, M, K, zp, ws, stream);
    else if (nch <= 7168) launch_rowquant<1024, 7>(X, M, K, zp, ws, stream);
    else if (nch <= 8192) launch_rowquant<1024, 8>(X, M, K, zp, ws, stream);
    else if (nch <= 16384) launch_rowquant<1024, 16>(X, M, K, zp, ws, stream);
    else launch_rowquant<1024, 17>(X, M, K, zp, ws, stream);
  }
  return hipGetLastError();
}

}  // namespace i8l
