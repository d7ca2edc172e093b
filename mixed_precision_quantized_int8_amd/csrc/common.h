// Shared device helpers of the gfx950 kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8l {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
#define I8L_MAX_K_DEV 133136

__device__ __forceinline__ float h2f(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t f2h(float f) {  // round to nearest even, overflow -> inf
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// |x| of an fp16 value as an fp16 bit pattern; for finite values the unsigned
// order of these patterns is the order of the magnitudes.
__device__ __forceinline__ uint32_t habs_bits(uint32_t b) { return b & 0x7fffu; }
// The same for the two fp16 values of a dword, with NaN patterns (above
// 0x7c00) mapped to 0: the outlier test asks whether some entry of a column
// has |x| >= threshold, which a NaN never does, so a column maximum built from
// these magnitudes ignores NaNs.  (m + 0x3ff carries into bit 15 of its half
// exactly when m > 0x7c00, and never into the other half.)
__device__ __forceinline__ uint32_t habs2_nonan(uint32_t x) {
  const uint32_t m = x & 0x7fff7fffu;
  const uint32_t nan = ((m + 0x03ff03ffu) >> 15) & 0x00010001u;
  return m & ~(nan * 0xffffu);
}

// Absmax code of one value: clamp(round_half_away(fp32(x) * inv), -127, 127),
// where inv = fl32(127 / absmax) is computed once per vector by the caller
// (IEEE division).  roundf rounds halfway cases away from zero.
__device__ __forceinline__ int quant_code(float x, float inv) {
  float v = x * inv;
  float r = __builtin_roundf(v);
  r = __builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__device__ __forceinline__ float quant_scale(float absmax) {
  return absmax > 0.0f ? 127.0f / absmax : 0.0f;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(d & 0xff) << 24);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses,
// then s_barrier.  Unlike __syncthreads() it does not wait for outstanding
// global loads, so loads issued earlier stay in flight across it.  The memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Raw buffer loads: the hardware checks every access against the size in the
// resource and returns zeros past it without touching memory, so an
// out-of-range lane needs no branch and no pointer select, only an offset at or
// past the end (kBufOff).  Offsets are in bytes; the resource holds the base
// and size (dword 3 = 0x00020000 is the gfx9 data format for raw byte access).
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
constexpr uint32_t kBufOff = 0x80000000u;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
template <int AUX = 0>
__device__ __forceinline__ v4i buf_load16(buf_rsrc r, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
}
__device__ __forceinline__ uint32_t buf_load_u32(buf_rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint16_t buf_load_u16(buf_rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint8_t buf_load_u8(buf_rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// Weight value rebuilt from its int8 code when no fp16 copy is kept:
// fp16(fl32(q * s) / 127), the product exact, one IEEE division, then round to
// nearest even ([blog, "Usage"]: code times the output feature's scale over 127).
__device__ __forceinline__ uint16_t dequant_w16(int q, float s) {
  return f2h(((float)q * s) / 127.0f);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Order-preserving u16 key of an fp16 value (finite values): positive values
// get the top bit set, negative ones are bit-inverted; applied to both halves.
__device__ __forceinline__ uint32_t f16x2_keys(uint32_t x) {
  const uint32_t neg = ((x >> 15) & 0x00010001u) * 0xffffu;
  return x ^ (0x80008000u | (neg & 0x7fff7fffu));
}
__device__ __forceinline__ float f16_of_key(uint32_t k) {
  return h2f((uint16_t)(k & 0x8000u ? k ^ 0x8000u : ~k & 0xffffu));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

}  // namespace i8l
