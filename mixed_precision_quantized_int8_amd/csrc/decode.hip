// Small-M ("decode") LLM.int8() linear layer.
//
// Same method as the prefill path ([blog, "A gentle summary of LLM.int8()"],
// [blog, "A closer look at the MatMul"]), shaped for M <= 16 rows, where the
// time is the single read of the int8 weight from HBM and a second launch
// costs more than the whole activation stage.
//
// Fused kernel (K <= 4096): the whole layer in one launch.  Each workgroup
// (8 waves) owns 64 output features (4 blocks of 16); the 8 waves split K into
// 8 chunks, and a wave owns its chunk of X over ALL rows, held in registers in
// the operand layout of v_mfma_i32_16x16x64_i8 (lane = row lr, 16-column
// group g).  Consequences:
//   * the outlier test of a column needs only the wave's own registers: an OR
//     of hit masks over the lanes of a row slot (DPP moves, no LDS);
//   * the row absmax over the regular columns is the only workgroup-wide
//     dependency: one LDS exchange and one barrier;
//   * the codes are computed in registers, already in MFMA operand layout;
//   * each wave adds the fp16 product of its own outlier columns on the matrix
//     cores (up to eight: the first four loaded into registers as soon as the
//     columns are known, the next four fetched into LDS behind the weight
//     stream; any further ones are read at the end);
//   * a second barrier sums the 8 waves' int32 partials (exact) and fp32
//     outlier partials, then the epilogue dequantizes and stores fp16.
// The weight is streamed with 16-byte buffer loads (default cache policy:
// measured faster here than the nontemporal hint), one 16-feature block after
// the other, all k-steps of a block back to back (~8 % more bandwidth than
// k-step by k-step across the blocks); the first PRE (8) loads of a wave are
// issued before the activation stage and the rest as soon as the wave's own
// row reduction is done, before the workgroup barrier.
// The K chunk a wave streams is rotated by the workgroup index (measured ~15%
// more HBM bandwidth than all starting at chunk 0).
// Workgroup 0 also writes the intermediates (Xq, sx, outlier list, X_O) to the
// workspace, right after its codes (behind its weight loads).
//
// Stream kernel (K > 4096): reads the intermediates written by the activation
// kernels and does the product and epilogue the same way, with the weight
// registers double-buffered across the wave's K chunk; in zero-point mode the
// accumulator is corrected by (128 - zp[m]) * wsum[n] and dequantized with
// sx * sw / 127.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace i8l {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kDecP = 4;                      // 16-feature blocks per workgroup
constexpr int kDecCols = 16 * kDecP;
constexpr int kDecMaxKS = 8;                  // fused kernel: k-steps per wave
constexpr int kDecOutPre = 4;                 // outlier columns per wave preloaded
constexpr int kDecOutDma = 4;                 // further ones fetched into LDS behind the stream
constexpr int kDecMaxOutLds = 64;             // stream kernel: outlier values in LDS
constexpr int kDecStreamRows = 64;            // stream kernel: rows of X (4 row groups)
constexpr int kDecOutReg = 8;                 // stream kernel: outlier weights per lane

#define I8L_DEC_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Zero bytes for lanes whose load is out of range (loads stay unconditional,
// so the number of loads in flight is fixed and waits stay exact).
__device__ __attribute__((aligned(64))) int8_t g_dec_zero[64];

struct DecodeArgs {
  const uint16_t* X;
  int M, K, N;
  const int8_t* Wq;
  const float* sw;
  const uint16_t* W_rows;
  const uint16_t* bias;   // fp16 [N] or NULL
  uint32_t thr;        // smallest fp16 magnitude pattern that is an outlier
                       // (0x10000 when the decomposition is off: never reached)
  uint16_t* Y;
  int32_t* n_out;
  int32_t* idx;
  float* sx;
  int8_t* Xq;
  uint16_t* X_O;
  int32_t* zp = nullptr;           // zero-point mode: zero points (read, or written by the fused kernel)
  const int32_t* wsum = nullptr;
};

bool decode_fits(int M, int K) { return M >= 1 && M <= 16 && K <= kDecWaves * kDecMaxKS * 64; }

__device__ __forceinline__ uint32_t half_at(const v4i (&v)[2], int e) {
  return ((uint32_t)v[e >> 3][(e & 7) >> 1] >> ((e & 1) * 16)) & 0xffffu;
}

// RHAZ(v) for |v| < 2^15, from w = trunc(v * 2^16): floor((|w| + 2^15) / 2^16)
// with the sign of w, computed as (w + 2^15 + (w < 0 ? -1 : 0)) >> 16
// (arithmetic shift); the code byte is byte 2 of that sum.
__device__ __forceinline__ uint32_t rhaz_sum(float v65) {
  const int w = (int)v65;   // truncates toward zero
  return (uint32_t)(w + 0x8000 + (w >> 31));
}

// 16 codes of one lane: round-half-away(x * inv) with inv65 = inv * 2^16
// (exact power-of-two scaling).  No clamp is needed: outlier values are
// zeroed beforehand and every other |x| <= absmax, so |x * inv| < 127.5.
__device__ __forceinline__ v4i codes16(const v4i (&x)[2], float inv65) {
  v4i a;
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // output dword i: elements 4i .. 4i+3
    uint32_t t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = rhaz_sum(h2f((uint16_t)half_at(x, 4 * i + e)) * inv65);
    const uint32_t p01 = __builtin_amdgcn_perm(t[1], t[0], 0x06020602u);   // t0.b2 t1.b2 ..
    const uint32_t p23 = __builtin_amdgcn_perm(t[3], t[2], 0x06020602u);   // .. t2.b2 t3.b2
    a[i] = (int)__builtin_amdgcn_perm(p23, p01, 0x07060100u);
  }
  return a;
}

// Zero-point codes of 16 values: clamp(round_half_away(x * inv) + zp, 0, 255)
// - 128 per byte, with inv65 = inv * 2^16 as above; |x * inv| <= 255, so the
// fixed-point rounding is exact.  Zeroed outlier values give zp - 128.
// zpc = 0x8000 + (zp - 128) * 2^16: adding a multiple of 2^16 before the
// arithmetic shift adds zp - 128 after it, so one add3 and one shift give
// round_half_away(x * inv) + zp - 128, and med3 clamps it to [-128, 127].
__device__ __forceinline__ v4i codes16_zp(const v4i (&x)[2], float inv65, int zpc) {
  v4i a;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int w = (int)(h2f((uint16_t)half_at(x, 4 * i + e)) * inv65);   // truncates
      const int q = (w + (w >> 31) + zpc) >> 16;
      b[e] = (uint32_t)(q < -128 ? -128 : (q > 127 ? 127 : q));   // v_med3_i32
    }
    const uint32_t p01 = __builtin_amdgcn_perm(b[1], b[0], 0x04000400u);   // b0.b0 b1.b0 ..
    const uint32_t p23 = __builtin_amdgcn_perm(b[3], b[2], 0x04000400u);   // b2.b0 b3.b0 ..
    a[i] = (int)__builtin_amdgcn_perm(p23, p01, 0x05040100u);
  }
  return a;
}



// KS: k-steps of 64 per wave (>= ceil(K / 64 / 8));
// R: k-steps packed into one register set (M <= 16 / R): lane row lr holds X
//    row lr % (16/R) of k-step (lr / (16/R)) of the set, so padding rows >= M
//    carry real data instead of zeros; the codes are moved to the MFMA operand
//    rows by lane shuffles;
// PRE: weight loads (of KS * kDecP, block by block) issued before the
//    activation stage.
// ZP: zero-point codes (row minimum and maximum instead of the absmax, codes
//    minus 128, accumulators corrected by (128 - zp) * wsum, scale range / 255).
// OR of h over the L lanes of one X row slot (lanes 16 g + L q + r, r < L; L
// a power of two up to 16) with DPP moves inside a 16-lane row: neighbour
// and pair swaps within quads, then the mirror image of each 8-lane half and
// of the row (no LDS round trip).
template <int L>
__device__ __forceinline__ uint32_t or_slot(uint32_t h) {
  if constexpr (L >= 2) h |= (uint32_t)__builtin_amdgcn_mov_dpp((int)h, 0xb1, 0xf, 0xf, false);   // quad_perm 1,0,3,2
  if constexpr (L >= 4) h |= (uint32_t)__builtin_amdgcn_mov_dpp((int)h, 0x4e, 0xf, 0xf, false);   // quad_perm 2,3,0,1
  if constexpr (L >= 8) h |= (uint32_t)__builtin_amdgcn_mov_dpp((int)h, 0x141, 0xf, 0xf, false);  // row_half_mirror
  if constexpr (L >= 16) h |= (uint32_t)__builtin_amdgcn_mov_dpp((int)h, 0x140, 0xf, 0xf, false); // row_mirror
  return h;
}

// Maximum (minimum) of v over the lanes lr, lr + L, lr + 2L, ... of each
// 16-lane row (L a power of two up to 16): DPP row rotations by 8, 4, ..., L.
template <int OFF>
__device__ __forceinline__ uint32_t row_ror(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x120 + OFF, 0xf, 0xf, false);
}
// v of lane (lr + s) mod 16 of the same 16-lane row (a rotation right by 16 - s
// moves each value s lanes down); s is a constant once inlined and unrolled
__device__ __forceinline__ uint32_t row_up(uint32_t v, int s) {
  switch (s & 15) {
    case 1: return row_ror<15>(v);
    case 2: return row_ror<14>(v);
    case 3: return row_ror<13>(v);
    case 4: return row_ror<12>(v);
    case 5: return row_ror<11>(v);
    case 6: return row_ror<10>(v);
    case 7: return row_ror<9>(v);
    case 8: return row_ror<8>(v);
    case 9: return row_ror<7>(v);
    case 10: return row_ror<6>(v);
    case 11: return row_ror<5>(v);
    case 12: return row_ror<4>(v);
    case 13: return row_ror<3>(v);
    case 14: return row_ror<2>(v);
    case 15: return row_ror<1>(v);
    default: return v;
  }
}
template <int L>
__device__ __forceinline__ uint32_t max_rows(uint32_t v) {
  if constexpr (L <= 8) v = __builtin_elementwise_max(v, row_ror<8>(v));
  if constexpr (L <= 4) v = __builtin_elementwise_max(v, row_ror<4>(v));
  if constexpr (L <= 2) v = __builtin_elementwise_max(v, row_ror<2>(v));
  if constexpr (L <= 1) v = __builtin_elementwise_max(v, row_ror<1>(v));
  return v;
}
template <int L>
__device__ __forceinline__ uint32_t min_rows(uint32_t v) {
  if constexpr (L <= 8) v = __builtin_elementwise_min(v, row_ror<8>(v));
  if constexpr (L <= 4) v = __builtin_elementwise_min(v, row_ror<4>(v));
  if constexpr (L <= 2) v = __builtin_elementwise_min(v, row_ror<2>(v));
  if constexpr (L <= 1) v = __builtin_elementwise_min(v, row_ror<1>(v));
  return v;
}

template <int KS, int R, int PRE, bool ZP>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeArgs d) {
  constexpr int MR = 16 / R;         // X rows per slot
  constexpr int NSET = KS / R;       // register sets
  __shared__ v4i sRed[kDecWaves][kDecP][64];        // int32 partials, D layout
  // fp32 outlier partials [col][m] (zero for a wave without outlier columns):
  // the epilogue reads a lane's four rows with one 16-byte read per wave
  __shared__ v4f sYo[kDecWaves][kDecCols][4];
  __shared__ uint32_t sRowMax[kDecWaves][16];       // per chunk, per row
  __shared__ uint32_t sRowMin[ZP ? kDecWaves : 1][16];   // zero-point mode: minimum key
  __shared__ int sCnt[kDecWaves];                   // outliers per K chunk
  // outlier columns kDecOutPre .. kDecOutPre + kDecOutDma - 1 of each wave:
  // weight values (lane = feature: the fp16 weight, or the code when no fp16
  // weight is kept; slots kDecOutPre ..) and X values (lane = row), written by
  // LDS-DMA loads, which give every lane a dword (the value zero-extended)
  // whatever the load size.  Slots 0 .. kDecOutPre - 1 of sOw take the fp16
  // weight values of the first columns (held in registers until then) for the
  // matrix-core product of the outlier columns.
  __shared__ uint32_t sOw[kDecWaves][kDecOutPre + kDecOutDma][64];
  __shared__ uint32_t sOx[kDecWaves][kDecOutDma][64];

  const int M = d.M, K = d.K, N = d.N;
  const int lane = threadIdx.x & 63;
  // the wave index is uniform; saying so keeps everything derived from it
  // (chunk bounds, outlier columns, resources) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, g = lane >> 4;
  const int rr = lr % MR, q = lr / MR;   // X row and slot of this lane
  const int n0 = blockIdx.x * kDecCols;
  const int nsteps = (K + 63) >> 6;
  const int kc = (wave + blockIdx.x) % kDecWaves;
  const int s0 = kc * nsteps / kDecWaves, s1 = (kc + 1) * nsteps / kDecWaves;   // s1 - s0 <= KS

  // ---- loads: X chunk of this wave, the output feature's scale, the weight ----
  // X rows >= M and columns outside this wave's chunk read as zero (buffer
  // range check); weight rows >= N read as zero, and weight bytes outside the
  // chunk meet zero codes.
  const buf_rsrc rx = make_rsrc(d.X, (uint32_t)(M * K * 2));
  v4i xr[NSET][2];   // X[rr][(s0 + j*R + q)*64 + 16g + 8h .. +8] as fp16
#pragma unroll
  for (int j = 0; j < NSET; ++j) {
    const int t = s0 + j * R + q, k = t * 64 + 16 * g;
    const uint32_t off = t < s1 && k < K ? (uint32_t)(rr * K + k) * 2u : kBufOff;
    xr[j][0] = buf_load16(rx, off);
    xr[j][1] = buf_load16(rx, off + 16u);
  }
  const int ne = n0 + (wave & (kDecP - 1)) * 16 + lr;   // epilogue feature of this lane
  const float swv = d.sw[ne < N ? ne : N - 1];
  const int wsn = ZP ? d.wsum[ne < N ? ne : N - 1] : 0;
  // bias (zero-sized resource when there is none: the load reads nothing)
  const uint16_t bvb = buf_load_u16(make_rsrc(d.bias, d.bias ? (uint32_t)N * 2u : 0u),
                                    (uint32_t)(ne < N ? ne : N - 1) * 2u);

  const int nrows = N - n0 < kDecCols ? N - n0 : kDecCols;
  const buf_rsrc rw = make_rsrc(d.Wq + (size_t)n0 * K, (uint32_t)(nrows * K));
  const uint32_t wb = (uint32_t)(lr * K + s0 * 64 + 16 * g);
  v4i fb[KS][kDecP];
  // load i of the wave's KS * kDecP: feature block i / KS, k-step i % KS, so
  // the chunk's bytes of each weight row are requested back to back
  auto load_b = [&](int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int c = i / KS, u = i % KS;
      fb[u][c] = buf_load16(rw, wb + (uint32_t)(c * 16 * K + u * 64));
    }
  };
  constexpr int kLoads = KS * kDecP;
  constexpr int kPre = PRE < kLoads ? PRE : kLoads;
  load_b(0, kPre);
  __builtin_amdgcn_sched_barrier(0);   // the stream goes out before the stage below

  // ---- outlier columns and row absmax of this chunk ------------------------------
  // Per register set: the packed u16 maximum of the magnitudes decides whether
  // any value reaches the threshold; only then (rare) are the per-column hit
  // masks built, OR-ed over the rows of the slot, and the outlier values
  // zeroed in registers (so the row max and the codes need no masking).
  const uint32_t T = d.thr;
  u16x2 rmv = {0, 0};
  u16x2 kmax = {0, 0}, kmin = {0xffff, 0xffff};   // zero-point mode: value keys
  uint32_t hm[NSET];         // this lane's 16 columns: outlier bits (0 if the set has none)
  uint32_t hitsets = 0;      // uniform: sets with an outlier column
#pragma unroll
  for (int j = 0; j < NSET; ++j) {
    u16x2 smax = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      smax = __builtin_elementwise_max(
          smax, __builtin_bit_cast(u16x2, (uint32_t)xr[j][i >> 2][i & 3] & 0x7fff7fffu));
    const uint32_t lmax = smax[0] > smax[1] ? smax[0] : smax[1];
    hm[j] = 0;
    if (__ballot(lmax >= T) != 0) {
      // a column is an outlier when some entry has |x| >= T; a NaN (pattern
      // above 0x7c00) never does.  Per pair of magnitude patterns m (packed
      // u16): with d = m - T (mod 2^16) and L = 0x7c01 - T, min(d, L) - L has
      // its top bit set exactly when T <= m <= 0x7c00.
      const u16x2 tt = {(unsigned short)T, (unsigned short)T};
      const u16x2 ll = {(unsigned short)(0x7c01u - T), (unsigned short)(0x7c01u - T)};
      uint32_t fl[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u16x2 m = __builtin_bit_cast(u16x2, (uint32_t)xr[j][i >> 2][i & 3] & 0x7fff7fffu);
        fl[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(m - tt, ll) - ll);
      }
      // the 16 flags (bits 15 and 31 of each pair) into bits 0..15: the four
      // flag bytes of two pairs side by side (byte permute), then their top
      // bits (7, 15, 23, 31) gathered into bits 28..31 by one multiplication
      // (the partial products land on distinct bits: no carries)
      uint32_t h = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t p = __builtin_amdgcn_perm(fl[2 * k + 1], fl[2 * k], 0x07050301u) & 0x80808080u;
        h |= ((p * 0x00204081u) >> 28) << (4 * k);
      }
      h = or_slot<MR>(h);
      hm[j] = h;
      smax = u16x2{0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // 0xffff over each outlier half of the pair (its flag bit sign-extended)
        const uint32_t z0 = (uint32_t)((int)(h << (31 - 2 * i)) >> 31);
        const uint32_t z1 = (uint32_t)((int)(h << (30 - 2 * i)) >> 31);
        const uint32_t z = __builtin_amdgcn_perm(z1, z0, 0x05040100u);
        xr[j][i >> 2][i & 3] &= (int)~z;
        smax = __builtin_elementwise_max(
            smax, __builtin_bit_cast(u16x2, (uint32_t)xr[j][i >> 2][i & 3] & 0x7fff7fffu));
      }
      hitsets |= 1u << j;
    }
    rmv = __builtin_elementwise_max(rmv, smax);
    if constexpr (ZP) {   // outlier values are zeroed by now: they count as 0
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u16x2 k2 = __builtin_bit_cast(u16x2, f16x2_keys((uint32_t)xr[j][i >> 2][i & 3]));
        kmax = __builtin_elementwise_max(kmax, k2);
        kmin = __builtin_elementwise_min(kmin, k2);
      }
    }
  }
  // outlier columns of chunk step t as a wave-wide mask: bit l <-> column
  // (s0+t)*64 + l, so ascending column order is (t, bit)
  // (16-bit group masks read from one lane of each slot: t is a constant
  // wherever this is called, and so are the lanes)
  auto step_mask = [&](int t) -> uint64_t {
    const int j = t / R, qq = t % R;
    if (!((hitsets >> j) & 1u)) return 0;
    uint64_t m = 0;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
      m |= (uint64_t)((uint32_t)__builtin_amdgcn_readlane((int)hm[j], 16 * gg + qq * MR) & 0xffffu)
           << (16 * gg);
    return m;
  };
  // The per-step masks (kept in scalar registers), the number of outlier
  // columns and the first kDecOutPre + kDecOutDma of them, ascending (uniform).
  int wcount = 0;
  uint64_t msk[KS];
  int ko[kDecOutPre + kDecOutDma];
#pragma unroll
  for (int t = 0; t < KS; ++t) msk[t] = 0;
#pragma unroll
  for (int j = 0; j < kDecOutPre + kDecOutDma; ++j) ko[j] = -1;
  if (hitsets) {
#pragma unroll
    for (int t = 0; t < KS; ++t) msk[t] = step_mask(t);
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      uint64_t w = msk[t];
      wcount += __popcll(w);
#pragma unroll
      for (int j = 0; j < kDecOutPre + kDecOutDma; ++j) {
        if (w != 0 && ko[j] < 0) {
          ko[j] = (s0 + t) * 64 + __builtin_ctzll(w);
          w &= w - 1;
        }
      }
    }
  }
  const int found = wcount < kDecOutPre ? wcount : kDecOutPre;
  // Beyond kDecOutPre + kDecOutDma columns (rare) the columns are found by rank
  // from the per-step masks and their values read kDecOutBatch columns per
  // memory round trip.
  constexpr int kDecOutBatch = 8;
  // column of the r-th outlier of this chunk, ascending (uniform), -1 past the last
  auto nth_outlier = [&](int r) -> int {
    int k = -1;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const int cnt = __popcll(msk[t]);
      if (k < 0 && r >= 0 && r < cnt) {
        uint64_t m = msk[t];
        for (int i = 0; i < r; ++i) m &= m - 1;
        k = (s0 + t) * 64 + __builtin_ctzll(m);
      }
      r -= cnt;
    }
    return k;
  };
  // X values (lane = row) and weight-row values (lane = feature) of the first
  // kDecOutPre outlier columns, loaded now and used after the product
  // Without an fp16 weight (W_rows NULL) the value is rebuilt from the code
  // Wq[n][k] and sw[n]; both loads are always issued (the unused one reads
  // nothing), so the number of loads in flight stays fixed.
  const bool rebuild = d.W_rows == nullptr;
  const float swl = d.sw[n0 + lane < N ? n0 + lane : N - 1];
  uint16_t xo[kDecOutPre], wo[kDecOutPre];
  uint8_t wc[kDecOutPre];
#pragma unroll
  for (int j = 0; j < kDecOutPre; ++j) {
    const bool ok = j < found;
    xo[j] = buf_load_u16(rx, ok ? (uint32_t)(lane * K + ko[j]) * 2u : kBufOff);
    const buf_rsrc ro = make_rsrc(ok && !rebuild ? d.W_rows + (size_t)ko[j] * N + n0 : d.W_rows,
                                  ok && !rebuild ? (uint32_t)nrows * 2u : 0u);
    wo[j] = buf_load_u16(ro, (uint32_t)lane * 2u);
    wc[j] = buf_load_u8(rw, ok && rebuild ? (uint32_t)(lane * K + ko[j]) : kBufOff);
  }

  uint32_t rm, rn = 0;
  if constexpr (ZP) {
    rm = kmax[0] > kmax[1] ? kmax[0] : kmax[1];
    rn = kmin[0] < kmin[1] ? kmin[0] : kmin[1];
  } else {
    rm = rmv[0] > rmv[1] ? rmv[0] : rmv[1];
  }
  // over the slots (DPP rotations inside a 16-lane row: lanes lr, lr + MR, ...
  // hold the same row), then over the column groups
  rm = max_rows<MR>(rm);
  if constexpr (ZP) rn = min_rows<MR>(rn);
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    const uint32_t o = __shfl_xor(rm, off, 64);
    rm = o > rm ? o : rm;
    if constexpr (ZP) {
      const uint32_t o2 = __shfl_xor(rn, off, 64);
      rn = o2 < rn ? o2 : rn;
    }
  }

  // the rest of the weight stream goes out before the barrier: a wave waiting
  // there for the slowest wave of its workgroup keeps its loads in flight
  load_b(kPre, kLoads);
  // columns kDecOutPre .. kDecOutPre + kDecOutDma - 1 of this wave (many
  // outliers only): fetched into LDS right after the codes, below
  int kx[kDecOutDma];
#pragma unroll
  for (int u = 0; u < kDecOutDma; ++u) kx[u] = -1;
  if (lane < MR) sRowMax[kc][lane] = rm;
  if (ZP && lane < MR) sRowMin[ZP ? kc : 0][lane] = rn;
  if (lane == 0) sCnt[kc] = wcount;
  lds_sync();

  // ---- codes and the int8 product, one register set at a time ---------------------
  uint32_t mx = 0;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) mx = sRowMax[w][rr] > mx ? sRowMax[w][rr] : mx;
  float inv65, rowscale;
  int zpv = 0;
  if constexpr (ZP) {
    // [blog, "Introduction to model quantization"], the unsigned scheme: the
    // row's range, widened to contain 0, maps onto [0, 255]
    uint32_t mn = 0xffffu;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mn = sRowMin[w][rr] < mn ? sRowMin[w][rr] : mn;
    const float hi = __builtin_fmaxf(f16_of_key(mx), 0.0f);
    const float lo = __builtin_fminf(f16_of_key(mn), 0.0f);
    const float range = hi - lo;
    const float inv = range > 0.0f ? 255.0f / range : 0.0f;
    zpv = (int)__builtin_roundf(-lo * inv);
    inv65 = inv * 65536.0f;
    rowscale = range / 255.0f;
  } else {
    rowscale = h2f((uint16_t)mx);
    inv65 = quant_scale(rowscale) * 65536.0f;
  }
  const int zpc = 0x8000 + (zpv - 128) * 65536;   // zero-point codes: see codes16_zp
  // the row scales (and zero points) of this lane's epilogue rows 4 g .. 4 g + 3,
  // from the lanes that hold those rows (lane m holds row m for m < M), now
  // rather than from LDS in the tail
  float sxe[4];
  int zpe[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sxe[r] = __shfl(rowscale, 4 * g + r, 64);
    zpe[r] = ZP ? __shfl(zpv, 4 * g + r, 64) : 0;
  }
  v4i acc[kDecP];
#pragma unroll
  for (int c = 0; c < kDecP; ++c) acc[c] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < NSET; ++j) asm volatile("" : "+v"(xr[j][0]), "+v"(xr[j][1]));
  // all codes first (the weight is still in flight), then the products in the
  // order the weight arrives
  v4i a[KS];
#pragma unroll
  for (int j = 0; j < NSET; ++j) {
    v4i cj;
    if constexpr (ZP) {
      // positions past K or past this wave's chunk must contribute nothing:
      // their code is 0 (the zero point's code is not)
      const int tq = s0 + j * R + q;
      cj = tq < s1 && tq * 64 + 16 * g < K ? codes16_zp(xr[j], inv65, zpc) : v4i{0, 0, 0, 0};
    } else {
      cj = codes16(xr[j], inv65);
    }
#pragma unroll
    for (int qq = 0; qq < R; ++qq) {
      const int t = j * R + qq;
      // operand row lr < MR takes the codes of row lr, slot qq (lane lr + qq*MR)
      if (qq == 0) {
        a[t] = cj;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[t][i] = (int)row_up((uint32_t)cj[i], qq * MR);
      }
      if (R > 1 && lr >= MR) a[t] = v4i{0, 0, 0, 0};
    }
  }
  // ---- workspace intermediates (workgroup 0), behind the weight loads ------------
  // Written now rather than after the products, so that workgroup 0 does not end
  // last: the codes from registers (lane: row lr, 16 columns of k-step s0 + t),
  // the first kDecOutPre outlier columns of this chunk at their rank, and the row
  // scales, zero points and outlier count.  The LDS-fetched and further columns
  // (many outliers only) are written after the products.
  if (blockIdx.x == 0) {   // uniform
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const int k = (s0 + t) * 64 + 16 * g;
      if (lr < M && s0 + t < s1 && k < K) *reinterpret_cast<v4i*>(d.Xq + (size_t)lr * K + k) = a[t];
    }
    int rank = 0;
    for (int w = 0; w < kc; ++w) rank += sCnt[w];
#pragma unroll
    for (int j = 0; j < kDecOutPre; ++j) {
      if (j < found) {
        if (lane == 0) d.idx[rank + j] = ko[j];
        if (lane < M) d.X_O[(size_t)lane * K + rank + j] = xo[j];
      }
    }
    if (wave == 0) {   // lane = row for lanes < M (M <= 16 / R)
      if (lane < M) d.sx[lane] = rowscale;
      if (ZP && lane < M) d.zp[lane] = zpv;
      if (lane == 0) {
        int tot = 0;
        for (int w = 0; w < kDecWaves; ++w) tot += sCnt[w];
        *d.n_out = tot;
      }
    }
  }
  // The further outlier columns follow the stream into LDS: issued behind this
  // wave's weight loads, they land with them, not one round trip after them.
  // They go out only now, after the codes' LDS writes: the compiler makes an
  // LDS write that it cannot tell apart from an LDS-DMA destination wait for
  // every load issued so far, which would hold the codes (and the products
  // after them) until the whole weight had landed.
  __builtin_amdgcn_sched_barrier(0);
  if (wcount > kDecOutPre) {   // uniform
#pragma unroll
    for (int u = 0; u < kDecOutDma; ++u) {
      kx[u] = ko[kDecOutPre + u];
      if (kx[u] >= 0) {
        // X[lane][k]: lanes >= M read 0 from the range check
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, I8L_DEC_LDS(&sOx[wave][u][0]), 2,
                                                 (int)((uint32_t)(lane * K + kx[u]) * 2u), 0, 0, 0);
        if (rebuild)   // the code Wq[n0 + lane][k]
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, I8L_DEC_LDS(&sOw[wave][kDecOutPre + u][0]), 1,
                                                   (int)(uint32_t)(lane * K + kx[u]), 0, 0, 0);
        else           // the fp16 weight W[k][n0 + lane]
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              make_rsrc(d.W_rows + (size_t)kx[u] * N + n0, (uint32_t)nrows * 2u),
              I8L_DEC_LDS(&sOw[wave][kDecOutPre + u][0]), 2, (int)((uint32_t)lane * 2u), 0, 0, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < kDecP; ++c)
#pragma unroll
    for (int t = 0; t < KS; ++t)
      acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], fb[t][c], acc[c], 0, 0, 0);

  // ---- outlier product of this chunk's columns ----------------------------------
  // Up to kDecOutPre + kDecOutDma columns on the matrix cores: X_O (16 rows x
  // the columns, zero-padded to 16) times their fp16 weight rows (the columns x
  // 64 features) with v_mfma_f32_16x16x16_f16, one product per 16-feature
  // block, into fp32.  Lane l holds operand row (or feature) l % 16 and
  // columns 4 (l / 16) .. 4 (l / 16) + 3 of the wave's outlier list; columns
  // past the list are zero in both operands (an unwritten slot could hold a
  // NaN pattern).  The result has the layout of the int8 partials: lane l,
  // feature l % 16 of the block, rows 4 (l / 16) .. + 3.
  if (wcount > 0) {
    constexpr int kDecOutMfma = kDecOutPre + kDecOutDma;   // 8: two of the four groups
    const int nv = wcount < kDecOutMfma ? wcount : kDecOutMfma;   // uniform
    if (wcount > kDecOutPre) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // DMA landed
    // weight values of the first columns into their slots, fp16 (lane = feature)
#pragma unroll
    for (int j = 0; j < kDecOutPre; ++j)
      if (j < found)
        sOw[wave][j][lane] = rebuild ? dequant_w16((int)(int8_t)wc[j], swl) : wo[j];
    if (rebuild && wcount > kDecOutPre) {   // the fetched codes become fp16 values
#pragma unroll
      for (int u = 0; u < kDecOutDma; ++u)
        if (kx[u] >= 0)
          sOw[wave][kDecOutPre + u][lane] =
              dequant_w16((int)(int8_t)(sOw[wave][kDecOutPre + u][lane] & 0xffu), swl);
    }
    const int jb = 4 * g;   // this lane's first column
    // every operand value is read unconditionally and pinned in a register
    // (so the compiler cannot sink the reads into branches, one LDS round
    // trip each); the columns past the list are masked afterwards
    uint32_t xv0[4], xv1[4], bw[kDecP][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv0[i] = (uint32_t)__shfl((int)xo[i], lr, 64);   // column i, lanes 0-15
      xv1[i] = sOx[wave][i][lr];                        // column 4 + i, lanes 16-31
    }
#pragma unroll
    for (int c = 0; c < kDecP; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) bw[c][i] = sOw[wave][(jb + i) & (kDecOutMfma - 1)][c * 16 + lr];
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(xv0[i]), "+v"(xv1[i]));
#pragma unroll
    for (int c = 0; c < kDecP; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(bw[c][i]));
    uint32_t keep[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) keep[i] = jb + i < nv ? 0xffffu : 0u;
    uint32_t ax[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ax[i] = (g == 0 ? xv0[i] : xv1[i]) & keep[i];
    const v4h av = __builtin_bit_cast(v4h, v2i{(int)(ax[0] | (ax[1] << 16)), (int)(ax[2] | (ax[3] << 16))});
    v4f po[kDecP];
#pragma unroll
    for (int c = 0; c < kDecP; ++c) {
      const v4h bv = __builtin_bit_cast(
          v4h, v2i{(int)((bw[c][0] & keep[0]) | ((bw[c][1] & keep[1]) << 16)),
                   (int)((bw[c][2] & keep[2]) | ((bw[c][3] & keep[3]) << 16))});
      po[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bv, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kDecP; ++c) sYo[wave][c * 16 + lr][g] = po[c];   // rows 4g .. 4g+3
    // the rest (beyond kDecOutMfma, rare), straight from memory on the vector
    // units (lane = feature n0 + lane): all loads of a batch go out before any
    // of their values is used
    if (wcount > kDecOutMfma) {   // uniform
      float yo[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) yo[m] = 0.0f;
      for (int j0 = kDecOutMfma; j0 < wcount; j0 += kDecOutBatch) {   // uniform
        int kk[kDecOutBatch], xv[kDecOutBatch];
        float wv[kDecOutBatch];
#pragma unroll
        for (int u = 0; u < kDecOutBatch; ++u) kk[u] = nth_outlier(j0 + u);
#pragma unroll
        for (int u = 0; u < kDecOutBatch; ++u) {
          wv[u] = 0.0f;
          xv[u] = 0;
          if (kk[u] >= 0) {   // uniform
            if (n0 + lane < N)
              wv[u] = rebuild ? h2f(dequant_w16(d.Wq[(size_t)(n0 + lane) * K + kk[u]], swl))
                              : h2f(d.W_rows[(size_t)kk[u] * N + n0 + lane]);
            if (lane < M) xv[u] = (int)d.X[(size_t)lane * K + kk[u]];
          }
        }
#pragma unroll
        for (int u = 0; u < kDecOutBatch; ++u)
#pragma unroll
          for (int m = 0; m < 16; ++m)
            if (m < M) yo[m] += h2f((uint16_t)__builtin_amdgcn_readlane(xv[u], m)) * wv[u];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sYo[wave][lane][i] += v4f{yo[4 * i], yo[4 * i + 1], yo[4 * i + 2], yo[4 * i + 3]};
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) sYo[wave][lane][i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // ---- sum the partials of the 8 waves ------------------------------------------------
#pragma unroll
  for (int c = 0; c < kDecP; ++c) sRed[wave][c][lane] = acc[c];
  lds_sync();

  // ---- workspace intermediates of the further outlier columns (workgroup 0) --------
  if (blockIdx.x == 0 && wcount > kDecOutPre) {   // uniform
    int rank = 0;
    for (int w = 0; w < kc; ++w) rank += sCnt[w];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int u = 0; u < kDecOutDma; ++u) {
      if (kx[u] >= 0) {
        if (lane == 0) d.idx[rank + kDecOutPre + u] = kx[u];
        if (lane < M)
          d.X_O[(size_t)lane * K + rank + kDecOutPre + u] = (uint16_t)(sOx[wave][u][lane] & 0xffffu);
      }
    }
    for (int j0 = kDecOutPre + kDecOutDma; j0 < wcount; j0 += kDecOutBatch) {   // uniform, batched as above
      int kk[kDecOutBatch];
      uint16_t xv[kDecOutBatch];
#pragma unroll
      for (int u = 0; u < kDecOutBatch; ++u) {
        kk[u] = nth_outlier(j0 + u);
        xv[u] = kk[u] >= 0 && lane < M ? d.X[(size_t)lane * K + kk[u]] : (uint16_t)0;
      }
#pragma unroll
      for (int u = 0; u < kDecOutBatch; ++u) {
        if (kk[u] >= 0) {
          if (lane == 0) d.idx[rank + j0 + u] = kk[u];
          if (lane < M) d.X_O[(size_t)lane * K + rank + j0 + u] = xv[u];
        }
      }
    }
  }

  if (wave >= kDecP) return;
  const int c = wave;
  v4i tot = {0, 0, 0, 0};
  v4f yo4 = {0.0f, 0.0f, 0.0f, 0.0f};
  const int mb = g * 4;   // D rows of this lane: mb .. mb + 3
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    const v4i p = sRed[w][c][lane];
    tot[0] += p[0]; tot[1] += p[1]; tot[2] += p[2]; tot[3] += p[3];
    yo4 += sYo[w][c * 16 + lr][g];
  }

  // ---- epilogue ----------------------------------------------------------------------
  const int n = ne;
  if (n >= N || mb >= M) return;
  const float swn = swv * (ZP ? 1.0f / 127.0f : 1.0f / 16129.0f);
  if constexpr (ZP) {   // sum (q - zp) w = sum (q - 128) w + (128 - zp) S[n], mod 2^32
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (mb + r < M) tot[r] = (int)((uint32_t)tot[r] + (uint32_t)(128 - zpe[r]) * (uint32_t)wsn);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = mb + r;
    if (m < M) d.Y[(size_t)m * N + n] = f2h((float)tot[r] * (sxe[r] * swn) + yo4[r] + h2f(bvb));
  }
}

// Stream kernel for M <= 64 when the fused kernel does not apply (K > 4096 or
// M > 16): the activation kernels have written the codes, the row scales and
// the outlier list to the workspace.  MG row groups of 16 rows (the A operand
// of one MFMA each) against the same weight registers; KU k-steps per weight
// buffer (fewer for more row groups, to stay within the register file).
template <int MG, int KU>
__global__ __launch_bounds__(kDecThreads) void decode_stream_kernel(DecodeArgs d) {
  __shared__ v4i sRed[kDecWaves][MG][kDecP][64];
  __shared__ float sXO[kDecStreamRows][kDecMaxOutLds];

  const int M = d.M, K = d.K, N = d.N;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform
  const int lr = lane & 15, kl = (lane >> 4) * 16;
  const int n0 = blockIdx.x * kDecCols;
  const int nsteps = (K + 63) >> 6;
  const int kc = (wave + blockIdx.x) % kDecWaves;
  const int s0 = kc * nsteps / kDecWaves, s1 = (kc + 1) * nsteps / kDecWaves;

  // weight registers double-buffered: the loads of the next KU k-steps are in
  // flight while the current ones are multiplied; each buffer is filled one
  // 16-feature block after the other, the k-steps of a block back to back.
  // Steps past s1 read the zero page, so the loop needs no tail.
  v4i fb[2][KU][kDecP];
  auto load_b = [&](int b, int s) {
#pragma unroll
    for (int c = 0; c < kDecP; ++c) {
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int k = (s + u) * 64 + kl;
        const int n = n0 + c * 16 + lr;
        const bool in = s + u < s1 && n < N && k < K;
        const int8_t* p = in ? d.Wq + (size_t)n * K + k : g_dec_zero;
        fb[b][u][c] = *reinterpret_cast<const v4i*>(p);
      }
    }
  };
  // codes of rows 16 * g + lr, zero past M, K or s1
  auto load_a = [&](int s, v4i (&fa)[MG][KU]) {
#pragma unroll
    for (int g = 0; g < MG; ++g)
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int k = (s + u) * 64 + kl, row = 16 * g + lr;
        const bool in = s + u < s1 && row < M && k < K;
        const void* p = in ? (const void*)(d.Xq + (size_t)row * K + k) : (const void*)g_dec_zero;
        fa[g][u] = *reinterpret_cast<const v4i*>(p);
      }
  };
  v4i acc[MG][kDecP];
#pragma unroll
  for (int g = 0; g < MG; ++g)
#pragma unroll
    for (int c = 0; c < kDecP; ++c) acc[g][c] = v4i{0, 0, 0, 0};
  auto mma = [&](int b, const v4i (&fa)[MG][KU]) {
#pragma unroll
    for (int c = 0; c < kDecP; ++c)
#pragma unroll
      for (int u = 0; u < KU; ++u)
#pragma unroll
        for (int g = 0; g < MG; ++g)
          acc[g][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[g][u], fb[b][u][c], acc[g][c], 0, 0, 0);
  };
  // Epilogue operands: the outlier count and the first kDecOutReg indices
  // (scalars) now; the outlier weight values of this wave's epilogue features
  // and the first X_O values of the LDS copy are loaded right behind the last
  // weight loads, so that they land with them instead of one memory round
  // trip after the stream.
  // (The scalar loads go out after the first weight loads and are read
  // unconditionally, K >= kDecOutReg entries: no wait for the count holds up
  // the stream.)
  const int c = wave & (kDecP - 1);
  const int n = n0 + c * 16 + lr;
  int nout, nl, oidx[kDecOutReg];
  uint32_t wraw[kDecOutReg];   // fp16 weight value, or the code (W_rows NULL)
  uint32_t xraw = 0;           // X_O element t of the LDS copy (row t / nl, column t % nl)
  // row scales and zero points of this lane's epilogue rows (row groups
  // wave / 4 and wave / 4 + 2), the bias and the weight code sum of its feature
  constexpr int GE = (MG + 1) / 2;   // row groups per wave in the epilogue
  float sxr[GE][4];
  int zpr[GE][4];
  uint32_t braw = 0, wsraw = 0;
  auto load_epi = [&]() {
#pragma unroll
    for (int j = 0; j < kDecOutReg; ++j) {
      wraw[j] = 0;
      if (j < nout && n < N)
        wraw[j] = d.W_rows ? (uint32_t)d.W_rows[(size_t)oidx[j] * N + n]
                           : (uint32_t)(uint8_t)d.Wq[(size_t)n * K + oidx[j]];
    }
    if (t < nl * M) xraw = d.X_O[(size_t)(t / nl) * K + t % nl];
#pragma unroll
    for (int gi = 0; gi < GE; ++gi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * (wave / kDecP + 2 * gi) + (lane >> 4) * 4 + r;
        sxr[gi][r] = m < M ? d.sx[m] : 0.0f;
        zpr[gi][r] = d.zp && m < M ? d.zp[m] : 0;
      }
    if (n < N) {
      if (d.bias) braw = d.bias[n];
      if (d.zp) wsraw = (uint32_t)d.wsum[n];
    }
  };
  load_b(0, s0);
  __builtin_amdgcn_sched_barrier(0);
  nout = *d.n_out;
  nl = min(nout, kDecMaxOutLds);
#pragma unroll
  for (int j = 0; j < kDecOutReg; ++j) oidx[j] = d.idx[j];
  int s = s0;
  for (; s + 2 * KU < s1; s += 2 * KU) {
    v4i fa0[MG][KU], fa1[MG][KU];
    // the codes go out before the next weight loads: the wait for them then
    // leaves those loads in flight
    load_a(s, fa0);
    load_b(1, s + KU);
    __builtin_amdgcn_sched_barrier(0);
    mma(0, fa0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(s + KU, fa1);
    load_b(0, s + 2 * KU);
    __builtin_amdgcn_sched_barrier(0);
    mma(1, fa1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // The last round (always run; steps past s1 read the zero page and add 0)
  // issues no weight loads after it, and none at all for a second buffer
  // that lies wholly past s1.  Two straight-line variants (uniform branch), so
  // each keeps exact load counts for its waits.
  if (s + KU < s1) {
    v4i fa0[MG][KU], fa1[MG][KU];
    load_a(s, fa0);
    load_b(1, s + KU);
    __builtin_amdgcn_sched_barrier(0);
    mma(0, fa0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(s + KU, fa1);
    load_epi();
    __builtin_amdgcn_sched_barrier(0);
    mma(1, fa1);
    __builtin_amdgcn_sched_barrier(0);
  } else {
    v4i fa0[MG][KU];
    load_a(s, fa0);
    load_epi();
    __builtin_amdgcn_sched_barrier(0);
    mma(0, fa0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // every wave finishes features c * 16 + lr of its block (c = wave % 4), for
  // row groups wave / 4, wave / 4 + 2, ...
  // outlier weight value: the fp16 row, or rebuilt from the code (W_rows NULL)
  const float swn_raw = d.sw[n < N ? n : N - 1];
  auto wval = [&](int k) -> float {
    return d.W_rows ? h2f(d.W_rows[(size_t)k * N + n])
                    : h2f(dequant_w16(d.Wq[(size_t)n * K + k], swn_raw));
  };
  float wo[kDecOutReg];
#pragma unroll
  for (int j = 0; j < kDecOutReg; ++j)
    wo[j] = j < nout && n < N ? (d.W_rows ? h2f((uint16_t)wraw[j])
                                          : h2f(dequant_w16((int8_t)(uint8_t)wraw[j], swn_raw)))
                              : 0.0f;
  if (t < nl * M) sXO[t / nl][t % nl] = h2f((uint16_t)xraw);
  for (int e = t + kDecThreads; e < nl * M; e += kDecThreads) {   // beyond the first 512 (rare)
    const int m = e / nl, j = e % nl;
    sXO[m][j] = h2f(d.X_O[(size_t)m * K + j]);
  }
#pragma unroll
  for (int g = 0; g < MG; ++g)
#pragma unroll
    for (int cc = 0; cc < kDecP; ++cc) sRed[wave][g][cc][lane] = acc[g][cc];
  lds_sync();
  if (n >= N) return;
  const float swn = swn_raw * (d.zp ? 1.0f / 127.0f : 1.0f / 16129.0f);
  const float bv = d.bias ? h2f((uint16_t)braw) : 0.0f;
  const uint32_t wsv = wsraw;
#pragma unroll
  for (int gi = 0; gi < GE; ++gi) {   // row group g = wave / 4 + 2 gi (uniform per wave)
    const int g = wave / kDecP + 2 * gi;
    if (g >= MG) continue;
    const int mb = 16 * g + (lane >> 4) * 4;   // D rows of this lane: mb .. mb + 3
    if (mb >= M) continue;
    v4i tot = {0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const v4i p = sRed[w][g][c][lane];
      tot[0] += p[0]; tot[1] += p[1]; tot[2] += p[2]; tot[3] += p[3];
    }
    if (d.zp) {   // sum (q - zp) w = sum (q - 128) w + (128 - zp) S[n], mod 2^32
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (mb + r < M) tot[r] = (int)((uint32_t)tot[r] + (uint32_t)(128 - zpr[gi][r]) * wsv);
    }
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mb + r;
      y[r] = m < M ? (float)tot[r] * (sxr[gi][r] * swn) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kDecOutReg; ++j)
      if (j < nout) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (mb + r < M) y[r] += sXO[mb + r][j] * wo[j];
      }
    for (int j = kDecOutReg; j < nout; ++j) {
      const float w = wval(d.idx[j]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mb + r;
        if (m < M) y[r] += (j < kDecMaxOutLds ? sXO[m][j] : h2f(d.X_O[(size_t)m * K + j])) * w;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mb + r;
      if (m < M) d.Y[(size_t)m * N + n] = f2h(y[r] + bv);
    }
  }
}

namespace {

float half_bits_value(uint32_t b) {   // non-negative fp16 pattern (inf counts as 2^16)
  const int e = (int)((b >> 10) & 31), m = (int)(b & 1023);
  return e == 0 ? std::ldexp((float)m, -24) : std::ldexp((float)(m | 1024), e - 25);
}

// Smallest fp16 magnitude pattern whose value is >= t (t > 0): comparing the
// magnitude bits of an fp16 value with it is the same as |x| >= t.
uint32_t threshold_bits(float t) {
  uint32_t lo = 0, hi = 0x7c00;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) / 2;
    if (half_bits_value(mid) >= t) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

}  // namespace

typedef void (*kfn)(DecodeArgs);

namespace {
// Stream kernel instantiation for M <= 64: row groups of 16 rows.
kfn stream_kernel(int M) {
  if (M <= 16) return decode_stream_kernel<1, 4>;
  if (M <= 32) return decode_stream_kernel<2, 4>;
  return decode_stream_kernel<4, 2>;
}

// Fused kernel instantiation for M <= 16, K <= 4096.
template <bool ZP>
kfn fused_decode_kernel(int M, int K) {
  const int steps = ((K + 63) / 64 + kDecWaves - 1) / kDecWaves;   // k-steps per wave
  const int ks = steps <= 1 ? 1 : steps <= 2 ? 2 : steps <= 4 ? 4 : 8;
  int r = 1;   // k-steps packed per register set: M <= 16 / r, r <= ks
  while (r < ks && M <= 16 / (2 * r)) r *= 2;
  kfn f = nullptr;
#define I8L_DEC(KS_, R_) if (ks == KS_ && r == R_) f = decode_kernel<KS_, R_, 8, ZP>;
  I8L_DEC(1, 1) I8L_DEC(2, 1) I8L_DEC(2, 2) I8L_DEC(4, 1) I8L_DEC(4, 2) I8L_DEC(4, 4)
  I8L_DEC(8, 1) I8L_DEC(8, 2) I8L_DEC(8, 4) I8L_DEC(8, 8)
#undef I8L_DEC
  return f;
}
}  // namespace

hipError_t launch_decode(const uint16_t* X, int M, int K, const int8_t* Wq, const float* sw,
                         int N, const uint16_t* W_rows, const uint16_t* bias, float threshold,
                         bool enabled, uint16_t* Y, const Workspace& ws, hipStream_t stream) {
  const uint32_t thr = enabled ? threshold_bits(threshold) : 0x10000u;
  DecodeArgs d{X, M, K, N, Wq, sw, W_rows, bias, thr, Y, ws.n_out, ws.idx, ws.sx, ws.Xq, ws.X_O};
  const dim3 grid((N + kDecCols - 1) / kDecCols), block(kDecThreads);
  if (decode_fits(M, K)) {
    hipLaunchKernelGGL(fused_decode_kernel<false>(M, K), grid, block, 0, stream, d);
    return hipGetLastError();
  }
  hipError_t e = launch_quantize_activation(X, M, K, threshold, enabled, ws, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stream_kernel(M), grid, block, 0, stream, d);
  return hipGetLastError();
}

hipError_t launch_decode_zp(const uint16_t* X, int M, int K, const int8_t* Wq, const float* sw,
                            const int32_t* wsum, int N, const uint16_t* W_rows,
                            const uint16_t* bias, float threshold, bool enabled, uint16_t* Y,
                            const Workspace& ws, hipStream_t stream) {
  const uint32_t thr = enabled ? threshold_bits(threshold) : 0x10000u;
  DecodeArgs d{X, M, K, N, Wq, sw, W_rows, bias, thr, Y, ws.n_out, ws.idx, ws.sx, ws.Xq, ws.X_O,
               ws.zp, wsum};
  const dim3 grid((N + kDecCols - 1) / kDecCols), block(kDecThreads);
  if (decode_fits(M, K)) {
    hipLaunchKernelGGL(fused_decode_kernel<true>(M, K), grid, block, 0, stream, d);
    return hipGetLastError();
  }
  hipError_t e = launch_quantize_activation(X, M, K, threshold, enabled, ws, stream, true);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stream_kernel(M), grid, block, 0, stream, d);
  return hipGetLastError();
}

}  // namespace i8l
