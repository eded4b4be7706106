// Device helpers shared by the CSA2 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kPage = 64;      // token positions per page
constexpr int kWindow = 128;   // sliding-window tokens per layer
constexpr int kGroup = 16;     // channels per E4M3 scale
constexpr int kBlock = 256;    // threads per block for every kernel here
constexpr int kKeyBias = 1 << 21;  // int8 scores at Di <= 128 lie in [-2^21 + 2^14, 2^21]
constexpr int kBins = 2048;    // radix digit = 11 bits; two digits cover the 22-bit key

// Byte layout of one page: 64 rows of R = D/2 + D/16 bytes (a row is its
// E2M1 codes, D/2 bytes, then its E4M3 scales, D/16 bytes, so one token's
// FP4 row is one contiguous run), then the 64 int8 key rows of Di bytes.
struct PageLayout {
  int row_bytes;      // R
  int keys_off;       // 64 * R
  int page_bytes;     // 64 * (R + Di)
};
__host__ __device__ constexpr PageLayout page_layout(int D, int Di) {
  return PageLayout{D / 2 + D / 16, kPage * (D / 2 + D / 16), kPage * (D / 2 + D / 16 + Di)};
}

// Radix key of an indexer score: score + 2^21 as a 22-bit unsigned number.
// The one score that reaches 2^21 is (-128)(-128)*128, and no int8 score lies
// strictly between 2^21 - 128 and 2^21, so folding it onto 2^22 - 1 keeps the
// order of every pair of distinct scores and every histogram bin below 2048.
__device__ __forceinline__ uint32_t score_key(int s) {
  const uint32_t k = (uint32_t)(s + kKeyBias);
  return k > 0x3FFFFFu ? 0x3FFFFFu : k;
}

// Scaled indexer value of one position: fl32(s * score), the product rounded
// once to float32 (round to nearest even).  An int8 score at Di <= 128 is
// exact in float32 (|score| <= 2^21), so the conversion adds no rounding.
// -0 becomes +0, so that the two zeros are one value (a tie).
__device__ __forceinline__ float scaled_value(int score, float s) {
  const float v = __fmul_rn((float)score, s);
  return v == 0.0f ? 0.0f : v;
}

// Order key of a float32 value: keys compare (unsigned) as the values do,
// -inf below every finite value below +inf.  Negative values flip every bit,
// the others set the sign bit.  The caller passes +0 for a zero.
__device__ __forceinline__ uint32_t value_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ lanes
__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Sum over aligned groups of 4 lanes (quad_perm swaps) and of 8 lanes
// (row_half_mirror: lane i of each 8-lane half-row reads lane 7-i, which sits
// in the other quad).
__device__ __forceinline__ int sum_quad(int v) {
  v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  return v;
}
__device__ __forceinline__ int sum_oct(int v) {
  v = sum_quad(v);
  v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave, all in DPP moves (no LDS
// round trip): shifts by 1, 2, 4 and 8 lanes inside each 16-lane row; then
// lane 15 of rows 0 and 2 is added to rows 1 and 3 (row_bcast:15), and lane
// 31, the total of rows 0-1, to rows 2 and 3 (row_bcast:31).  A lane whose
// source lies outside its row, or whose row is masked off, adds 0.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return x;
}

// Inclusive running maximum over the 64 lanes of a wave of values >= 0 (the
// same DPP steps as wave_inclusive_scan; a lane with no source keeps its own
// value); lane 63 holds the wave's maximum.
__device__ __forceinline__ int wave_inclusive_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false));   // row_shr:1
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false));   // row_shr:2
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false));   // row_shr:4
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false));   // row_shr:8
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false));   // row_bcast:15
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return x;
}

// Given the NT/64 wave totals in `scratch` (after a barrier): the sum of the
// totals of the waves before the calling one, and of all of them, both
// wave-uniform.  Lane w < NT/64 reads total w; one wave scan and two lane
// reads replace a per-wave loop over the totals.
template <int NT>
__device__ __forceinline__ int2 waves_before_and_total(const int* scratch) {
  constexpr int NW = NT / 64;
  static_assert(NW <= 64, "one total per lane");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int x = wave_inclusive_scan(lane < NW ? scratch[lane] : 0);
  const int before = wave == 0 ? 0 : __builtin_amdgcn_readlane(x, wave - 1);
  return make_int2(before, __builtin_amdgcn_readlane(x, NW - 1));
}

// The same for two totals per wave (`tot`: NT/64 int2 after a barrier):
// {before.x, before.y, total.x, total.y}, wave-uniform.
template <int NT>
__device__ __forceinline__ int4 waves_before_and_total2(const int2* tot) {
  constexpr int NW = NT / 64;
  static_assert(NW <= 64, "one total per lane");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int2 v = lane < NW ? tot[lane] : make_int2(0, 0);
  const int x = wave_inclusive_scan(v.x), y = wave_inclusive_scan(v.y);
  const int bx = wave == 0 ? 0 : __builtin_amdgcn_readlane(x, wave - 1);
  const int by = wave == 0 ? 0 : __builtin_amdgcn_readlane(y, wave - 1);
  return make_int4(bx, by, __builtin_amdgcn_readlane(x, NW - 1),
                   __builtin_amdgcn_readlane(y, NW - 1));
}

// Exclusive prefix sum over an NT-thread block; returns the prefix, sets *total.
// `scratch` must hold NT/64 ints of shared memory.  Contains barriers: every
// thread of the block must call it.  SYNC_AFTER = false leaves out the
// closing barrier: the caller then passes a barrier before `scratch` is
// written again.
template <int NT = kBlock, bool SYNC_AFTER = true>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  const int2 bt = waves_before_and_total<NT>(scratch);
  if constexpr (SYNC_AFTER) __syncthreads();
  *total = bt.y;
  return bt.x + x - v;
}

// ------------------------------------------------------------------ FP8 / FP4
// Value of an E4M3 (OCP "FN") byte with the sign bit clear, as float (exact).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e == 0 ? (float)m * (1.0f / 512.0f) : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Value of any E4M3 (FN) byte: the sign applied, NaN for S.1111.111.
__device__ __forceinline__ float e4m3_signed_value(uint32_t b) {
  const float v = (b & 0x7Fu) == 0x7Fu ? __builtin_nanf("") : e4m3_value(b & 0x7Fu);
  return (b & 0x80u) ? -v : v;
}

// E4M3 code of q >= 0: nearest value, ties to the even code, saturating at
// 448 (0x7E).  q = amax/6 is never within a few ulps of an E4M3 midpoint
// unless it equals it (amax has 8 significant bits, 6*midpoint at most 8), so
// rounding q from the fp32 quotient is exact.
__device__ __forceinline__ uint32_t e4m3_code(float q) {
  if (!(q < 448.0f)) return 0x7Eu;
  if (q < 0.015625f) {                               // subnormal grid m * 2^-9, m = 0..8
    return (uint32_t)__builtin_rintf(q * 512.0f);    // exact scaling, RNE; 8 = 0x08 = 2^-6
  }
  uint32_t u = __float_as_uint(q);
  uint32_t e = ((u >> 23) & 0xFFu) - 120u;          // E4M3 exponent field (1..15)
  uint32_t mant = u & 0x7FFFFFu;
  uint32_t m3 = mant >> 20, rem = mant & 0xFFFFFu;
  uint32_t code = (e << 3) | m3;
  code += (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ? 1u : 0u;
  return code > 0x7Eu ? 0x7Eu : code;
}

// E2M1 magnitude code of |x| = xa on the grid {0,.5,1,1.5,2,3,4,6} * s,
// nearest with ties to the even code.  Midpoint k (between codes k and k+1)
// sends a tie up when k+1 is even.  All midpoints * s are exact in fp32.
__device__ __forceinline__ uint32_t e2m1_mag_code(float xa, float s) {
  uint32_t c = 0;
  c += xa > 0.25f * s;
  c += xa >= 0.75f * s;
  c += xa > 1.25f * s;
  c += xa >= 1.75f * s;
  c += xa > 2.5f * s;
  c += xa >= 3.5f * s;
  c += xa > 5.0f * s;
  return s > 0.0f ? c : 0u;
}

}  // namespace csa2
