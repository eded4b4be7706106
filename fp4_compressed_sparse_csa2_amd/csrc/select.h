// Block-level pieces of the deterministic Top-K: radix-digit search over a
// 2048-bin histogram and the in-order emission of the selected ids.
//
// Ranking is score descending, position ascending (ties go to the lower
// position).  Scores are biased to 22-bit unsigned keys (score_key), so two
// 11-bit digits fix the K-th largest key tau exactly; every key above tau is
// selected, and of the keys equal to tau the ones with the lowest ids fill
// the remaining slots.  Candidates are kept in ascending id order from the
// start, so the emission is one stable compaction: no sort, no bitmap.
#pragma once

#include "common.h"

namespace csa2 {

// The 8 histogram bins thread i scans, top first: h[k] = hist[2047 - 8i - k].
struct DigitBins {
  int h[8];
};

template <typename HistT>
__device__ __forceinline__ DigitBins load_digit_bins(const HistT* hist) {
  DigitBins d;
  const int top = kBins - 8 * (int)threadIdx.x;
#pragma unroll
  for (int k = 0; k < 8; ++k) d.h[k] = (int)hist[top - 1 - k];
  return d;
}

// Same from a 16-byte aligned global histogram with two 16-byte loads.
__device__ __forceinline__ DigitBins load_digit_bins_vec(const uint32_t* hist) {
  const uint4* p = reinterpret_cast<const uint4*>(hist + kBins - 8 * (int)threadIdx.x - 8);
  const uint4 lo = p[0], hi = p[1];
  DigitBins d;
  d.h[0] = (int)hi.w; d.h[1] = (int)hi.z; d.h[2] = (int)hi.y; d.h[3] = (int)hi.x;
  d.h[4] = (int)lo.w; d.h[5] = (int)lo.z; d.h[6] = (int)lo.y; d.h[7] = (int)lo.x;
  return d;
}

// Largest digit t with sum_{bin >= t} hist[bin] >= need (need >= 1), and the
// count strictly above it, from the bins each thread holds.  All threads must
// call; results land in *t_out / *above_out (shared) and are visible to every
// thread on return.  If the histogram holds fewer than `need` entries,
// *t_out = -1.
__device__ inline void find_digit_in(const DigitBins& d, int need, int* scan_scratch, int* t_out,
                                     int* above_out) {
  const int top = kBins - 8 * (int)threadIdx.x;
  int s = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += d.h[k];
  if (threadIdx.x == 0) *t_out = -1;
  int total;
  const int excl = block_exclusive_scan(s, scan_scratch, &total);
  if (excl < need && need <= excl + s) {
    int run = excl;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (run + d.h[k] >= need) {
        *t_out = top - 1 - k;
        *above_out = run;
        break;
      }
      run += d.h[k];
    }
  }
  __syncthreads();
}

template <typename HistT>
__device__ void find_digit(const HistT* hist, int need, int* scan_scratch, int* t_out,
                           int* above_out) {
  find_digit_in(load_digit_bins(hist), need, scan_scratch, t_out, above_out);
}

constexpr int kEmitPerThread = 8;   // entries per thread per round of the emission

// Emit the selection from candidates that arrive in ascending id order.
//   get(f) -> uint2{key, id} for f < total, ids strictly ascending in f.
//   key > tau: selected; key == tau: the first `need_ties` of them (lowest
//   ids) are selected; key < tau: dropped.
// Writes out[j] = id of the j-th selected entry (ascending ids) for j < K and
// returns the number selected (uniform).  `scan_scratch`: 4 shared ints.
// All threads must call.
template <typename Get>
__device__ int emit_in_order(Get get, int total, uint32_t tau, int need_ties, int32_t* out,
                             int K, int* scan_scratch) {
  constexpr int E = kEmitPerThread;
  int carry_gt = 0, carry_tie = 0;
  for (int base = 0; base < total; base += kBlock * E) {
    const int f0 = base + (int)threadIdx.x * E;
    uint2 c[E];
    int n_gt = 0, n_tie = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      c[e] = (f0 + e < total) ? get(f0 + e) : make_uint2(0u, 0u);
      const bool live = f0 + e < total;
      n_gt += (live && c[e].x > tau) ? 1 : 0;
      n_tie += (live && c[e].x == tau) ? 1 : 0;
    }
    // one scan carries both counts: per round each is <= 256 * E < 2^16
    int round_total;
    const int pre = block_exclusive_scan(n_gt | (n_tie << 16), scan_scratch, &round_total);
    int g = carry_gt + (pre & 0xFFFF), t = carry_tie + (pre >> 16);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (f0 + e >= total) break;
      if (c[e].x > tau) {
        const int slot = g + (t < need_ties ? t : need_ties);
        if (slot < K) out[slot] = (int32_t)c[e].y;
        ++g;
      } else if (c[e].x == tau) {
        if (t < need_ties && g + t < K) out[g + t] = (int32_t)c[e].y;
        ++t;
      }
    }
    carry_gt += round_total & 0xFFFF;
    carry_tie += round_total >> 16;
  }
  const int n = carry_gt + (carry_tie < need_ties ? carry_tie : need_ties);
  return n < K ? n : K;
}

}  // namespace csa2
