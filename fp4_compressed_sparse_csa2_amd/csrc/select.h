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

// Per-sequence control words of a selection (uint32): the top-digit histogram
// the scoring kernel fills, then spare words.  The size does not depend on the
// call's sizes, so a zeroed workspace stays zeroed between calls of any shape.
constexpr int kCtrlWords = kBins + 64;
constexpr int kMaxSelChunks = 4096;      // 4096-entry filter chunks of a 2^24-entry sequence
constexpr int kSingleMax = 1 << 14;      // longest sequence for the one-block selection

// Row stride (in entries) of score and candidate arrays: a multiple of 64 so
// that every row starts 256-byte aligned.
__host__ __device__ inline int row_stride(int n) { return (n + 63) & ~63; }

// The bins thread i of an NT-thread block scans, top first:
// h[k] = hist[2047 - BPT*i - k], BPT = 2048 / NT.
template <int NT>
struct DigitBins {
  static constexpr int BPT = kBins / NT;
  int h[BPT];
};

template <int NT = kBlock, typename HistT>
__device__ __forceinline__ DigitBins<NT> load_digit_bins(const HistT* hist) {
  DigitBins<NT> d;
  const int top = kBins - DigitBins<NT>::BPT * (int)threadIdx.x;
#pragma unroll
  for (int k = 0; k < DigitBins<NT>::BPT; ++k) d.h[k] = (int)hist[top - 1 - k];
  return d;
}

// Largest digit t with sum_{bin >= t} hist[bin] >= need (need >= 1), and the
// count strictly above it, from the bins each thread holds.  All threads must
// call; results land in *t_out / *above_out (shared) and are visible to every
// thread on return.  If the histogram holds fewer than `need` entries,
// *t_out = -1.  `scan_scratch`: NT/64 shared ints.
template <int NT = kBlock>
__device__ inline void find_digit_in(const DigitBins<NT>& d, int need, int* scan_scratch,
                                     int* t_out, int* above_out) {
  constexpr int BPT = DigitBins<NT>::BPT;
  const int top = kBins - BPT * (int)threadIdx.x;
  int s = 0;
#pragma unroll
  for (int k = 0; k < BPT; ++k) s += d.h[k];
  if (threadIdx.x == 0) *t_out = -1;
  int total;
  const int excl = block_exclusive_scan<NT>(s, scan_scratch, &total);
  if (excl < need && need <= excl + s) {
    int run = excl;
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
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

template <int NT = kBlock, typename HistT>
__device__ void find_digit(const HistT* hist, int need, int* scan_scratch, int* t_out,
                           int* above_out) {
  find_digit_in<NT>(load_digit_bins<NT>(hist), need, scan_scratch, t_out, above_out);
}

constexpr int kEmitPerThread = 8;   // entries per thread per round of the emission

// Emit the selection from candidates that arrive in ascending id order.
//   get(f) -> uint2{key, id} for f < total, ids strictly ascending in f.
//   key > tau: selected; key == tau: the first `need_ties` of them (lowest
//   ids) are selected; key < tau: dropped.
// Calls put(j, id) for the j-th selected entry (ascending ids), j < K, and
// returns the number selected (uniform).  `scan_scratch`: NT/64 shared ints.
// All threads must call.
template <int NT = kBlock, typename Get, typename Put>
__device__ int emit_in_order(Get get, int total, uint32_t tau, int need_ties, int K,
                             int* scan_scratch, Put put) {
  constexpr int E = kEmitPerThread;
  int carry_gt = 0, carry_tie = 0;
  for (int base = 0; base < total; base += NT * E) {
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
    // one scan carries both counts: per round each is <= NT * E < 2^16
    int round_total;
    const int pre = block_exclusive_scan<NT>(n_gt | (n_tie << 16), scan_scratch, &round_total);
    int g = carry_gt + (pre & 0xFFFF), t = carry_tie + (pre >> 16);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (f0 + e >= total) break;
      if (c[e].x > tau) {
        const int slot = g + (t < need_ties ? t : need_ties);
        if (slot < K) put(slot, c[e].y);
        ++g;
      } else if (c[e].x == tau) {
        if (t < need_ties && g + t < K) put(g + t, c[e].y);
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
