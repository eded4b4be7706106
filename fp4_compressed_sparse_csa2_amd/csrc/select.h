// Block-level pieces of the deterministic Top-K: radix-digit search over a
// 2048-bin histogram and the in-order emission of the selected ids.
//
// Ranking is score descending, position ascending (ties go to the lower
// position).  Scores are biased to 22-bit unsigned keys (score_key), so two
// 11-bit digits fix the K-th largest key tau exactly (float32 values of a
// scaled indexer take 32-bit order keys and a third, 10-bit digit); every
// key above tau is selected, and of the keys equal to tau the ones with the
// lowest ids fill the remaining slots.  Candidates are kept in ascending id
// order from the start, so the emission is one stable compaction: no sort,
// no bitmap.
#pragma once

#include "common.h"

namespace csa2 {

// Per-sequence control words of a selection (uint32): the top-digit histogram
// the scoring kernel fills, as kHistReps replicas of kBins words that sum to
// it (score block i adds into replica i % kHistReps, which spreads the
// atomics on the busiest bins over two addresses), the low-digit histogram
// of the entries whose top digit is the threshold's (kBins words, filled by
// the multi-block filter), the top digit and the count above it as the
// filter found them (two words), then spare words.  Sequence b's words sit
// at b * kCtrlWords from the start of the workspace whatever the call's
// sizes, and every call returns them to zero; the scratch that follows them
// starts after batch * kCtrlWords words, so a workspace handed to a call
// with another batch must be zeroed again first.
constexpr int kHistReps = 2;
constexpr int kCtrlHist2 = kHistReps * kBins;
constexpr int kCtrlTop = kCtrlHist2 + kBins;
constexpr int kCtrlWords = kCtrlTop + 64;
static_assert(kCtrlWords % 4 == 0, "control words are cleared 16 bytes at a time");
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

// REPS > 1: the histogram is the sum of REPS replicas kBins words apart.
template <int NT = kBlock, int REPS = 1, typename HistT>
__device__ __forceinline__ DigitBins<NT> load_digit_bins(const HistT* hist) {
  DigitBins<NT> d;
  const int top = kBins - DigitBins<NT>::BPT * (int)threadIdx.x;
#pragma unroll
  for (int k = 0; k < DigitBins<NT>::BPT; ++k) d.h[k] = (int)hist[top - 1 - k];
#pragma unroll
  for (int r = 1; r < REPS; ++r) {
#pragma unroll
    for (int k = 0; k < DigitBins<NT>::BPT; ++k) d.h[k] += (int)hist[r * kBins + top - 1 - k];
  }
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
  if (threadIdx.x == 0) {
    *t_out = -1;
    *above_out = 0;
  }
  int total;
  // (scan_scratch is next written after the closing barrier below)
  const int excl = block_exclusive_scan<NT, false>(s, scan_scratch, &total);
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

// The int32 score of a biased key (score_key's inverse; the folded top key
// is the one score 2^21).
__device__ __forceinline__ int32_t key_score(uint32_t key) {
  return key == 0x3FFFFFu ? (1 << 21) : (int32_t)key - kKeyBias;
}

// How the 32-bit words of a score row map to radix keys.
//   IntKeys   - int32 indexer scores; 22-bit biased keys (score_key), two
//               11-bit digits.
//   FloatKeys - the words are already order keys of float32 values
//               (value_key); three digits of 11, 11 and 10 bits.
// top(k) is the digit of the scoring kernels' histogram, mid(k) the digit of
// the second histogram, low(k) the third digit (FloatKeys only).
// out_word(k) is what a selection reports for the entry: the int32 score, or
// the bits of the float32 value.
struct IntKeys {
  static constexpr bool kThree = false;
  static constexpr int kTopShift = 11;
  __device__ static uint32_t key(int32_t w) { return score_key(w); }
  __device__ static uint32_t mid(uint32_t k) { return k & (kBins - 1); }
  __device__ static uint32_t low(uint32_t) { return 0u; }
  __device__ static int32_t out_word(uint32_t k) { return key_score(k); }
  __device__ static int32_t stored_out(int32_t w) { return w; }
};
struct FloatKeys {
  static constexpr bool kThree = true;
  static constexpr int kTopShift = 21;
  static constexpr int kLowBits = 10;
  __device__ static uint32_t key(int32_t w) { return (uint32_t)w; }
  __device__ static uint32_t mid(uint32_t k) { return (k >> kLowBits) & (kBins - 1); }
  __device__ static uint32_t low(uint32_t k) { return k & ((1u << kLowBits) - 1u); }
  __device__ static int32_t out_word(uint32_t k) { return (int32_t)__float_as_uint(key_value(k)); }
  __device__ static int32_t stored_out(int32_t w) { return out_word((uint32_t)w); }
};

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Emit the selection from candidates that arrive in ascending id order.
//   get(f) -> uint2{key, id} for f < total, ids strictly ascending in f.
//   key > tau: selected; key == tau: the first `need_ties` of them (lowest
//   ids) are selected; key < tau: dropped.
// Calls put(j, c) for the j-th selected entry c = {key, id} (ascending ids),
// j < K, and
// returns the number selected (uniform).  Each wave takes one contiguous run
// of candidates, counts its selections with ballots, and after one barrier
// (the per-wave totals, `wave_tot`: NT/64 shared int2) places them with
// in-wave prefix counts.  All threads must call, once per kernel.
template <int NT, typename Get, typename Put>
__device__ int emit_in_order(Get get, int total, uint32_t tau, int need_ties, int K,
                             int2* wave_tot, Put put) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int run = ((total + NT - 1) / NT) * 64;          // a multiple of 64 per wave
  const int f0 = wave * run;
  const int f1 = min(f0 + run, total);
  int g = 0, t = 0;
  for (int f = f0 + lane; f - lane < f1; f += 64) {      // wave-uniform trip count
    const bool live = f < f1;
    const uint32_t key = live ? get(f).x : 0u;
    g += __popcll(__ballot(live && key > tau));
    t += __popcll(__ballot(live && key == tau));
  }
  if (lane == 0) wave_tot[wave] = make_int2(g, t);
  __syncthreads();
  const int4 bt = waves_before_and_total2<NT>(wave_tot);
  int g0 = bt.x, t0 = bt.y;
  const int G = bt.z, T = bt.w;
  for (int f = f0 + lane; f - lane < f1; f += 64) {
    const bool live = f < f1;
    const uint2 c = live ? get(f) : make_uint2(0u, 0u);
    const bool gt = live && c.x > tau, tie = live && c.x == tau;
    const uint64_t bg = __ballot(gt), bt = __ballot(tie);
    const int gb = g0 + lanes_below(bg), tb = t0 + lanes_below(bt);   // before this entry
    if (gt) {
      const int slot = gb + (tb < need_ties ? tb : need_ties);
      if (slot < K) put(slot, c);
    } else if (tie) {
      if (tb < need_ties && gb + tb < K) put(gb + tb, c);
    }
    g0 += __popcll(bg);
    t0 += __popcll(bt);
  }
  const int ties = T < need_ties ? T : need_ties;
  const int n = G + (ties > 0 ? ties : 0);
  return n < K ? n : K;
}

}  // namespace csa2
