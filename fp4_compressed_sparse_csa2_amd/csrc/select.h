// Block-level pieces of the deterministic Top-K: radix-digit search over a
// 2048-bin histogram and bitmap-ordered emission of the selected ids.
//
// Ranking is score descending, position ascending (ties go to the lower
// position).  Scores are biased to 22-bit unsigned keys (key = score + 2^21),
// so two 11-bit digits fix the K-th largest key tau exactly; every key above
// tau is selected, and of the keys equal to tau the lowest ids fill the
// remaining slots.  Ids are emitted in ascending order by walking a bitmap,
// which also makes the output independent of the order candidates arrived in.
#pragma once

#include "common.h"

namespace csa2 {

// Largest digit t with sum_{bin >= t} hist[bin] >= need (need >= 1), and the
// count strictly above it.  Thread i reads bins [2048-8(i+1), 2048-8i), top
// first.  All threads must call; results land in *t_out / *above_out (shared)
// and are visible to every thread on return.  If the histogram holds fewer
// than `need` entries, *t_out = -1.
template <typename HistT>
__device__ void find_digit(const HistT* hist, int need, int* scan_scratch, int* t_out,
                           int* above_out) {
  const int top = kBins - 8 * (int)threadIdx.x;
  int h[8];
  int s = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    h[k] = (int)hist[top - 1 - k];
    s += h[k];
  }
  if (threadIdx.x == 0) *t_out = -1;
  int total;
  const int excl = block_exclusive_scan(s, scan_scratch, &total);
  if (excl < need && need <= excl + s) {
    int run = excl;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (run + h[k] >= need) {
        *t_out = top - 1 - k;
        *above_out = run;
        break;
      }
      run += h[k];
    }
  }
  __syncthreads();
}

constexpr int kSegWords = 2048;                 // bitmap words per segment
constexpr int kSegIds = kSegWords * 32;         // 65536 ids per segment

// Emit the selected ids in ascending order.
//   get(i) -> uint2{key, id} for candidate i < n_cand (ids < id_end, distinct)
//   key > tau: selected; key == tau: tie, the first `need_ties` ties by
//   ascending id are selected; key < tau: dropped.
//   put(j, id): write output slot j.
// Returns the number written (uniform).  `sel`/`tie` are shared bitmaps of
// kSegWords words each; `scan_scratch` 4 shared ints.  All threads must call.
template <typename Get, typename Put>
__device__ int emit_selected(Get get, int n_cand, uint32_t tau, int need_ties, int id_end,
                             uint32_t* sel, uint32_t* tie, int* scan_scratch, Put put) {
  constexpr int WPT = kSegWords / kBlock;       // words per thread
  int out_run = 0, tie_run = 0;
  for (int seg0 = 0; seg0 < id_end; seg0 += kSegIds) {
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      sel[threadIdx.x * WPT + k] = 0u;
      tie[threadIdx.x * WPT + k] = 0u;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n_cand; i += kBlock) {
      const uint2 c = get(i);
      const int rel = (int)c.y - seg0;
      if (rel < 0 || rel >= kSegIds || c.x < tau) continue;
      uint32_t* bits = c.x > tau ? sel : tie;
      atomicOr(&bits[rel >> 5], 1u << (rel & 31));
    }
    __syncthreads();
    uint32_t s_w[WPT], t_w[WPT];
    int nt = 0;
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      s_w[k] = sel[threadIdx.x * WPT + k];
      t_w[k] = tie[threadIdx.x * WPT + k];
      nt += __popc(t_w[k]);
    }
    int tie_total;
    int rank = tie_run + block_exclusive_scan(nt, scan_scratch, &tie_total);
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      uint32_t t = t_w[k];
      while (t != 0u) {
        const uint32_t bit = t & (0u - t);
        if (rank < need_ties) s_w[k] |= bit;
        ++rank;
        t ^= bit;
      }
    }
    tie_run += tie_total;
    int ns = 0;
#pragma unroll
    for (int k = 0; k < WPT; ++k) ns += __popc(s_w[k]);
    int sel_total;
    int slot = out_run + block_exclusive_scan(ns, scan_scratch, &sel_total);
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      uint32_t s = s_w[k];
      while (s != 0u) {
        const int bit = __ffs(s) - 1;
        put(slot++, seg0 + (int)(threadIdx.x * WPT + k) * 32 + bit);
        s &= s - 1u;
      }
    }
    out_run += sel_total;
  }
  return out_run;
}

}  // namespace csa2
