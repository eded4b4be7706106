// Deterministic Top-K over int32 indexer scores: the selection kernels shared
// by csa2_index_topk (the Full layer's candidates 0 <= p < L - 128) and
// csa2_reindex (the entries of the Full layer's pool).
//
// The Full layer makes the sparse selection whose Top-K addressing indices
// later layers reuse, and deeper indexer layers refilter only the pool the
// Full layer built (neodrop.ai V4.1-Flash report, 架构拆解 item 2; zulogic
// "DeepSeek V4 1-Flash 架构拆解", section 3).  Order: score descending,
// position ascending.
//
// Input: the scores and, per sequence, a 2048-bin histogram of the top 11
// bits of the biased 22-bit key (built by the scoring kernel).  Two plans, no
// cross-block synchronisation inside a kernel (visibility comes from kernel
// boundaries):
//   single  - up to kSingleMax entries: one block per sequence finds the
//             K-th largest top digit t1, reads the scores once (every load of
//             a 32K-entry round in flight together) keeping the entries with
//             digit >= t1 in entry order (one block scan per round) and
//             histogramming the low digit of those equal to t1, fixes the
//             exact threshold and emits in order.
//   filter  - longer sequences: 4096-entry blocks keep their digit >= t1
//   + final   entries, in order, in their own slots; then one block per
//             sequence concatenates the slot lists (already in order),
//             histograms the low digit, fixes the threshold and emits.
// Both return the sequence's histogram to zero for the next call.
#include "common.h"
#include "launch.h"
#include "select.h"

namespace csa2 {

constexpr int kSelNT = 512;                      // threads of the one-block-per-sequence kernels
constexpr int kSelPT = 64;                       // entries per thread per round
constexpr int kSelRound = kSelNT * kSelPT;       // 32768 entries (128 KB) per round
constexpr int kListCap = 6144;                   // candidates the final kernel keeps in LDS
constexpr int kSingleListCap = 2944;             // candidates the single kernel keeps in LDS
constexpr int kFiltPer = 16;                     // entries per thread in the filter kernel
constexpr int kFiltChunk = kBlock * kFiltPer;    // 4096 entries per filter block

// Number of entries of sequence b.
__device__ __forceinline__ int sel_entries(const SelectArgs& a, int b) {
  if (a.pool_count != nullptr) {
    const int c = a.pool_count[b];
    return c < 0 ? 0 : (c > a.P ? a.P : c);
  }
  int L = a.ctx_len[b];
  L = L < 0 ? 0 : L;
  L = L > a.max_ctx ? a.max_ctx : L;
  L = L > a.max_pages * kPage ? a.max_pages * kPage : L;
  return L > kWindow ? L - kWindow : 0;
}

// Output id of entry i: the position itself, or the pool's position.
__device__ __forceinline__ int32_t sel_id(const SelectArgs& a, int b, uint32_t i) {
  return a.pool != nullptr ? a.pool[(size_t)b * a.P + i] : (int32_t)i;
}

// K = 0 or every entry selected: the first min(K, n) entries in order, then -1.
__device__ __forceinline__ void select_all(const SelectArgs& a, int b, int n, int nt) {
  int32_t* out = a.out_idx + (size_t)b * a.K;
  for (int i = threadIdx.x; i < a.K; i += nt) out[i] = i < n ? sel_id(a, b, (uint32_t)i) : -1;
  if (threadIdx.x == 0) a.out_count[b] = n < a.K ? n : a.K;
}

// ------------------------------------------------------------------ single
// Thread t takes the 64 entries at r * 32768 + 64t of round r; every load of
// a round (and, for the first, the histogram) is issued before any result is
// used, so each 32768-entry round costs one memory round trip.
// The streaming passes touch LDS only to write the (rare) kept entries; the
// low-digit histogram is built afterwards from the kept list.
__global__ __launch_bounds__(kSelNT) void select_single_kernel(SelectArgs a) {
  __shared__ uint32_t hist2[kBins];
  __shared__ uint2 list[kSingleListCap];
  __shared__ int scan_scratch[kSelNT / 64];
  __shared__ int sh_t1, sh_above1, sh_t2, sh_above2;

  const int b = blockIdx.x;
  const int n = sel_entries(a, b);
  const int K = a.K;
  if (K == 0 || n <= K) {
    select_all(a, b, n, kSelNT);
    return;
  }
  const int tid = threadIdx.x;
  uint32_t* h1 = a.hist1 + (size_t)b * kCtrlWords;
  const int32_t* row = a.scores + (size_t)b * a.stride;
  uint2* ovf = a.cand + (size_t)b * a.stride;
  const int rounds = (n + kSelRound - 1) / kSelRound;

  // Entry indices and the row stride are multiples of 16, so a 16-entry run
  // that starts below n lies inside the row; runs past n load entry 0.
  uint4 v[kSelPT / 4];
  auto load_round = [&](int r) {
#pragma unroll
    for (int c = 0; c < kSelPT / 16; ++c) {
      const int q0 = r * kSelRound + tid * kSelPT + 16 * c;
      const uint4* src = reinterpret_cast<const uint4*>(row + (q0 < n ? q0 : 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * c + i] = src[i];
    }
  };
  load_round(0);
  const DigitBins<kSelNT> bins = load_digit_bins<kSelNT>(h1);
  for (int i = tid; i < kBins; i += kSelNT) hist2[i] = 0u;
  find_digit_in<kSelNT>(bins, K, scan_scratch, &sh_t1, &sh_above1);
  const uint32_t t1 = (uint32_t)sh_t1;
  // digit >= t1  <=>  score >= lo (score_key folds only the top score, which
  // is above every threshold a digit can set)
  const int lo = sh_t1 < 0 ? INT_MAX : (int)(t1 << 11) - kKeyBias;

  int total = 0;
  for (int r = 0; r < rounds; ++r) {
    if (r > 0) load_round(r);
    const int p0 = r * kSelRound + tid * kSelPT;
    int nk = 0;
#pragma unroll
    for (int i = 0; i < kSelPT / 4; ++i) {
      const int w[4] = {(int)v[i].x, (int)v[i].y, (int)v[i].z, (int)v[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) nk += (w[k] >= lo && p0 + 4 * i + k < n) ? 1 : 0;
    }
    int round_total;
    int slot = total + block_exclusive_scan<kSelNT>(nk, scan_scratch, &round_total);
    if (nk > 0) {
#pragma unroll
      for (int i = 0; i < kSelPT / 4; ++i) {
        const int w[4] = {(int)v[i].x, (int)v[i].y, (int)v[i].z, (int)v[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int p = p0 + 4 * i + k;
          if (w[k] >= lo && p < n) {
            const uint2 c = make_uint2(score_key(w[k]), (uint32_t)p);
            if (slot < kSingleListCap) list[slot] = c; else ovf[slot] = c;
            ++slot;
          }
        }
      }
    }
    total += round_total;
  }
  __syncthreads();
  // low-digit histogram of the kept entries whose top digit is t1
  for (int f = tid; f < total; f += kSelNT) {
    const uint2 c = f < kSingleListCap ? list[f] : ovf[f];
    if ((c.x >> 11) == t1) atomicAdd(&hist2[c.x & (kBins - 1)], 1u);
  }
  __syncthreads();

  find_digit<kSelNT>(hist2, K - sh_above1, scan_scratch, &sh_t2, &sh_above2);
  const uint32_t tau = (t1 << 11) | (uint32_t)sh_t2;
  const int need_ties = K - sh_above1 - sh_above2;
  int32_t* out = a.out_idx + (size_t)b * K;
  const int written = emit_in_order<kSelNT>(
      [&](int f) { return f < kSingleListCap ? list[f] : ovf[f]; }, total, tau, need_ties, K,
      scan_scratch, [&](int j, uint32_t id) { out[j] = sel_id(a, b, id); });
  for (int j = written + tid; j < K; j += kSelNT) out[j] = -1;
  if (tid == 0) a.out_count[b] = written;
  for (int i = tid; i < kBins; i += kSelNT) h1[i] = 0u;     // ready for the next call
}

// ------------------------------------------------------------------ filter
__global__ __launch_bounds__(kBlock) void select_filter_kernel(SelectArgs a) {
  __shared__ int scan_scratch[kBlock / 64];
  __shared__ int sh_t1, sh_above1;

  const int b = blockIdx.y;
  const int n = sel_entries(a, b);
  const int chunk = blockIdx.x, chunk0 = chunk * kFiltChunk;
  if (a.K == 0 || n <= a.K || chunk0 >= n) return;
  const int32_t* row = a.scores + (size_t)b * a.stride;

  // this thread's 16 scores and the block's share of the histogram, loaded together
  const int p0 = chunk0 + (int)threadIdx.x * kFiltPer;
  uint4 sv[kFiltPer / 4];
  if (p0 < n) {
    const uint4* src = reinterpret_cast<const uint4*>(row + p0);
#pragma unroll
    for (int i = 0; i < kFiltPer / 4; ++i) sv[i] = src[i];
  }
  const DigitBins<kBlock> bins = load_digit_bins<kBlock>(a.hist1 + (size_t)b * kCtrlWords);
  find_digit_in<kBlock>(bins, a.K, scan_scratch, &sh_t1, &sh_above1);
  const uint32_t t1 = (uint32_t)sh_t1;

  uint32_t key[kFiltPer];
  int nk = 0;
#pragma unroll
  for (int i = 0; i < kFiltPer / 4; ++i) {
    const int w[4] = {(int)sv[i].x, (int)sv[i].y, (int)sv[i].z, (int)sv[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t kk = score_key(w[k]);
      const bool keep = p0 + 4 * i + k < n && (kk >> 11) >= t1;
      key[4 * i + k] = keep ? kk : 0u;
      nk += keep ? 1 : 0;
    }
  }
  int chunk_total;
  int slot = block_exclusive_scan<kBlock>(nk, scan_scratch, &chunk_total);
  uint2* dst = a.cand + (size_t)b * a.stride + chunk0;
#pragma unroll
  for (int e = 0; e < kFiltPer; ++e)
    if (key[e] != 0u) dst[slot++] = make_uint2(key[e], (uint32_t)(p0 + e));
  if (threadIdx.x == 0) a.chunk_counts[(size_t)b * kMaxSelChunks + chunk] = (uint32_t)chunk_total;
}

// ------------------------------------------------------------------ final
__global__ __launch_bounds__(kSelNT) void select_final_kernel(SelectArgs a) {
  __shared__ uint32_t hist2[kBins];
  __shared__ int offs[kMaxSelChunks + 1];
  __shared__ uint2 list[kListCap];
  __shared__ int scan_scratch[kSelNT / 64];
  __shared__ int sh_t1, sh_above1, sh_t2, sh_above2;

  const int b = blockIdx.x;
  const int n = sel_entries(a, b);
  const int K = a.K;
  if (K == 0 || n <= K) {
    select_all(a, b, n, kSelNT);
    return;
  }
  const int tid = threadIdx.x;
  uint32_t* h1 = a.hist1 + (size_t)b * kCtrlWords;
  const uint32_t* counts = a.chunk_counts + (size_t)b * kMaxSelChunks;
  const uint2* cand_row = a.cand + (size_t)b * a.stride;
  const int n_chunks = (n + kFiltChunk - 1) / kFiltChunk;

  const DigitBins<kSelNT> bins = load_digit_bins<kSelNT>(h1);
  for (int i = tid; i < kBins; i += kSelNT) hist2[i] = 0u;
  find_digit_in<kSelNT>(bins, K, scan_scratch, &sh_t1, &sh_above1);
  const uint32_t t1 = (uint32_t)sh_t1;

  int total = 0;
  for (int c0 = 0; c0 < n_chunks; c0 += kSelNT) {
    const int c = c0 + tid;
    const int v = c < n_chunks ? (int)counts[c] : 0;
    int round_total;
    const int pre = block_exclusive_scan<kSelNT>(v, scan_scratch, &round_total);
    if (c < n_chunks) offs[c] = total + pre;
    total += round_total;
  }
  if (tid == 0) offs[n_chunks] = total;
  __syncthreads();

  // entry f of the concatenated slot lists (already in entry order)
  auto get_global = [&](int f) -> uint2 {
    int lo = 0, hi = n_chunks - 1;          // largest c with offs[c] <= f
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (offs[mid] <= f) lo = mid; else hi = mid - 1;
    }
    return cand_row[(size_t)lo * kFiltChunk + (f - offs[lo])];
  };
  const bool cached = total <= kListCap;
  if (cached) {             // every candidate into LDS, 6 loads in flight per thread
    uint2 v[kListCap / kSelNT];
#pragma unroll
    for (int e = 0; e < kListCap / kSelNT; ++e) {
      const int f = e * kSelNT + tid;
      if (f < total) v[e] = get_global(f);
    }
#pragma unroll
    for (int e = 0; e < kListCap / kSelNT; ++e) {
      const int f = e * kSelNT + tid;
      if (f < total) list[f] = v[e];
    }
    __syncthreads();
  }
  auto get = [&](int f) -> uint2 { return cached ? list[f] : get_global(f); };

  for (int f = tid; f < total; f += kSelNT) {
    const uint2 c = get(f);
    if ((c.x >> 11) == t1) atomicAdd(&hist2[c.x & (kBins - 1)], 1u);
  }
  __syncthreads();
  find_digit<kSelNT>(hist2, K - sh_above1, scan_scratch, &sh_t2, &sh_above2);
  const uint32_t tau = (t1 << 11) | (uint32_t)sh_t2;
  const int need_ties = K - sh_above1 - sh_above2;
  int32_t* out = a.out_idx + (size_t)b * K;
  const int written = emit_in_order<kSelNT>(
      get, total, tau, need_ties, K, scan_scratch,
      [&](int j, uint32_t id) { out[j] = sel_id(a, b, id); });
  for (int j = written + tid; j < K; j += kSelNT) out[j] = -1;
  if (tid == 0) a.out_count[b] = written;
  for (int i = tid; i < kBins; i += kSelNT) h1[i] = 0u;     // ready for the next call
}

// ------------------------------------------------------------------ host
hipError_t run_select(const SelectArgs& a, int max_entries, hipStream_t st) {
  if (max_entries <= kSingleMax) {
    hipLaunchKernelGGL(select_single_kernel, dim3(a.batch), dim3(kSelNT), 0, st, a);
    return hipGetLastError();
  }
  const int chunks = (max_entries + kFiltChunk - 1) / kFiltChunk;
  hipLaunchKernelGGL(select_filter_kernel, dim3(chunks, a.batch), dim3(kBlock), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_final_kernel, dim3(a.batch), dim3(kSelNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa2
