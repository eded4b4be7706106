// csa2_index_topk: int8 indexer scores over every cached position outside
// the window, then a deterministic Top-K (score desc, position asc).
//
// The Full layer builds the indexer state and makes the sparse selection
// whose Top-K addressing indices later layers reuse (neodrop.ai V4.1-Flash
// report, 架构拆解 item 2; zulogic "DeepSeek V4 1-Flash 架构拆解", section 3).
//
// Two kernels:
//   score  - streams the int8 keys page by page (coalesced 1 KB wave loads),
//            int8 dot products with v_dot4, lane-group sums over DPP; writes
//            int32 scores and a histogram of the top 11 bits of the biased
//            22-bit key into the sequence's global histogram.
//   select - every block finds the K-th largest top digit t1 and keeps the
//            positions of its 4096-position chunk whose digit is >= t1, in
//            position order, in the chunk's own candidate slots (one block
//            scan, no shared counter); the last block of each sequence to
//            finish histograms the low digit over the candidates, fixes the
//            exact threshold and emits the chunks' lists in order -- they
//            are already ascending -- taking ties by position, then returns
//            the control words to zero.
#include "common.h"
#include "launch.h"
#include "select.h"

namespace csa2 {

// Pages of keys per score block (4 waves; each wave streams a quarter).
#ifndef CSA2_SCORE_CHUNK_PAGES
#define CSA2_SCORE_CHUNK_PAGES 16
#endif
constexpr int kChunkPages = CSA2_SCORE_CHUNK_PAGES;
constexpr int kChunk = kChunkPages * kPage;      // positions per score block
constexpr int kPagesPerWave = kChunkPages / (kBlock / 64);
static_assert(kPagesPerWave >= 1 && kChunkPages % (kBlock / 64) == 0, "whole pages per wave");

// Per-sequence control block in the workspace (uint32 words).  Its size does
// not depend on the call's sizes, so a zeroed workspace stays zeroed between
// calls of any shape.
constexpr int kCtrlHist1 = 0;
constexpr int kCtrlDone = kBins;
constexpr int kCtrlWords = kBins + 64;

constexpr int kSelPer = 16;                    // scores per thread in the select kernel
constexpr int kSelChunk = kBlock * kSelPer;    // 4096 positions per select block
constexpr int kMaxSelChunks = (1 << 24) / kSelChunk;

// Row stride (in entries) of the score and candidate arrays: a multiple of 64
// so that every row starts 256-byte aligned.
__host__ __device__ inline int row_stride(int max_ctx) { return (max_ctx + 63) & ~63; }

__device__ __forceinline__ int seq_candidates(const int32_t* ctx_len, int b, int max_ctx,
                                              int max_pages) {
  int L = ctx_len[b];
  L = L < 0 ? 0 : L;
  L = L > max_ctx ? max_ctx : L;
  L = L > max_pages * kPage ? max_pages * kPage : L;
  return L > kWindow ? L - kWindow : 0;
}

// ------------------------------------------------------------------ score
template <int DI>
__global__ __launch_bounds__(kBlock) void index_score_kernel(
    const uint8_t* __restrict__ pages, const int32_t* __restrict__ page_table, int num_pages,
    int max_pages, int keys_off, int page_bytes, const int32_t* __restrict__ ctx_len,
    int max_ctx, const int8_t* __restrict__ q_idx, int K, int32_t* __restrict__ scores,
    int32_t* __restrict__ out_scores, uint32_t* __restrict__ ctrl) {
  constexpr int LPP = DI / 16;        // lanes per position (16 key bytes each)
  constexpr int PPL = 64 / LPP;       // positions per 1 KB wave load
  __shared__ uint32_t hist[kBins];

  const int b = blockIdx.y;
  const int n = seq_candidates(ctx_len, b, max_ctx, max_pages);
  const int chunk0 = blockIdx.x * kChunk;
  if (chunk0 >= n) return;
  const bool do_hist = K > 0 && n > K;
  if (do_hist) {
    for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = 0u;
    __syncthreads();
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int4 qc = *reinterpret_cast<const int4*>(q_idx + (size_t)b * DI + (lane % LPP) * 16);
  const int32_t* pt = page_table + (size_t)b * max_pages;
  int32_t* sc_row = scores + (size_t)b * row_stride(max_ctx);
  int32_t* user_row = out_scores ? out_scores + (size_t)b * max_ctx : nullptr;
  // after the lane-group sums, lane l keeps the score of page row ppos
  const int ppos = PPL * (lane % LPP) + lane / LPP;

  const int lp0 = chunk0 / kPage + wave * kPagesPerWave;
  uint4 v[kPagesPerWave][LPP];
  bool live[kPagesPerWave];
#pragma unroll
  for (int pi = 0; pi < kPagesPerWave; ++pi) {          // issue every load first
    const int lp = lp0 + pi;
    const int pg = (lp * kPage < n) ? pt[lp] : -1;
    live[pi] = pg >= 0 && pg < num_pages;
    if (live[pi]) {
      const uint4* kp =
          reinterpret_cast<const uint4*>(pages + (size_t)pg * page_bytes + keys_off);
#pragma unroll
      for (int j = 0; j < LPP; ++j) v[pi][j] = kp[j * 64 + lane];
    }
  }
#pragma unroll
  for (int pi = 0; pi < kPagesPerWave; ++pi) {
    if (!live[pi]) continue;
    int keep = 0;
#pragma unroll
    for (int j = 0; j < LPP; ++j) {
      int d = __builtin_amdgcn_sdot4((int)v[pi][j].x, qc.x, 0, false);
      d = __builtin_amdgcn_sdot4((int)v[pi][j].y, qc.y, d, false);
      d = __builtin_amdgcn_sdot4((int)v[pi][j].z, qc.z, d, false);
      d = __builtin_amdgcn_sdot4((int)v[pi][j].w, qc.w, d, false);
      d = (LPP == 8) ? sum_oct(d) : sum_quad(d);
      keep = ((lane % LPP) == j) ? d : keep;
    }
    const int p = (lp0 + pi) * kPage + ppos;
    if (p < n) {
      sc_row[p] = keep;
      if (user_row) user_row[p] = keep;
      if (do_hist) atomicAdd(&hist[score_key(keep) >> 11], 1u);
    }
  }
  if (do_hist) {
    __syncthreads();
    uint32_t* g = ctrl + (size_t)b * kCtrlWords + kCtrlHist1;
    for (int i = threadIdx.x; i < kBins; i += kBlock) {
      const uint32_t h = hist[i];
      if (h) atomicAdd(&g[i], h);
    }
  }
}

// ------------------------------------------------------------------ select
constexpr int kCandCache = 6144;               // candidates the last block keeps in LDS

__global__ __launch_bounds__(kBlock) void index_select_kernel(
    const int32_t* __restrict__ ctx_len, int max_ctx, int max_pages, int K,
    const int32_t* __restrict__ scores, uint32_t* __restrict__ ctrl,
    uint32_t* __restrict__ chunk_counts, uint2* __restrict__ cand, int32_t* __restrict__ out_idx,
    int32_t* __restrict__ out_count) {
  __shared__ uint32_t hist2[kBins];
  __shared__ int offs[kMaxSelChunks + 1];
  __shared__ uint2 cache[kCandCache];
  __shared__ int scan_scratch[4];
  __shared__ int sh_t1, sh_above1, sh_t2, sh_above2, sh_last;

  const int b = blockIdx.y;
  const int n = seq_candidates(ctx_len, b, max_ctx, max_pages);
  const int chunk = blockIdx.x, chunk0 = chunk * kSelChunk;
  int32_t* out = out_idx + (size_t)b * K;

  // Trivial cases: no candidates, K = 0, or every candidate selected.
  if (K == 0 || n <= K) {
    for (int i = chunk0 + threadIdx.x; i < chunk0 + kSelChunk && i < K; i += kBlock)
      out[i] = i < n ? i : -1;
    if (chunk == 0 && threadIdx.x == 0) out_count[b] = n < K ? n : K;
    return;
  }
  if (chunk0 >= n) return;
  const int n_chunks = (n + kSelChunk - 1) / kSelChunk;
  const int stride = row_stride(max_ctx);
  uint32_t* cb = ctrl + (size_t)b * kCtrlWords;
  uint32_t* counts = chunk_counts + (size_t)b * kMaxSelChunks;
  uint2* cand_row = cand + (size_t)b * stride;

  // 1. this thread's 16 scores and 8 histogram bins, loaded together
  const int p0 = chunk0 + (int)threadIdx.x * kSelPer;
  uint4 sv[kSelPer / 4];
  if (p0 < n) {             // p0 and the stride are multiples of 16: the row holds p0..p0+15
    const uint4* src = reinterpret_cast<const uint4*>(scores + (size_t)b * stride + p0);
#pragma unroll
    for (int i = 0; i < kSelPer / 4; ++i) sv[i] = src[i];
  }
  const DigitBins bins = load_digit_bins_vec(cb + kCtrlHist1);

  // 2. top digit t1: the K-th largest key lies in bin t1
  find_digit_in(bins, K, scan_scratch, &sh_t1, &sh_above1);
  const uint32_t t1 = (uint32_t)sh_t1;

  // 3. keep digit >= t1, in position order, in this chunk's candidate slots
  {
    uint32_t key[kSelPer];
    int nk = 0;
#pragma unroll
    for (int i = 0; i < kSelPer / 4; ++i) {
      const int w[4] = {(int)sv[i].x, (int)sv[i].y, (int)sv[i].z, (int)sv[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t kk = score_key(w[k]);
        const bool keep = p0 + 4 * i + k < n && (kk >> 11) >= t1;
        key[4 * i + k] = keep ? kk : 0u;      // every real key is >= 2^14, so 0 marks "dropped"
        nk += keep ? 1 : 0;
      }
    }
    int chunk_total;
    int slot = block_exclusive_scan(nk, scan_scratch, &chunk_total);
    uint2* dst = cand_row + chunk0;
#pragma unroll
    for (int e = 0; e < kSelPer; ++e)
      if (key[e] != 0u) dst[slot++] = make_uint2(key[e], (uint32_t)(p0 + e));
    if (threadIdx.x == 0) counts[chunk] = (uint32_t)chunk_total;
  }

  // 4. the last block of this sequence finishes the selection
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) sh_last = (atomicAdd(&cb[kCtrlDone], 1u) == (uint32_t)(n_chunks - 1));
  __syncthreads();
  if (!sh_last) return;
  __threadfence();

  int total = 0;
  for (int c0 = 0; c0 < n_chunks; c0 += kBlock) {
    const int c = c0 + (int)threadIdx.x;
    const int v = c < n_chunks ? (int)counts[c] : 0;
    int round_total;
    const int pre = block_exclusive_scan(v, scan_scratch, &round_total);
    if (c < n_chunks) offs[c] = total + pre;
    total += round_total;
  }
  if (threadIdx.x == 0) offs[n_chunks] = total;
  for (int i = threadIdx.x; i < kBins; i += kBlock) hist2[i] = 0u;
  __syncthreads();

  // flat index over the concatenated chunk lists -> (key, position) in global memory
  auto get_global = [&](int f) -> uint2 {
    int lo = 0, hi = n_chunks - 1;          // largest c with offs[c] <= f
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (offs[mid] <= f) lo = mid; else hi = mid - 1;
    }
    return cand_row[(size_t)lo * kSelChunk + (f - offs[lo])];
  };
  const bool cached = total <= kCandCache;
  if (cached) {             // pull every candidate into LDS, 8 loads in flight per thread
    for (int f0 = 0; f0 < total; f0 += kBlock * 8) {
      uint2 v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int f = f0 + e * kBlock + (int)threadIdx.x;
        if (f < total) v[e] = get_global(f);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int f = f0 + e * kBlock + (int)threadIdx.x;
        if (f < total) cache[f] = v[e];
      }
    }
    __syncthreads();
  }
  auto get = [&](int f) -> uint2 { return cached ? cache[f] : get_global(f); };

  for (int f = threadIdx.x; f < total; f += kBlock) {
    const uint2 c = get(f);
    if ((c.x >> 11) == t1) atomicAdd(&hist2[c.x & (kBins - 1)], 1u);
  }
  __syncthreads();
  const int need1 = K - sh_above1;
  find_digit(hist2, need1, scan_scratch, &sh_t2, &sh_above2);
  const uint32_t tau = (t1 << 11) | (uint32_t)sh_t2;
  const int need_ties = need1 - sh_above2;
  const int written = emit_in_order(get, total, tau, need_ties, out, K, scan_scratch);
  for (int j = written + threadIdx.x; j < K; j += kBlock) out[j] = -1;
  if (threadIdx.x == 0) out_count[b] = written;

  // 5. leave the control words zero for the next call
  for (int i = threadIdx.x; i < kCtrlWords; i += kBlock) cb[i] = 0u;
}

// ------------------------------------------------------------------ host
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct TopkWs {
  size_t ctrl, counts, scores, cand, total;
};
static TopkWs topk_ws(int batch, int max_ctx) {
  const size_t stride = (size_t)row_stride(max_ctx);
  TopkWs w;
  w.ctrl = 0;
  w.counts = align256((size_t)batch * kCtrlWords * 4);
  w.scores = w.counts + align256((size_t)batch * kMaxSelChunks * 4);
  w.cand = w.scores + align256((size_t)batch * stride * 4);
  w.total = w.cand + align256((size_t)batch * stride * 8);
  return w;
}

size_t index_topk_ws_bytes(int batch, int max_ctx, int /*K*/) {
  return topk_ws(batch, max_ctx).total;
}

hipError_t run_index_topk(const CacheArgs& c, const int32_t* ctx_len, int max_ctx,
                          const int8_t* q_idx, int K, int32_t* out_idx, int32_t* out_count,
                          int32_t* out_scores, void* ws, hipStream_t st) {
  const TopkWs w = topk_ws(c.batch, max_ctx);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint32_t* ctrl = reinterpret_cast<uint32_t*>(base + w.ctrl);
  uint32_t* counts = reinterpret_cast<uint32_t*>(base + w.counts);
  int32_t* scores = reinterpret_cast<int32_t*>(base + w.scores);
  uint2* cand = reinterpret_cast<uint2*>(base + w.cand);
  const PageLayout lay = page_layout(c.D, c.Di);
  const int n_chunks = (max_ctx + kChunk - 1) / kChunk;
  const dim3 grid(n_chunks > 0 ? n_chunks : 1, c.batch);
  if (c.Di == 128)
    hipLaunchKernelGGL(index_score_kernel<128>, grid, dim3(kBlock), 0, st,
                       (const uint8_t*)c.pages, c.page_table, c.num_pages, c.max_pages,
                       lay.keys_off, lay.page_bytes, ctx_len, max_ctx, q_idx, K, scores,
                       out_scores, ctrl);
  else
    hipLaunchKernelGGL(index_score_kernel<64>, grid, dim3(kBlock), 0, st,
                       (const uint8_t*)c.pages, c.page_table, c.num_pages, c.max_pages,
                       lay.keys_off, lay.page_bytes, ctx_len, max_ctx, q_idx, K, scores,
                       out_scores, ctrl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int span = max_ctx > K ? max_ctx : K;
  const int sel_chunks = (span + kSelChunk - 1) / kSelChunk;
  hipLaunchKernelGGL(index_select_kernel, dim3(sel_chunks > 0 ? sel_chunks : 1, c.batch),
                     dim3(kBlock), 0, st, ctx_len, max_ctx, c.max_pages, K, scores, ctrl, counts,
                     cand, out_idx, out_count);
  return hipGetLastError();
}

}  // namespace csa2
