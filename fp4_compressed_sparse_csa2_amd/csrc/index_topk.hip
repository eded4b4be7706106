// csa2_index_topk: int8 indexer scores over every cached position outside
// the window, then a deterministic Top-K (score desc, position asc).
//
// The Full layer builds the indexer state and makes the sparse selection
// whose Top-K addressing indices later layers reuse (neodrop.ai V4.1-Flash
// report, 架构拆解 item 2; zulogic "DeepSeek V4 1-Flash 架构拆解", section 3).
//
// The score kernel streams the int8 keys page by page (coalesced 1 KB wave
// loads), takes int8 dot products with v_dot4 and lane-group sums over DPP,
// and writes int32 scores plus a histogram of the top 11 bits of the biased
// 22-bit key into the sequence's global histogram.  The selection kernels in
// select.hip then take the deterministic Top-K.
//
// Scaled variant: each position also carries an fp32 key scale s_p (the
// pages pair the indexer keys with a scale), stored [page][row] beside the
// cache; the ranked value is fl32(s_p * score_p), kept as a 32-bit order key
// whose top 11 bits feed the same histogram.
#include "append.h"
#include "common.h"
#include "launch.h"
#include "select.h"

namespace csa2 {

// Pages of keys per score block (4 waves; each wave streams a quarter): 16,
// or 8 for grids of at least kSmallBlockGrid 16-page blocks, where the
// smaller blocks overlap more of one block's tail with another's loads
// (measured: 8 pages 1.9% faster at 128 sequences of 8K-128K, slower at 8 x
// 64K and at 1M).
constexpr int kChunkPages = 16;
constexpr int kSmallChunkPages = 8;
constexpr int kSmallBlockGrid = 4096;


// Candidates of sequence b: positions p_begin <= p < min(p_end, L - 128);
// entry i is position p_begin + i.
__device__ __forceinline__ int seq_candidates(const int32_t* ctx_len, int b, int max_ctx,
                                              int max_pages, int p_begin, int p_end) {
  int L = ctx_len[b];
  L = L < 0 ? 0 : L;
  L = L > max_ctx ? max_ctx : L;
  L = L > max_pages * kPage ? max_pages * kPage : L;
  int hi = L > kWindow ? L - kWindow : 0;
  hi = hi < p_end ? hi : p_end;
  return hi > p_begin ? hi - p_begin : 0;
}

// ------------------------------------------------------------------ score
struct ScoreArgs {
  const uint8_t* pages;
  const int32_t* page_table;
  int num_pages;
  int max_pages;
  int keys_off;
  int page_bytes;
  const int32_t* ctx_len;
  int max_ctx;
  int p_begin;
  int p_end;
  const int8_t* q_idx;
  const float* key_scales;    // scaled variant only
  int K;
  int32_t* scores;
  int32_t* out_scores;
  uint32_t* ctrl;
};

// Score block `chunk` of sequence b, CP pages (hist: kBins words of LDS).
template <int DI, bool SCALED, int CP>
__device__ __forceinline__ void score_block(const ScoreArgs& sa, int chunk, int b,
                                            uint32_t* hist) {
  constexpr int kChunk = CP * kPage;                  // positions per score block
  constexpr int kPagesPerWave = CP / (kBlock / 64);
  static_assert(kPagesPerWave >= 1 && CP % (kBlock / 64) == 0, "whole pages per wave");
  constexpr int LPP = DI / 16;        // lanes per position (16 key bytes each)
  constexpr int PPL = 64 / LPP;       // positions per 1 KB wave load
  const uint8_t* __restrict__ pages = sa.pages;
  const int32_t* __restrict__ page_table = sa.page_table;
  const int num_pages = sa.num_pages, max_pages = sa.max_pages, keys_off = sa.keys_off;
  const int page_bytes = sa.page_bytes, max_ctx = sa.max_ctx, p_begin = sa.p_begin;
  const int8_t* __restrict__ q_idx = sa.q_idx;
  const float* __restrict__ key_scales = sa.key_scales;
  const int K = sa.K;
  int32_t* __restrict__ scores = sa.scores;
  int32_t* __restrict__ out_scores = sa.out_scores;
  uint32_t* __restrict__ ctrl = sa.ctrl;

  const int chunk0 = chunk * kChunk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the wave's pages: a wave-uniform index, so the page-table reads are
  // scalar loads.  They go out together with the sequence's length, before
  // it is known which of the pages hold candidates (an index past the
  // table's end reads its last entry and is dropped below).
  const int lp0 = chunk0 / kPage + __builtin_amdgcn_readfirstlane(wave) * kPagesPerWave;
  const int lp_last = max_pages - 1 - p_begin / kPage;   // last entry of the table's row
  const int32_t* pt = page_table + (size_t)b * max_pages + p_begin / kPage;
  int ptv[kPagesPerWave];
  if (lp_last >= 0) {
#pragma unroll
    for (int pi = 0; pi < kPagesPerWave; ++pi) ptv[pi] = pt[min(lp0 + pi, lp_last)];
  }
  const int n = seq_candidates(sa.ctx_len, b, max_ctx, max_pages, p_begin, sa.p_end);
  if (chunk0 >= n) return;               // n > 0 implies lp_last >= 0
  const bool do_hist = K > 0 && n > K;

  const int4 qc = *reinterpret_cast<const int4*>(q_idx + (size_t)b * DI + (lane % LPP) * 16);
  __builtin_amdgcn_sched_barrier(0);     // the query goes out before the keys
  int32_t* sc_row = scores + (size_t)b * row_stride(max_ctx);
  int32_t* user_row = out_scores ? out_scores + (size_t)b * max_ctx : nullptr;
  // after the lane-group sums, lane l keeps the score of page row ppos
  const int ppos = PPL * (lane % LPP) + lane / LPP;
  int pg[kPagesPerWave];
#pragma unroll
  for (int pi = 0; pi < kPagesPerWave; ++pi) pg[pi] = ((lp0 + pi) * kPage < n) ? ptv[pi] : -1;
  // then every key load, unconditionally (a page that is not live reads
  // page 0, which always exists, and is skipped), so that page pi's compute
  // waits only for its own loads.  The keys are read once per call:
  // non-temporal loads keep them from evicting what the next kernels reuse.
  uint4 v[kPagesPerWave][LPP];
  float ks[kPagesPerWave];               // scaled: the key scale of page row ppos
  bool live[kPagesPerWave];
#pragma unroll
  for (int pi = 0; pi < kPagesPerWave; ++pi) {
    live[pi] = pg[pi] >= 0 && pg[pi] < num_pages;
    const u32x4* kp = reinterpret_cast<const u32x4*>(
        pages + (size_t)(live[pi] ? pg[pi] : 0) * page_bytes + keys_off);
#pragma unroll
    for (int j = 0; j < LPP; ++j) {
      const u32x4 t = __builtin_nontemporal_load(kp + j * 64 + lane);
      v[pi][j] = make_uint4(t.x, t.y, t.z, t.w);
    }
    if constexpr (SCALED)
      ks[pi] = __builtin_nontemporal_load(key_scales + (size_t)(live[pi] ? pg[pi] : 0) * kPage +
                                          ppos);
    __builtin_amdgcn_sched_barrier(0);   // keep the pages' loads in page order
  }
  if (do_hist) {                         // while the keys are on their way
    for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = 0u;
    __syncthreads();
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
      if constexpr (SCALED) {
        const float val = scaled_value(keep, ks[pi]);
        const uint32_t key = value_key(val);
        sc_row[p] = (int32_t)key;
        if (user_row) user_row[p_begin + p] = (int32_t)__float_as_uint(val);
        if (do_hist) atomicAdd(&hist[key >> FloatKeys::kTopShift], 1u);
      } else {
        sc_row[p] = keep;
        if (user_row) user_row[p_begin + p] = keep;
        if (do_hist) atomicAdd(&hist[score_key(keep) >> 11], 1u);
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // pages in arrival order
  }
  if (do_hist) {
    __syncthreads();
    uint32_t* g = ctrl + (size_t)b * kCtrlWords + (chunk % kHistReps) * kBins;
    uint32_t h[kBins / kBlock];
#pragma unroll
    for (int k = 0; k < kBins / kBlock; ++k) h[k] = hist[k * kBlock + threadIdx.x];
#pragma unroll
    for (int k = 0; k < kBins / kBlock; ++k)
      if (h[k]) atomicAdd(&g[k * kBlock + threadIdx.x], h[k]);
  }
}

template <int DI, bool SCALED, int CP>
__global__ __launch_bounds__(kBlock) void index_score_kernel(ScoreArgs sa) {
  __shared__ uint32_t hist[kBins];
  score_block<DI, SCALED, CP>(sa, blockIdx.x, blockIdx.y, hist);
}

// The Full layer's append fused into its scoring grid: rows 0..batch-1 of
// the grid score, row `batch` appends (tokens at scoring candidates are
// skipped, so no append write overlaps a scoring read).
template <int D, int DI, int CP>
__global__ __launch_bounds__(kBlock) void append_score_kernel(ScoreArgs sa, AppendArgs ap) {
  __shared__ uint32_t hist[kBins];
  if ((int)blockIdx.y == ap.batch) {
    append_block<D, DI>(ap, blockIdx.x);
    return;
  }
  score_block<DI, false, CP>(sa, blockIdx.x, blockIdx.y, hist);
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

template <int D, int DI, int CP>
static void launch_append_score(const dim3& grid, hipStream_t st, const ScoreArgs& sa,
                                const AppendArgs& ap) {
  const int app_blocks =
      (ap.n_tokens + append_tokens_per_block<D>() - 1) / append_tokens_per_block<D>();
  const dim3 g(grid.x > (unsigned)app_blocks ? grid.x : (unsigned)app_blocks, grid.y + 1);
  hipLaunchKernelGGL((append_score_kernel<D, DI, CP>), g, dim3(kBlock), 0, st, sa, ap);
}

// The scoring launch with CP pages per block over the grid's chunks.
template <int CP>
static void launch_score(const CacheArgs& c, int max_entries, hipStream_t st,
                         const ScoreArgs& sa, const AppendArgs* append, bool scaled) {
  constexpr int kChunk = CP * kPage;
  const int n_chunks = (max_entries + kChunk - 1) / kChunk;
  const dim3 grid(n_chunks > 0 ? n_chunks : 1, c.batch);
  if (append != nullptr && append->n_tokens > 0) {
    AppendArgs ap = *append;
    ap.ctx_len = sa.ctx_len;
    ap.max_ctx = sa.max_ctx;
#define AS_CASE(D_, DI_) \
    if (c.D == D_ && c.Di == DI_) launch_append_score<D_, DI_, CP>(grid, st, sa, ap);
    AS_CASE(128, 64) AS_CASE(128, 128) AS_CASE(256, 64) AS_CASE(256, 128)
    AS_CASE(512, 64) AS_CASE(512, 128)
#undef AS_CASE
  } else if (c.Di == 128 && !scaled) {
    hipLaunchKernelGGL((index_score_kernel<128, false, CP>), grid, dim3(kBlock), 0, st, sa);
  } else if (c.Di == 128) {
    hipLaunchKernelGGL((index_score_kernel<128, true, CP>), grid, dim3(kBlock), 0, st, sa);
  } else if (!scaled) {
    hipLaunchKernelGGL((index_score_kernel<64, false, CP>), grid, dim3(kBlock), 0, st, sa);
  } else {
    hipLaunchKernelGGL((index_score_kernel<64, true, CP>), grid, dim3(kBlock), 0, st, sa);
  }
}

hipError_t run_index_topk(const CacheArgs& c, const int32_t* ctx_len, int max_ctx,
                          const int8_t* q_idx, const float* key_scales, int K, int p_begin,
                          int p_end, int32_t* out_idx, int32_t* out_count, int32_t* out_scores,
                          int32_t* out_sel_scores, void* ws, hipStream_t st,
                          const AppendArgs* append) {
  const TopkWs w = topk_ws(c.batch, max_ctx);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint32_t* ctrl = reinterpret_cast<uint32_t*>(base + w.ctrl);
  int32_t* scores = reinterpret_cast<int32_t*>(base + w.scores);
  const PageLayout lay = page_layout(c.D, c.Di);
  int hi = max_ctx > kWindow ? max_ctx - kWindow : 0;   // most candidates a sequence can have
  hi = hi < p_end ? hi : p_end;
  const int max_entries = hi > p_begin ? hi - p_begin : 0;
  const bool scaled = key_scales != nullptr;
  ScoreArgs sa;
  sa.pages = static_cast<const uint8_t*>(c.pages);
  sa.page_table = c.page_table;
  sa.num_pages = c.num_pages;
  sa.max_pages = c.max_pages;
  sa.keys_off = lay.keys_off;
  sa.page_bytes = lay.page_bytes;
  sa.ctx_len = ctx_len;
  sa.max_ctx = max_ctx;
  sa.p_begin = p_begin;
  sa.p_end = p_end;
  sa.q_idx = q_idx;
  sa.key_scales = key_scales;
  sa.K = K;
  sa.scores = scores;
  sa.out_scores = out_scores;
  sa.ctrl = ctrl;
  const long long big_blocks =
      (long long)c.batch * ((max_entries + kChunkPages * kPage - 1) / (kChunkPages * kPage));
  if (big_blocks >= kSmallBlockGrid)
    launch_score<kSmallChunkPages>(c, max_entries, st, sa, append, scaled);
  else
    launch_score<kChunkPages>(c, max_entries, st, sa, append, scaled);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SelectArgs a;
  a.ctx_len = ctx_len;
  a.max_ctx = max_ctx;
  a.max_pages = c.max_pages;
  a.p_begin = p_begin;
  a.p_end = p_end;
  a.pool = nullptr;
  a.pool_count = nullptr;
  a.P = 0;
  a.batch = c.batch;
  a.K = K;
  a.scores = scores;
  a.stride = row_stride(max_ctx);
  a.hist1 = ctrl;
  a.cand = reinterpret_cast<uint2*>(base + w.cand);
  a.chunk_counts = reinterpret_cast<uint32_t*>(base + w.counts);
  a.out_idx = out_idx;
  a.out_count = out_count;
  a.out_sel_scores = out_sel_scores;
  a.float_keys = scaled ? 1 : 0;
  return run_select(a, max_entries, st);
}

}  // namespace csa2
