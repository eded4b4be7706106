// csa2_reindex: a Reindex layer rescoring the Full layer's candidate pool
// with its own int8 indexer query, then Top-K' under the same order and tie
// rule (score desc, position asc).
//
// Deeper indexer layers refilter only inside the candidate pool of the first
// Full layer, so their cost does not grow with the context (neodrop.ai
// V4.1-Flash report, 架构拆解 item 2); a Reindex layer reuses the KV but
// recomputes index / candidates (zulogic "DeepSeek V4 1-Flash 架构拆解",
// section 3 table).  The indexer keys are the owner's, shared by all layers.
//
// The score kernel gathers the keys of blocks of 256 pool entries (each
// entry's 64 or 128 key bytes read by 4 or 8 lanes), scores them with v_dot4
// and histograms the top digit; the selection kernels of select.hip then
// take Top-K' over the pool entries, which are in ascending position order,
// and map the winners back to positions.  The scaled variant ranks the
// float32 values fl32(s_p * score_p) with the per-token key scales instead.
#include "common.h"
#include "launch.h"
#include "select.h"

namespace csa2 {

constexpr int kREntries = 256;          // pool entries per block
constexpr int kRPtCache = 1024;         // page-table entries staged in LDS (65536 positions)
constexpr int kRPtPer = kRPtCache / kBlock;

template <int DI, bool SCALED>
__global__ __launch_bounds__(kBlock) void reindex_score_kernel(
    const uint8_t* __restrict__ pages, const int32_t* __restrict__ page_table, int num_pages,
    int max_pages, int keys_off, int page_bytes, const int8_t* __restrict__ q_idx,
    const float* __restrict__ key_scales,
    const int32_t* __restrict__ pool, const int32_t* __restrict__ pool_count, int P, int K,
    int32_t* __restrict__ scores, int stride, int32_t* __restrict__ out_scores,
    uint32_t* __restrict__ ctrl) {
  constexpr int LPP = DI / 16;
  constexpr int PPL = 64 / LPP;
  __shared__ uint32_t hist[kBins];
  __shared__ int32_t pt_lds[kRPtCache];

  const int b = blockIdx.y;
  int c = pool_count[b];
  c = c < 0 ? 0 : (c > P ? P : c);
  const int e0 = blockIdx.x * kREntries;
  const bool do_hist = K > 0 && c > K;          // a selection will run
  if (e0 >= c || (!do_hist && out_scores == nullptr)) return;
  const int32_t* prow = pool + (size_t)b * P;
  int32_t* sc_row = scores + (size_t)b * stride;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t* pt = page_table + (size_t)b * max_pages;
  const int wbase = e0 + wave * 64;

  // The pool entries, the query and (up to kRPtCache pages) the sequence's
  // page table are loaded together; the page of an entry is then an LDS
  // read, so a key row is the second dependent trip, not the third.
  const bool pt_in_lds = max_pages <= kRPtCache;
  int pe[LPP];
#pragma unroll
  for (int j = 0; j < LPP; ++j) {       // entry wbase + j*PPL + lane/LPP
    const int e = wbase + j * PPL + lane / LPP;
    pe[j] = e < c ? prow[e] : -1;
  }
  const int4 qc = *reinterpret_cast<const int4*>(q_idx + (size_t)b * DI + (lane % LPP) * 16);
  if (pt_in_lds) {
    int ptv[kRPtPer];
#pragma unroll
    for (int i = 0; i < kRPtPer; ++i) {
      const int k = threadIdx.x + i * kBlock;
      ptv[i] = k < max_pages ? pt[k] : -1;
    }
#pragma unroll
    for (int i = 0; i < kRPtPer; ++i) pt_lds[threadIdx.x + i * kBlock] = ptv[i];
  }
  if (do_hist)
    for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = 0u;
  if (pt_in_lds || do_hist) __syncthreads();       // block-uniform

  // pages of the LPP entries first, then their key rows: every key load of
  // the lane is in flight at once
  int pg[LPP];
  if (pt_in_lds) {
#pragma unroll
    for (int j = 0; j < LPP; ++j) {
      const bool in = pe[j] >= 0 && pe[j] < max_pages * kPage;
      const int g = pt_lds[in ? pe[j] / kPage : 0];
      pg[j] = in ? g : -1;
    }
  } else {
#pragma unroll
    for (int j = 0; j < LPP; ++j)
      pg[j] = (pe[j] >= 0 && pe[j] < max_pages * kPage) ? pt[pe[j] / kPage] : -1;
  }
  uint4 v[LPP];
  bool ok[LPP];
  int srow = -1;                        // scaled: key-scale slot of the entry this lane keeps
#pragma unroll
  for (int j = 0; j < LPP; ++j) {
    const int p = pe[j];
    ok[j] = pg[j] >= 0 && pg[j] < num_pages;
    if (ok[j])
      v[j] = *reinterpret_cast<const uint4*>(pages + (size_t)pg[j] * page_bytes + keys_off +
                                             (p % kPage) * DI + (lane % LPP) * 16);
    if (SCALED && (lane % LPP) == j && ok[j]) srow = pg[j] * kPage + p % kPage;
  }
  float ks = 0.0f;
  if constexpr (SCALED) ks = srow >= 0 ? key_scales[srow] : 0.0f;
  int keep = 0;
  bool keep_ok = false;
#pragma unroll
  for (int j = 0; j < LPP; ++j) {
    int d = 0;
    if (ok[j]) {
      d = __builtin_amdgcn_sdot4((int)v[j].x, qc.x, 0, false);
      d = __builtin_amdgcn_sdot4((int)v[j].y, qc.y, d, false);
      d = __builtin_amdgcn_sdot4((int)v[j].z, qc.z, d, false);
      d = __builtin_amdgcn_sdot4((int)v[j].w, qc.w, d, false);
    }
    d = (LPP == 8) ? sum_oct(d) : sum_quad(d);
    if ((lane % LPP) == j) {
      keep = d;
      keep_ok = ok[j];
    }
  }
  const int e = wbase + PPL * (lane % LPP) + lane / LPP;
  if (e < c) {
    if constexpr (SCALED) {
      // an unusable entry ranks as -inf, below every finite value
      const float val = keep_ok ? scaled_value(keep, ks) : -__builtin_inff();
      const uint32_t key = value_key(val);
      sc_row[e] = (int32_t)key;
      if (out_scores != nullptr) out_scores[(size_t)b * P + e] = (int32_t)__float_as_uint(val);
      if (do_hist) atomicAdd(&hist[key >> FloatKeys::kTopShift], 1u);
    } else {
      // an unusable entry (contract violation) ranks below every real score
      const int s = keep_ok ? keep : -kKeyBias;
      sc_row[e] = s;
      if (out_scores != nullptr) out_scores[(size_t)b * P + e] = s;
      if (do_hist) atomicAdd(&hist[score_key(s) >> 11], 1u);
    }
  }
  if (do_hist) {
    __syncthreads();
    // block i adds into histogram replica i % kHistReps
    uint32_t* g = ctrl + (size_t)b * kCtrlWords + (size_t)(blockIdx.x % kHistReps) * kBins;
    for (int i = threadIdx.x; i < kBins; i += kBlock) {
      const uint32_t h = hist[i];
      if (h) atomicAdd(&g[i], h);
    }
  }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct ReindexWs {
  size_t ctrl, counts, scores, cand, total;
};
static ReindexWs reindex_ws(int batch, int P) {
  const size_t stride = (size_t)row_stride(P);
  ReindexWs w;
  w.ctrl = 0;
  w.counts = align256((size_t)batch * kCtrlWords * 4);
  w.scores = w.counts + align256((size_t)batch * kMaxSelChunks * 4);
  w.cand = w.scores + align256((size_t)batch * stride * 4);
  w.total = w.cand + align256((size_t)batch * stride * 8);
  return w;
}

size_t reindex_ws_bytes(int batch, int P, int /*K*/) { return reindex_ws(batch, P).total; }

template <int DI, bool SCALED>
static void launch_rescore(const dim3& grid, hipStream_t st, const CacheArgs& c,
                           const PageLayout& lay, const int8_t* q_idx, const float* key_scales,
                           const int32_t* pool, const int32_t* pool_count, int P, int K,
                           int32_t* scores, int stride, int32_t* out_scores, uint32_t* ctrl) {
  hipLaunchKernelGGL((reindex_score_kernel<DI, SCALED>), grid, dim3(kBlock), 0, st,
                     (const uint8_t*)c.pages, c.page_table, c.num_pages, c.max_pages,
                     lay.keys_off, lay.page_bytes, q_idx, key_scales, pool, pool_count, P, K,
                     scores, stride, out_scores, ctrl);
}

hipError_t run_reindex(const CacheArgs& c, const int8_t* q_idx, const float* key_scales,
                       const int32_t* pool, const int32_t* pool_count, int P, int K,
                       int32_t* out_idx, int32_t* out_count, int32_t* out_scores, void* ws,
                       hipStream_t st) {
  const ReindexWs w = reindex_ws(c.batch, P);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint32_t* ctrl = reinterpret_cast<uint32_t*>(base + w.ctrl);
  int32_t* scores = reinterpret_cast<int32_t*>(base + w.scores);
  const int stride = row_stride(P);
  const PageLayout lay = page_layout(c.D, c.Di);
  if (P > 0) {
    const dim3 grid((P + kREntries - 1) / kREntries, c.batch);
    if (c.Di == 128 && key_scales == nullptr)
      launch_rescore<128, false>(grid, st, c, lay, q_idx, nullptr, pool, pool_count, P, K,
                                 scores, stride, out_scores, ctrl);
    else if (c.Di == 128)
      launch_rescore<128, true>(grid, st, c, lay, q_idx, key_scales, pool, pool_count, P, K,
                                scores, stride, out_scores, ctrl);
    else if (key_scales == nullptr)
      launch_rescore<64, false>(grid, st, c, lay, q_idx, nullptr, pool, pool_count, P, K,
                                scores, stride, out_scores, ctrl);
    else
      launch_rescore<64, true>(grid, st, c, lay, q_idx, key_scales, pool, pool_count, P, K,
                               scores, stride, out_scores, ctrl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  SelectArgs a;
  a.ctx_len = nullptr;
  a.max_ctx = 0;
  a.max_pages = c.max_pages;
  a.p_begin = 0;
  a.p_end = 0;
  a.pool = pool;
  a.pool_count = pool_count;
  a.P = P;
  a.batch = c.batch;
  a.K = K;
  a.scores = scores;
  a.stride = stride;
  a.hist1 = ctrl;
  a.cand = reinterpret_cast<uint2*>(base + w.cand);
  a.chunk_counts = reinterpret_cast<uint32_t*>(base + w.counts);
  a.out_idx = out_idx;
  a.out_count = out_count;
  a.out_sel_scores = nullptr;
  a.float_keys = key_scales != nullptr ? 1 : 0;
  return run_select(a, P, st);
}

}  // namespace csa2
