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
// One kernel: blocks of 256 pool entries gather the keys (each entry's 64 or
// 128 key bytes read by 4 or 8 lanes), score them with v_dot4 and histogram
// the top digit; the last block of each sequence fixes the exact threshold
// and emits the winners in ascending pool order (= ascending position, the
// pool being ascending).
#include "common.h"
#include "launch.h"
#include "select.h"

namespace csa2 {

constexpr int kREntries = 256;          // pool entries per block
constexpr int kRCtrlWords = kBins + 64; // hist1 [2048], done at kBins

template <int DI>
__global__ __launch_bounds__(kBlock) void reindex_kernel(
    const uint8_t* __restrict__ pages, const int32_t* __restrict__ page_table, int num_pages,
    int max_pages, int keys_off, int page_bytes, const int8_t* __restrict__ q_idx,
    const int32_t* __restrict__ pool, const int32_t* __restrict__ pool_count, int P, int K,
    int32_t* __restrict__ scores, uint32_t* __restrict__ ctrl, int32_t* __restrict__ out_idx,
    int32_t* __restrict__ out_count) {
  constexpr int LPP = DI / 16;
  constexpr int PPL = 64 / LPP;
  __shared__ uint32_t hist[kBins];
  __shared__ int scan_scratch[4];
  __shared__ int sh_t1, sh_above1, sh_t2, sh_above2, sh_last;

  const int b = blockIdx.y;
  int c = pool_count[b];
  c = c < 0 ? 0 : (c > P ? P : c);
  const int e0 = blockIdx.x * kREntries;
  const int32_t* prow = pool + (size_t)b * P;
  int32_t* out = out_idx + (size_t)b * K;

  if (K == 0 || c <= K) {               // every pool entry survives
    for (int i = e0 + threadIdx.x; i < e0 + kREntries && i < K; i += kBlock)
      out[i] = i < c ? prow[i] : -1;
    if (blockIdx.x == 0 && threadIdx.x == 0) out_count[b] = c < K ? c : K;
    return;
  }
  if (e0 >= c) return;
  const int n_blocks = (c + kREntries - 1) / kREntries;
  uint32_t* cb = ctrl + (size_t)b * kRCtrlWords;
  int32_t* sc_row = scores + (size_t)b * P;

  for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = 0u;
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int4 qc = *reinterpret_cast<const int4*>(q_idx + (size_t)b * DI + (lane % LPP) * 16);
  const int32_t* pt = page_table + (size_t)b * max_pages;
  const int wbase = e0 + wave * 64;
  uint4 v[LPP];
  bool ok[LPP];
#pragma unroll
  for (int j = 0; j < LPP; ++j) {       // entry wbase + j*PPL + lane/LPP
    const int e = wbase + j * PPL + lane / LPP;
    const int p = e < c ? prow[e] : -1;
    const int pg = (p >= 0 && p < max_pages * kPage) ? pt[p / kPage] : -1;
    ok[j] = pg >= 0 && pg < num_pages;
    if (ok[j])
      v[j] = *reinterpret_cast<const uint4*>(pages + (size_t)pg * page_bytes + keys_off +
                                             (p % kPage) * DI + (lane % LPP) * 16);
  }
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
    // an unusable entry (contract violation) ranks below every real score
    const int s = keep_ok ? keep : -kKeyBias;
    sc_row[e] = s;
    atomicAdd(&hist[score_key(s) >> 11], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += kBlock) {
    const uint32_t h = hist[i];
    if (h) atomicAdd(&cb[i], h);
  }

  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) sh_last = (atomicAdd(&cb[kBins], 1u) == (uint32_t)(n_blocks - 1));
  __syncthreads();
  if (!sh_last) return;
  __threadfence();

  // last block of this sequence: exact threshold over the whole pool
  find_digit(cb, K, scan_scratch, &sh_t1, &sh_above1);
  const uint32_t t1 = (uint32_t)sh_t1;
  for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < c; i += kBlock) {
    const uint32_t key = score_key(sc_row[i]);
    if ((key >> 11) == t1) atomicAdd(&hist[key & (kBins - 1)], 1u);
  }
  __syncthreads();
  const int need1 = K - sh_above1;
  find_digit(hist, need1, scan_scratch, &sh_t2, &sh_above2);
  const uint32_t tau = (t1 << 11) | (uint32_t)sh_t2;
  const int need_ties = need1 - sh_above2;
  // the pool is ascending, so pool order is position order
  const int written = emit_in_order(
      [&](int i) { return make_uint2(score_key(sc_row[i]), (uint32_t)prow[i]); }, c, tau,
      need_ties, out, K, scan_scratch);
  for (int j = written + threadIdx.x; j < K; j += kBlock) out[j] = -1;
  if (threadIdx.x == 0) out_count[b] = written;
  for (int i = threadIdx.x; i < kRCtrlWords; i += kBlock) cb[i] = 0u;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t reindex_ws_bytes(int batch, int P, int /*K*/) {
  return align256((size_t)batch * kRCtrlWords * 4) + align256((size_t)batch * P * 4);
}

hipError_t run_reindex(const CacheArgs& c, const int8_t* q_idx, const int32_t* pool,
                       const int32_t* pool_count, int P, int K, int32_t* out_idx,
                       int32_t* out_count, int32_t* out_scores, void* ws, hipStream_t st) {
  uint32_t* ctrl = static_cast<uint32_t*>(ws);
  int32_t* scores = out_scores ? out_scores
                               : reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) +
                                                            align256((size_t)c.batch * kRCtrlWords * 4));
  const PageLayout lay = page_layout(c.D, c.Di);
  const int span = P > K ? P : K;
  const dim3 grid(span > 0 ? (span + kREntries - 1) / kREntries : 1, c.batch);
  if (c.Di == 128)
    hipLaunchKernelGGL(reindex_kernel<128>, grid, dim3(kBlock), 0, st, (const uint8_t*)c.pages,
                       c.page_table, c.num_pages, c.max_pages, lay.keys_off, lay.page_bytes,
                       q_idx, pool, pool_count, P, K, scores, ctrl, out_idx, out_count);
  else
    hipLaunchKernelGGL(reindex_kernel<64>, grid, dim3(kBlock), 0, st, (const uint8_t*)c.pages,
                       c.page_table, c.num_pages, c.max_pages, lay.keys_off, lay.page_bytes,
                       q_idx, pool, pool_count, P, K, scores, ctrl, out_idx, out_count);
  return hipGetLastError();
}

}  // namespace csa2
