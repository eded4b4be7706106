// Merges for context-sharded decoding: the Top-K of several shard-local
// selections, and the LSE merge of attention over several key sets.
//
// A shard (one device's contiguous page range of one long sequence) ranks its
// own candidates by the same total order (score desc, position asc) and keeps
// its local Top-K; the global Top-K is the Top-K of the union of the local
// lists, because an entry of the global selection is beaten by fewer than K
// entries overall, hence by fewer than K within its shard.  The selection
// rule itself is the Full layer's (neodrop.ai V4.1-Flash report, 架构拆解
// item 2); the merged attention is one softmax over the union of the shards'
// rows (infernews.com V4.1 Flash page, section 2), which the LSE merge of the
// parts reproduces exactly in real arithmetic.
#include "common.h"
#include "launch.h"
#include "select.h"

namespace csa2 {

// Block (part s, sequence b): append part s's first counts[s][b] entries (a
// strictly ascending position list with its scores) at its offset in the
// concatenation of the parts, and add their top digits to the sequence's
// histogram when a selection will run.  Block (0, b) writes the total.
// VALUES: the scores are float32 values (scaled indexer), stored as their
// order keys.
template <bool VALUES>
__global__ __launch_bounds__(kBlock) void merge_concat_kernel(
    int n_parts, int K_in, int K, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ scores, const int32_t* __restrict__ counts, int batch,
    int32_t* __restrict__ pool, int32_t* __restrict__ cat_scores, int32_t* __restrict__ pool_count,
    int stride, uint32_t* __restrict__ ctrl) {
  __shared__ uint32_t hist[kBins];
  const int s = blockIdx.x, b = blockIdx.y;
  int off = 0, total = 0, mine = 0;
  for (int t = 0; t < n_parts; ++t) {
    int c = counts[(size_t)t * batch + b];
    c = c < 0 ? 0 : (c > K_in ? K_in : c);
    off += t < s ? c : 0;
    mine = t == s ? c : mine;
    total += c;
  }
  if (s == 0 && threadIdx.x == 0) pool_count[b] = total;
  const bool do_hist = K > 0 && total > K;
  if (do_hist) {
    for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = 0u;
    __syncthreads();
  }
  const size_t src = ((size_t)s * batch + b) * K_in;
  const size_t dst = (size_t)b * stride + off;
  for (int i = threadIdx.x; i < mine; i += kBlock) {
    const int32_t sc = scores[src + i];
    pool[dst + i] = idx[src + i];
    if constexpr (VALUES) {
      const float v = __int_as_float(sc);
      const uint32_t key = value_key(v == 0.0f ? 0.0f : v);
      cat_scores[dst + i] = (int32_t)key;
      if (do_hist) atomicAdd(&hist[key >> FloatKeys::kTopShift], 1u);
    } else {
      cat_scores[dst + i] = sc;
      if (do_hist) atomicAdd(&hist[score_key(sc) >> 11], 1u);
    }
  }
  if (do_hist) {
    __syncthreads();
    uint32_t* g = ctrl + (size_t)b * kCtrlWords;
    for (int i = threadIdx.x; i < kBins; i += kBlock) {
      const uint32_t h = hist[i];
      if (h) atomicAdd(&g[i], h);
    }
  }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct MergeWs {
  size_t ctrl, counts, pool_count, pool, scores, cand, total;
};
static MergeWs merge_ws(int batch, int P) {
  const size_t stride = (size_t)row_stride(P);
  MergeWs w;
  w.ctrl = 0;
  w.counts = align256((size_t)batch * kCtrlWords * 4);
  w.pool_count = w.counts + align256((size_t)batch * kMaxSelChunks * 4);
  w.pool = w.pool_count + align256((size_t)batch * 4);
  w.scores = w.pool + align256((size_t)batch * stride * 4);
  w.cand = w.scores + align256((size_t)batch * stride * 4);
  w.total = w.cand + align256((size_t)batch * stride * 8);
  return w;
}

size_t topk_merge_ws_bytes(int batch, int n_parts, int K_in, int /*K*/) {
  return merge_ws(batch, n_parts * K_in).total;
}

hipError_t run_topk_merge(int batch, int n_parts, int K_in, const int32_t* idx,
                          const int32_t* scores, const int32_t* counts, int K, int32_t* out_idx,
                          int32_t* out_count, int32_t* out_sel_scores, void* ws, hipStream_t st,
                          bool values) {
  const int P = n_parts * K_in;
  const MergeWs w = merge_ws(batch, P);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint32_t* ctrl = reinterpret_cast<uint32_t*>(base + w.ctrl);
  int32_t* pool = reinterpret_cast<int32_t*>(base + w.pool);
  int32_t* cat = reinterpret_cast<int32_t*>(base + w.scores);
  int32_t* pool_count = reinterpret_cast<int32_t*>(base + w.pool_count);
  const int stride = row_stride(P);
  const bool some = n_parts > 0 && K_in > 0;
  const dim3 grid(some ? n_parts : 1, batch);
  const int np = some ? n_parts : 0, kin = some ? K_in : 0;
  if (values)
    hipLaunchKernelGGL(merge_concat_kernel<true>, grid, dim3(kBlock), 0, st, np, kin, K, idx,
                       scores, counts, batch, pool, cat, pool_count, stride, ctrl);
  else
    hipLaunchKernelGGL(merge_concat_kernel<false>, grid, dim3(kBlock), 0, st, np, kin, K, idx,
                       scores, counts, batch, pool, cat, pool_count, stride, ctrl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SelectArgs a;
  a.ctx_len = nullptr;
  a.max_ctx = 0;
  a.max_pages = 0;
  a.p_begin = 0;
  a.p_end = 0;
  a.pool = pool;
  a.pool_count = pool_count;
  a.P = stride;              // pool rows are `stride` apart
  a.batch = batch;
  a.K = K;
  a.scores = cat;
  a.stride = stride;
  a.hist1 = ctrl;
  a.cand = reinterpret_cast<uint2*>(base + w.cand);
  a.chunk_counts = reinterpret_cast<uint32_t*>(base + w.counts);
  a.out_idx = out_idx;
  a.out_count = out_count;
  a.out_sel_scores = out_sel_scores;
  a.float_keys = values ? 1 : 0;
  return run_select(a, P, st);
}

// ------------------------------------------------------------------ LSE merge
// Block = one (sequence, head); thread t owns float4s t, t+64, ... of D.
// M = max_s lse_s; w_s = exp(lse_s - M) (0 for a part with no keys);
// out = sum_s w_s out_s / sum_s w_s; lse = M + ln sum_s w_s.
constexpr int kLseThreads = 64;

__global__ __launch_bounds__(kLseThreads) void lse_merge_kernel(
    int n_parts, int rows, int D, const float* __restrict__ outs, const float* __restrict__ lses,
    float* __restrict__ out, float* __restrict__ lse) {
  const int r = blockIdx.x;                     // b * H + h
  float M = -INFINITY;
  for (int s = 0; s < n_parts; ++s) M = fmaxf(M, lses[(size_t)s * rows + r]);
  const float Mu = M == -INFINITY ? 0.0f : M;
  float z = 0.0f;
  for (int s = 0; s < n_parts; ++s) {
    const float l = lses[(size_t)s * rows + r];
    z += l == -INFINITY ? 0.0f : expf(l - Mu);
  }
  const float iz = z > 0.0f ? 1.0f / z : 0.0f;
  for (int d4 = threadIdx.x; d4 < D / 4; d4 += kLseThreads) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < n_parts; ++s) {
      const float l = lses[(size_t)s * rows + r];
      if (l == -INFINITY) continue;
      const float ws = expf(l - Mu);
      const float4 v = reinterpret_cast<const float4*>(outs + ((size_t)s * rows + r) * D)[d4];
      acc.x += ws * v.x;
      acc.y += ws * v.y;
      acc.z += ws * v.z;
      acc.w += ws * v.w;
    }
    reinterpret_cast<float4*>(out + (size_t)r * D)[d4] =
        make_float4(acc.x * iz, acc.y * iz, acc.z * iz, acc.w * iz);
  }
  if (threadIdx.x == 0 && lse != nullptr) lse[r] = z > 0.0f ? Mu + logf(z) : -INFINITY;
}

hipError_t run_lse_merge(int n_parts, int batch, int H, int D, const float* outs,
                         const float* lses, float* out, float* lse, hipStream_t st) {
  const int rows = batch * H;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_merge_kernel, dim3(rows), dim3(kLseThreads), 0, st, n_parts, rows, D,
                     outs, lses, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
