// The C ABI (include/csa2.h): host-side argument validation, then kernel
// launches on the caller's stream.  No allocation, no synchronisation, no
// reads of device memory on the host.
#include "csa2.h"

#include <atomic>
#include <mutex>

#include "append.h"
#include "common.h"
#include "launch.h"

namespace csa2 {

__global__ __launch_bounds__(kBlock) void fill_zero_kernel(uint4* p, size_t n16, uint8_t* tail,
                                                            size_t ntail) {
  const size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0u, 0u, 0u, 0u);
  if (i < ntail) tail[i] = 0;
}

hipError_t run_fill_zero(void* ws, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  const size_t work = n16 > ntail ? n16 : ntail;
  const size_t blocks = (work + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st,
                     static_cast<uint4*>(ws), n16, static_cast<uint8_t*>(ws) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace csa2

using csa2::CacheArgs;

namespace {

bool supported_d(int D) { return D == 128 || D == 256 || D == 512; }
bool supported_di(int Di) { return Di == 64 || Di == 128; }

// Common cache checks: returns CSA2_OK or an error code.
int check_cache(const csa2_cache* c) {
  if (c == nullptr || c->pages == nullptr || c->page_table == nullptr) return CSA2_E_NULL;
  if (!supported_d(c->head_dim) || !supported_di(c->idx_dim)) return CSA2_E_UNSUPPORTED;
  if (c->batch < 1 || c->num_pages < 1 || c->max_pages_per_seq < 1) return CSA2_E_SHAPE;
  if ((int64_t)c->max_pages_per_seq * CSA2_PAGE_TOKENS > (int64_t)1 << 30) return CSA2_E_SHAPE;
  return CSA2_OK;
}

CacheArgs args_of(const csa2_cache* c) {
  return CacheArgs{c->pages, c->page_table, c->num_pages, c->max_pages_per_seq,
                   c->batch, c->head_dim, c->idx_dim};
}

int status_of(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_E_HIP; }

constexpr int32_t kMaxK = 65536;
constexpr int32_t kMaxCtx = 1 << 24;
constexpr int32_t kMaxParts = 64;

// Scratch of csa2_sparse_decode_noalloc: one copy per device, alive until the
// process ends.  On the host `scratch` names a host-side stand-in, not device
// memory, so host code only ever passes the address hipGetSymbolAddress
// returns for the current device.
constexpr size_t kNoAllocScratch = CSA2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratch];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's scratch address, looked up on its first use.
hipError_t device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t csa2_page_bytes(int32_t head_dim, int32_t idx_dim) {
  if (!supported_d(head_dim) || !supported_di(idx_dim)) return 0;
  return (size_t)csa2::page_layout(head_dim, idx_dim).page_bytes;
}

const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "CSA2_OK";
    case CSA2_E_NULL: return "CSA2_E_NULL: a required pointer is NULL";
    case CSA2_E_SHAPE: return "CSA2_E_SHAPE: a size or count is out of range";
    case CSA2_E_UNSUPPORTED: return "CSA2_E_UNSUPPORTED: head_dim/idx_dim/heads not supported";
    case CSA2_E_WORKSPACE: return "CSA2_E_WORKSPACE: workspace NULL or too small";
    case CSA2_E_HIP: return "CSA2_E_HIP: a kernel launch failed";
    case CSA2_E_SCRATCH:
      return "CSA2_E_SCRATCH: the call needs more than the fixed allocation-free scratch";
    default: return "unknown csa2 status";
  }
}

int csa2_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return CSA2_OK;
  if (src == nullptr || sink == nullptr) return CSA2_E_NULL;
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0) return CSA2_E_SHAPE;
  return status_of(csa2::run_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

int csa2_workspace_init(void* ws, size_t bytes, void* stream) {
  if (bytes > 0 && ws == nullptr) return CSA2_E_NULL;
  return status_of(csa2::run_fill_zero(ws, bytes, static_cast<hipStream_t>(stream)));
}

int csa2_quantize_append(const csa2_cache* cache, int32_t n_tokens, const uint16_t* x,
                         const int8_t* key_i8, const int32_t* seq, const int32_t* pos,
                         uint16_t* swa, void* stream) {
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (n_tokens < 0) return CSA2_E_SHAPE;
  if (n_tokens > 0 && (x == nullptr || seq == nullptr || pos == nullptr)) return CSA2_E_NULL;
  return status_of(csa2::run_quantize_append(args_of(cache), n_tokens, x, key_i8, seq, pos, swa,
                                             static_cast<hipStream_t>(stream)));
}

size_t csa2_index_topk_workspace_size(int32_t batch, int32_t max_ctx, int32_t K) {
  if (batch < 1 || max_ctx < 0 || max_ctx > kMaxCtx || K < 0 || K > kMaxK) return 0;
  return csa2::index_topk_ws_bytes(batch, max_ctx, K);
}

int csa2_index_topk(const csa2_cache* cache, const int32_t* ctx_len, int32_t max_ctx,
                    const int8_t* q_idx, int32_t K, int32_t* out_idx, int32_t* out_count,
                    int32_t* out_scores, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (ctx_len == nullptr || q_idx == nullptr || out_count == nullptr) return CSA2_E_NULL;
  if (K > 0 && out_idx == nullptr) return CSA2_E_NULL;
  if (K < 0 || K > kMaxK || max_ctx < 0 || max_ctx > kMaxCtx) return CSA2_E_SHAPE;
  const size_t need = csa2::index_topk_ws_bytes(cache->batch, max_ctx, K);
  if (ws == nullptr || ws_bytes < need) return CSA2_E_WORKSPACE;
  return status_of(csa2::run_index_topk(args_of(cache), ctx_len, max_ctx, q_idx, nullptr, K, 0,
                                        kMaxCtx, out_idx, out_count, out_scores, nullptr, ws,
                                        static_cast<hipStream_t>(stream)));
}

int csa2_append_index_topk(const csa2_cache* cache, int32_t n_tokens, const uint16_t* x,
                           const int8_t* key_i8, const int32_t* seq, const int32_t* pos,
                           uint16_t* swa, const int32_t* ctx_len, int32_t max_ctx,
                           const int8_t* q_idx, int32_t K, int32_t* out_idx, int32_t* out_count,
                           int32_t* out_scores, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (n_tokens < 0) return CSA2_E_SHAPE;
  if (n_tokens > 0 && (x == nullptr || seq == nullptr || pos == nullptr)) return CSA2_E_NULL;
  if (ctx_len == nullptr || q_idx == nullptr || out_count == nullptr) return CSA2_E_NULL;
  if (K > 0 && out_idx == nullptr) return CSA2_E_NULL;
  if (K < 0 || K > kMaxK || max_ctx < 0 || max_ctx > kMaxCtx) return CSA2_E_SHAPE;
  const size_t need = csa2::index_topk_ws_bytes(cache->batch, max_ctx, K);
  if (ws == nullptr || ws_bytes < need) return CSA2_E_WORKSPACE;
  const CacheArgs c = args_of(cache);
  const csa2::AppendArgs ap = csa2::append_args(c, n_tokens, x, key_i8, seq, pos, swa);
  return status_of(csa2::run_index_topk(c, ctx_len, max_ctx, q_idx, nullptr, K, 0, kMaxCtx,
                                        out_idx, out_count, out_scores, nullptr, ws,
                                        static_cast<hipStream_t>(stream), &ap));
}

static int store_key_scales(const csa2_cache* cache, int32_t n_tokens, const void* scale,
                            bool e4m3, const int32_t* seq, const int32_t* pos, float* key_scales,
                            void* stream) {
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (n_tokens < 0) return CSA2_E_SHAPE;
  if (n_tokens > 0 && (scale == nullptr || seq == nullptr || pos == nullptr ||
                       key_scales == nullptr))
    return CSA2_E_NULL;
  return status_of(csa2::run_store_key_scales(args_of(cache), n_tokens, scale, e4m3, seq, pos,
                                              key_scales, static_cast<hipStream_t>(stream)));
}

int csa2_store_key_scales(const csa2_cache* cache, int32_t n_tokens, const float* scale,
                          const int32_t* seq, const int32_t* pos, float* key_scales,
                          void* stream) {
  return store_key_scales(cache, n_tokens, scale, false, seq, pos, key_scales, stream);
}

int csa2_store_key_scales_e4m3(const csa2_cache* cache, int32_t n_tokens,
                               const uint8_t* scale_e4m3, const int32_t* seq, const int32_t* pos,
                               float* key_scales, void* stream) {
  return store_key_scales(cache, n_tokens, scale_e4m3, true, seq, pos, key_scales, stream);
}

int csa2_index_topk_scaled(const csa2_cache* cache, const int32_t* ctx_len, int32_t max_ctx,
                           const int8_t* q_idx, const float* key_scales, int32_t K,
                           int32_t* out_idx, int32_t* out_count, float* out_values,
                           float* out_sel_values, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (ctx_len == nullptr || q_idx == nullptr || key_scales == nullptr || out_count == nullptr)
    return CSA2_E_NULL;
  if (K > 0 && out_idx == nullptr) return CSA2_E_NULL;
  if (K < 0 || K > kMaxK || max_ctx < 0 || max_ctx > kMaxCtx) return CSA2_E_SHAPE;
  const size_t need = csa2::index_topk_ws_bytes(cache->batch, max_ctx, K);
  if (ws == nullptr || ws_bytes < need) return CSA2_E_WORKSPACE;
  return status_of(csa2::run_index_topk(args_of(cache), ctx_len, max_ctx, q_idx, key_scales, K,
                                        0, kMaxCtx, out_idx, out_count,
                                        reinterpret_cast<int32_t*>(out_values),
                                        reinterpret_cast<int32_t*>(out_sel_values), ws,
                                        static_cast<hipStream_t>(stream)));
}

int csa2_index_topk_range(const csa2_cache* cache, const int32_t* ctx_len, int32_t max_ctx,
                          const int8_t* q_idx, int32_t K, int32_t p_begin, int32_t p_end,
                          int32_t* out_idx, int32_t* out_count, int32_t* out_sel_scores,
                          void* ws, size_t ws_bytes, void* stream) {
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (ctx_len == nullptr || q_idx == nullptr || out_count == nullptr) return CSA2_E_NULL;
  if (K > 0 && out_idx == nullptr) return CSA2_E_NULL;
  if (K < 0 || K > kMaxK || max_ctx < 0 || max_ctx > kMaxCtx) return CSA2_E_SHAPE;
  if (p_begin < 0 || p_begin % CSA2_PAGE_TOKENS != 0 || p_end < p_begin) return CSA2_E_SHAPE;
  const size_t need = csa2::index_topk_ws_bytes(cache->batch, max_ctx, K);
  if (ws == nullptr || ws_bytes < need) return CSA2_E_WORKSPACE;
  return status_of(csa2::run_index_topk(args_of(cache), ctx_len, max_ctx, q_idx, nullptr, K,
                                        p_begin, p_end, out_idx, out_count, nullptr,
                                        out_sel_scores, ws, static_cast<hipStream_t>(stream)));
}

size_t csa2_topk_merge_workspace_size(int32_t batch, int32_t n_parts, int32_t K_in, int32_t K) {
  if (batch < 1 || n_parts < 1 || n_parts > kMaxParts || K_in < 0 || K_in > kMaxK || K < 0 ||
      K > kMaxK || (int64_t)n_parts * K_in > kMaxK * 8 || K > n_parts * K_in)
    return 0;
  return csa2::topk_merge_ws_bytes(batch, n_parts, K_in, K);
}

static int topk_merge(int32_t batch, int32_t n_parts, int32_t K_in, const int32_t* idx,
                      const void* scores, const int32_t* counts, int32_t K, int32_t* out_idx,
                      int32_t* out_count, void* out_sel_scores, void* ws, size_t ws_bytes,
                      void* stream, bool values) {
  if (counts == nullptr || out_count == nullptr) return CSA2_E_NULL;
  if (K_in > 0 && (idx == nullptr || scores == nullptr)) return CSA2_E_NULL;
  if (K > 0 && out_idx == nullptr) return CSA2_E_NULL;
  if (batch < 1 || n_parts < 1 || n_parts > kMaxParts || K_in < 0 || K_in > kMaxK || K < 0 ||
      K > kMaxK || (int64_t)n_parts * K_in > kMaxK * 8 || K > n_parts * K_in)
    return CSA2_E_SHAPE;
  const size_t need = csa2::topk_merge_ws_bytes(batch, n_parts, K_in, K);
  if (ws == nullptr || ws_bytes < need) return CSA2_E_WORKSPACE;
  return status_of(csa2::run_topk_merge(batch, n_parts, K_in, idx,
                                        static_cast<const int32_t*>(scores), counts, K, out_idx,
                                        out_count, static_cast<int32_t*>(out_sel_scores), ws,
                                        static_cast<hipStream_t>(stream), values));
}

int csa2_topk_merge(int32_t batch, int32_t n_parts, int32_t K_in, const int32_t* idx,
                    const int32_t* scores, const int32_t* counts, int32_t K, int32_t* out_idx,
                    int32_t* out_count, int32_t* out_sel_scores, void* ws, size_t ws_bytes,
                    void* stream) {
  return topk_merge(batch, n_parts, K_in, idx, scores, counts, K, out_idx, out_count,
                    out_sel_scores, ws, ws_bytes, stream, false);
}

int csa2_topk_merge_values(int32_t batch, int32_t n_parts, int32_t K_in, const int32_t* idx,
                           const float* values, const int32_t* counts, int32_t K,
                           int32_t* out_idx, int32_t* out_count, float* out_sel_values, void* ws,
                           size_t ws_bytes, void* stream) {
  return topk_merge(batch, n_parts, K_in, idx, values, counts, K, out_idx, out_count,
                    out_sel_values, ws, ws_bytes, stream, true);
}

int csa2_validate_selection(const csa2_cache* cache, const int32_t* ctx_len,
                            const int32_t* idx, const int32_t* idx_count, int32_t K,
                            uint32_t* flags, void* stream) {
  static_assert(csa2::kBadLength == CSA2_SEL_BAD_LENGTH && csa2::kBadCount == CSA2_SEL_BAD_COUNT &&
                    csa2::kBadPosition == CSA2_SEL_BAD_POSITION &&
                    csa2::kBadPage == CSA2_SEL_BAD_PAGE &&
                    csa2::kNotAscending == CSA2_SEL_NOT_ASCENDING,
                "violation bits");
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (ctx_len == nullptr || idx_count == nullptr || flags == nullptr) return CSA2_E_NULL;
  if (K > 0 && idx == nullptr) return CSA2_E_NULL;
  if (K < 0 || K > kMaxK) return CSA2_E_SHAPE;
  return status_of(csa2::run_validate_selection(args_of(cache), ctx_len, idx, idx_count, K, flags,
                                                static_cast<hipStream_t>(stream)));
}

int csa2_validate_window(const csa2_cache* cache, const int32_t* ctx_len, const uint16_t* swa,
                         uint32_t* flags, void* stream) {
  static_assert(csa2::kWinNotF16 == CSA2_WIN_NOT_F16 && csa2::kWinNotFinite == CSA2_WIN_NOT_FINITE,
                "window bits");
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (ctx_len == nullptr || swa == nullptr || flags == nullptr) return CSA2_E_NULL;
  return status_of(csa2::run_validate_window(args_of(cache), ctx_len, swa, flags,
                                             static_cast<hipStream_t>(stream)));
}

int csa2_lse_merge(int32_t n_parts, int32_t batch, int32_t H, int32_t head_dim,
                   const float* outs, const float* lses, float* out, float* lse, void* stream) {
  if (outs == nullptr || lses == nullptr || out == nullptr) return CSA2_E_NULL;
  if (n_parts < 1 || n_parts > kMaxParts || batch < 1 || H < 1 || H > 128) return CSA2_E_SHAPE;
  if (!supported_d(head_dim)) return CSA2_E_UNSUPPORTED;
  return status_of(csa2::run_lse_merge(n_parts, batch, H, head_dim, outs, lses, out, lse,
                                       static_cast<hipStream_t>(stream)));
}

size_t csa2_reindex_workspace_size(int32_t batch, int32_t P, int32_t K) {
  if (batch < 1 || P < 0 || P > kMaxK || K < 0 || K > P) return 0;
  return csa2::reindex_ws_bytes(batch, P, K);
}

int csa2_reindex(const csa2_cache* cache, const int8_t* q_idx, const int32_t* pool,
                 const int32_t* pool_count, int32_t P, int32_t K, int32_t* out_idx,
                 int32_t* out_count, int32_t* out_scores, void* ws, size_t ws_bytes,
                 void* stream) {
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (q_idx == nullptr || pool_count == nullptr || out_count == nullptr) return CSA2_E_NULL;
  if ((P > 0 && pool == nullptr) || (K > 0 && out_idx == nullptr)) return CSA2_E_NULL;
  if (P < 0 || P > kMaxK || K < 0 || K > P) return CSA2_E_SHAPE;
  const size_t need = csa2::reindex_ws_bytes(cache->batch, P, K);
  if (ws == nullptr || ws_bytes < need) return CSA2_E_WORKSPACE;
  return status_of(csa2::run_reindex(args_of(cache), q_idx, nullptr, pool, pool_count, P, K,
                                     out_idx, out_count, out_scores, ws,
                                     static_cast<hipStream_t>(stream)));
}

int csa2_index_topk_range_scaled(const csa2_cache* cache, const int32_t* ctx_len,
                                 int32_t max_ctx, const int8_t* q_idx, const float* key_scales,
                                 int32_t K, int32_t p_begin, int32_t p_end, int32_t* out_idx,
                                 int32_t* out_count, float* out_sel_values, void* ws,
                                 size_t ws_bytes, void* stream) {
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (ctx_len == nullptr || q_idx == nullptr || key_scales == nullptr || out_count == nullptr)
    return CSA2_E_NULL;
  if (K > 0 && out_idx == nullptr) return CSA2_E_NULL;
  if (K < 0 || K > kMaxK || max_ctx < 0 || max_ctx > kMaxCtx) return CSA2_E_SHAPE;
  if (p_begin < 0 || p_begin % CSA2_PAGE_TOKENS != 0 || p_end < p_begin) return CSA2_E_SHAPE;
  const size_t need = csa2::index_topk_ws_bytes(cache->batch, max_ctx, K);
  if (ws == nullptr || ws_bytes < need) return CSA2_E_WORKSPACE;
  return status_of(csa2::run_index_topk(args_of(cache), ctx_len, max_ctx, q_idx, key_scales, K,
                                        p_begin, p_end, out_idx, out_count, nullptr,
                                        reinterpret_cast<int32_t*>(out_sel_values), ws,
                                        static_cast<hipStream_t>(stream)));
}

int csa2_reindex_scaled(const csa2_cache* cache, const int8_t* q_idx, const float* key_scales,
                        const int32_t* pool, const int32_t* pool_count, int32_t P, int32_t K,
                        int32_t* out_idx, int32_t* out_count, float* out_values, void* ws,
                        size_t ws_bytes, void* stream) {
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (q_idx == nullptr || key_scales == nullptr || pool_count == nullptr || out_count == nullptr)
    return CSA2_E_NULL;
  if ((P > 0 && pool == nullptr) || (K > 0 && out_idx == nullptr)) return CSA2_E_NULL;
  if (P < 0 || P > kMaxK || K < 0 || K > P) return CSA2_E_SHAPE;
  const size_t need = csa2::reindex_ws_bytes(cache->batch, P, K);
  if (ws == nullptr || ws_bytes < need) return CSA2_E_WORKSPACE;
  return status_of(csa2::run_reindex(args_of(cache), q_idx, key_scales, pool, pool_count, P, K,
                                     out_idx, out_count, reinterpret_cast<int32_t*>(out_values),
                                     ws, static_cast<hipStream_t>(stream)));
}

size_t csa2_sparse_decode_workspace_size(int32_t batch, int32_t H, int32_t head_dim, int32_t K) {
  if (batch < 1 || H < 16 || H > 128 || H % 16 != 0 || !supported_d(head_dim) || K < 0 ||
      K > kMaxK)
    return 0;
  return csa2::sparse_decode_ws_bytes(batch, H, head_dim, K);
}

int csa2_sparse_decode(const csa2_cache* cache, const int32_t* ctx_len, int32_t H,
                       const uint16_t* q, float softmax_scale, const int32_t* idx,
                       const int32_t* idx_count, int32_t K, const uint16_t* swa, float* out,
                       float* lse, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (ctx_len == nullptr || q == nullptr || idx_count == nullptr || out == nullptr)
    return CSA2_E_NULL;
  if (K > 0 && idx == nullptr) return CSA2_E_NULL;
  if (H < 16 || H > 128 || H % 16 != 0) return CSA2_E_UNSUPPORTED;
  if (K < 0 || K > kMaxK) return CSA2_E_SHAPE;
  const size_t need = csa2::sparse_decode_ws_bytes(cache->batch, H, cache->head_dim, K);
  if (ws == nullptr || ws_bytes < need) return CSA2_E_WORKSPACE;
  return status_of(csa2::run_sparse_decode(args_of(cache), ctx_len, H, q, softmax_scale, idx,
                                           idx_count, K, swa, out, lse, ws,
                                           static_cast<hipStream_t>(stream)));
}

int csa2_sparse_decode_noalloc(const csa2_cache* cache, const int32_t* ctx_len, int32_t H,
                               const uint16_t* q, float softmax_scale, const int32_t* idx,
                               const int32_t* idx_count, int32_t K, const uint16_t* swa,
                               float* out, float* lse, void* stream) {
  int st = check_cache(cache);
  if (st != CSA2_OK) return st;
  if (ctx_len == nullptr || q == nullptr || idx_count == nullptr || out == nullptr)
    return CSA2_E_NULL;
  if (K > 0 && idx == nullptr) return CSA2_E_NULL;
  if (H < 16 || H > 128 || H % 16 != 0) return CSA2_E_UNSUPPORTED;
  if (K < 0 || K > kMaxK) return CSA2_E_SHAPE;
  if (csa2::sparse_decode_ws_bytes(cache->batch, H, cache->head_dim, K) > kNoAllocScratch)
    return CSA2_E_SCRATCH;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (hs != nullptr) {
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(hs, &sdev) != hipSuccess)
      return CSA2_E_HIP;
    if (cur != sdev) return CSA2_E_UNSUPPORTED;
  }
  void* ws = nullptr;
  if (device_scratch(&ws) != hipSuccess) return CSA2_E_HIP;
  return status_of(csa2::run_sparse_decode(args_of(cache), ctx_len, H, q, softmax_scale, idx,
                                           idx_count, K, swa, out, lse, ws, hs));
}

}  // extern "C"
