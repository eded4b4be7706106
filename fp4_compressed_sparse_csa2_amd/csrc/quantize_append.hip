// csa2_quantize_append: FP4 E2M1 / E4M3-per-16 pack-and-quantise append
// (the per-token work is append_token in append.h).
#include "append.h"
#include "common.h"
#include "launch.h"

namespace csa2 {

template <int D, int DI>
__global__ __launch_bounds__(kBlock) void quantize_append_kernel(AppendArgs a) {
  append_block<D, DI>(a, blockIdx.x);
}

template <int D, int DI>
static hipError_t launch_qa(const AppendArgs& a, hipStream_t st) {
  const int grid = (a.n_tokens + append_tokens_per_block<D>() - 1) / append_tokens_per_block<D>();
  hipLaunchKernelGGL((quantize_append_kernel<D, DI>), dim3(grid), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

AppendArgs append_args(const CacheArgs& c, int n, const uint16_t* x, const int8_t* key,
                       const int32_t* seq, const int32_t* pos, uint16_t* swa) {
  AppendArgs a;
  a.pages = static_cast<uint8_t*>(c.pages);
  a.page_table = c.page_table;
  a.num_pages = c.num_pages;
  a.max_pages = c.max_pages;
  a.batch = c.batch;
  a.n_tokens = n;
  a.x = x;
  a.key = key;
  a.seq = seq;
  a.pos = pos;
  a.swa = swa;
  a.ctx_len = nullptr;
  a.max_ctx = 0;
  return a;
}

hipError_t run_quantize_append(const CacheArgs& c, int n, const uint16_t* x, const int8_t* key,
                               const int32_t* seq, const int32_t* pos, uint16_t* swa,
                               hipStream_t st) {
  if (n == 0) return hipSuccess;
  const AppendArgs a = append_args(c, n, x, key, seq, pos, swa);
#define QA_CASE(D_, DI_) \
  if (c.D == D_ && c.Di == DI_) return launch_qa<D_, DI_>(a, st);
  QA_CASE(128, 64) QA_CASE(128, 128) QA_CASE(256, 64) QA_CASE(256, 128)
  QA_CASE(512, 64) QA_CASE(512, 128)
#undef QA_CASE
  return hipErrorInvalidValue;
}

// Key scales of appended tokens: scale[i] (fp32, or an E4M3 byte decoded
// exactly) goes to key_scales[pg][p % 64] for token i at (seq[i], pos[i])
// with pg its page; tokens that do not map to a page are skipped, as in the
// append above.
template <bool E4M3>
__global__ __launch_bounds__(kBlock) void store_key_scales_kernel(
    const int32_t* __restrict__ page_table, int num_pages, int max_pages, int batch, int n,
    const void* __restrict__ scale, const int32_t* __restrict__ seq,
    const int32_t* __restrict__ pos, float* __restrict__ key_scales) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  const int b = seq[i], p = pos[i];
  if (b < 0 || b >= batch || p < 0 || p >= max_pages * kPage) return;
  const int pg = page_table[(size_t)b * max_pages + p / kPage];
  if (pg < 0 || pg >= num_pages) return;
  const float s = E4M3 ? e4m3_signed_value(static_cast<const uint8_t*>(scale)[i])
                       : static_cast<const float*>(scale)[i];
  key_scales[(size_t)pg * kPage + p % kPage] = s;
}

hipError_t run_store_key_scales(const CacheArgs& c, int n, const void* scale, bool e4m3,
                                const int32_t* seq, const int32_t* pos, float* key_scales,
                                hipStream_t st) {
  if (n == 0) return hipSuccess;
  const dim3 grid((n + kBlock - 1) / kBlock);
  if (e4m3)
    hipLaunchKernelGGL(store_key_scales_kernel<true>, grid, dim3(kBlock), 0, st, c.page_table,
                       c.num_pages, c.max_pages, c.batch, n, scale, seq, pos, key_scales);
  else
    hipLaunchKernelGGL(store_key_scales_kernel<false>, grid, dim3(kBlock), 0, st, c.page_table,
                       c.num_pages, c.max_pages, c.batch, n, scale, seq, pos, key_scales);
  return hipGetLastError();
}

}  // namespace csa2
