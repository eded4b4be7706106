// csa2_validate_selection: a debug-time check of the device-side contract of
// csa2_sparse_decode's inputs, which the kernels themselves only survive
// (they skip what is out of range without touching memory outside the
// buffers).  One block per sequence; every read is bounds-checked.
#include "common.h"
#include "launch.h"

namespace csa2 {

__global__ __launch_bounds__(kBlock) void validate_selection_kernel(
    const int32_t* __restrict__ page_table, int num_pages, int max_pages,
    const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ idx_count, int K, uint32_t* __restrict__ flags) {
  __shared__ uint32_t f;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) f = 0u;
  __syncthreads();
  uint32_t mine = 0;
  const int L = ctx_len[b];
  if (L < 0 || L > max_pages * kPage) mine |= kBadLength;
  const int Lc = L < 0 ? 0 : (L > max_pages * kPage ? max_pages * kPage : L);
  const int n = Lc > kWindow ? Lc - kWindow : 0;          // candidate positions [0, n)
  int c = idx_count[b];
  if (c < 0 || c > K) mine |= kBadCount;
  c = c < 0 ? 0 : (c > K ? K : c);
  const int32_t* row = idx + (size_t)b * K;
  for (int j = threadIdx.x; j < c; j += kBlock) {
    const int p = row[j];
    if (p < 0 || p >= n) {
      mine |= kBadPosition;
      continue;
    }
    const int pg = page_table[(size_t)b * max_pages + p / kPage];
    if (pg < 0 || pg >= num_pages) mine |= kBadPage;
    if (j > 0 && row[j - 1] >= p) mine |= kNotAscending;
  }
  if (mine) atomicOr(&f, mine);
  __syncthreads();
  if (threadIdx.x == 0) flags[b] = f;
}

// One block per sequence: every live window slot (the slots of positions
// [max(0, L - 128), L)) is converted bf16 -> f32 -> f16 -> f32; a value that
// does not come back unchanged is outside what the decode's f16 window
// operands hold exactly.
__global__ __launch_bounds__(kBlock) void validate_window_kernel(
    int max_pages, const int32_t* __restrict__ ctx_len, const uint16_t* __restrict__ swa, int D,
    uint32_t* __restrict__ flags) {
  __shared__ uint32_t f;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) f = 0u;
  __syncthreads();
  uint32_t mine = 0;
  int L = ctx_len[b];
  L = L < 0 ? 0 : (L > max_pages * kPage ? max_pages * kPage : L);
  const int live = L < kWindow ? L : kWindow;              // slots [0, live) hold tokens
  const uint16_t* ring = swa + (size_t)b * kWindow * D;
  for (int i = threadIdx.x; i < live * D; i += kBlock) {
    const float v = __uint_as_float((uint32_t)ring[i] << 16);
    if (!__builtin_isfinite(v)) {
      mine |= kWinNotFinite;
    } else if ((float)(_Float16)v != v) {
      mine |= kWinNotF16;
    }
  }
  if (mine) atomicOr(&f, mine);
  __syncthreads();
  if (threadIdx.x == 0) flags[b] = f;
}

hipError_t run_validate_window(const CacheArgs& c, const int32_t* ctx_len, const uint16_t* swa,
                               uint32_t* flags, hipStream_t st) {
  hipLaunchKernelGGL(validate_window_kernel, dim3(c.batch), dim3(kBlock), 0, st, c.max_pages,
                     ctx_len, swa, c.D, flags);
  return hipGetLastError();
}

hipError_t run_validate_selection(const CacheArgs& c, const int32_t* ctx_len, const int32_t* idx,
                                  const int32_t* idx_count, int K, uint32_t* flags,
                                  hipStream_t st) {
  hipLaunchKernelGGL(validate_selection_kernel, dim3(c.batch), dim3(kBlock), 0, st, c.page_table,
                     c.num_pages, c.max_pages, ctx_len, idx, idx_count, K, flags);
  return hipGetLastError();
}

}  // namespace csa2
