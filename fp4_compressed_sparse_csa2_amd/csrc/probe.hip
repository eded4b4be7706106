// csa2_stream_read: one pass of 16-byte non-temporal loads over a device
// buffer, the in-run reference for what a read-only kernel reaches on this
// HBM (the method's calls read far more than they write).  The loads are
// folded into one XOR word so that none of them can be dropped.
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kReadUnroll = 4;          // 16-byte loads in flight per thread

__global__ __launch_bounds__(kBlock) void stream_read_kernel(const u32x4* __restrict__ src,
                                                             size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kBlock;
  size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m);
  if ((threadIdx.x & 63) == 0 && x != 0u) atomicXor(sink, x);
}

hipError_t run_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  constexpr size_t kMaxBlocks = 256 * 16;           // 16 blocks per CU
  size_t blocks = (n16 + (size_t)kBlock * kReadUnroll - 1) / ((size_t)kBlock * kReadUnroll);
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st,
                     static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace csa2
