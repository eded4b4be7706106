// csa2_stream_read: one pass of 16-byte non-temporal loads over a device
// buffer, the in-run reference for what a read-only kernel reaches on this
// HBM (the method's calls read far more than they write).  Each block reads
// one contiguous 16 KB run (four loads per thread, 1 KB per wave
// instruction) and exits: on MI355X that reaches about 7 TB/s over 2 GiB,
// where a grid-stride loop over the same buffer stays near 6.1.  The loads
// are folded into one XOR word so that none of them can be dropped.
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kReadUnroll = 4;          // 16-byte loads in flight per thread
constexpr size_t kReadRun = (size_t)kBlock * kReadUnroll;   // 16-byte units per block

__global__ __launch_bounds__(kBlock) void stream_read_kernel(const u32x4* __restrict__ src,
                                                             size_t n16, uint32_t* sink) {
  const size_t base = (size_t)blockIdx.x * kReadRun + threadIdx.x;
  u32x4 v[kReadUnroll];
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) {
    const size_t i = base + (size_t)u * kBlock;
    v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m);
  if ((threadIdx.x & 63) == 0 && x != 0u) atomicXor(sink, x);
}

hipError_t run_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t blocks = (n16 + kReadRun - 1) / kReadRun;
  if (blocks > 0x7FFFFFFFu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st,
                     static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace csa2
