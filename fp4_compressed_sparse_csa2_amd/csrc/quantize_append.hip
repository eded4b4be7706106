// csa2_quantize_append: FP4 E2M1 / E4M3-per-16 pack-and-quantise append.
//
// The FP4 main KV cache holds E2M1 elements with one E4M3 scale per 16
// channels (neodrop.ai V4.1-Flash report, 架构拆解 item 3); every layer keeps
// a 128-token window of recent tokens (zulogic "DeepSeek V4 1-Flash 架构拆解",
// section 4).  One token per D/8 lanes: each lane owns 8 consecutive
// channels (16 bytes of bf16), a lane pair owns one 16-channel group.
#include "common.h"
#include "launch.h"

namespace csa2 {

template <int D, int DI>
__global__ __launch_bounds__(kBlock) void quantize_append_kernel(
    uint8_t* __restrict__ pages, const int32_t* __restrict__ page_table, int num_pages,
    int max_pages, int batch, int n_tokens, const uint16_t* __restrict__ x,
    const int8_t* __restrict__ key, const int32_t* __restrict__ seq,
    const int32_t* __restrict__ pos, uint16_t* __restrict__ swa) {
  constexpr int TPT = D / 8;                 // lanes per token
  constexpr int TPB = kBlock / TPT;          // tokens per block
  constexpr PageLayout lay = page_layout(D, DI);
  const int tok = blockIdx.x * TPB + threadIdx.x / TPT;
  const int l = threadIdx.x % TPT;
  if (tok >= n_tokens) return;               // uniform over the token's lanes

  const int b = seq[tok], p = pos[tok];
  bool ok = b >= 0 && b < batch && p >= 0 && p < max_pages * kPage;
  const int pg = ok ? page_table[(size_t)b * max_pages + p / kPage] : -1;
  ok = ok && pg >= 0 && pg < num_pages;
  if (!ok) return;                           // uniform over the token's lanes

  const uint4 raw = *reinterpret_cast<const uint4*>(x + (size_t)tok * D + l * 8);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};

  // group amax: |bf16| bit patterns order like their magnitudes
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    m = max(m, w[k] & 0x7FFFu);
    m = max(m, (w[k] >> 16) & 0x7FFFu);
  }
  m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));   // partner lane holds the other 8 channels
  const float amax = __uint_as_float(m << 16);
  const uint32_t sc = e4m3_code(amax / 6.0f);
  const float s = e4m3_value(sc);

  uint32_t packed = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t h = (w[c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
    const float xa = __uint_as_float((h & 0x7FFFu) << 16);
    const uint32_t code = e2m1_mag_code(xa, s) | ((h >> 15) << 3);
    packed |= code << (4 * c);
  }

  uint8_t* page = pages + (size_t)pg * lay.page_bytes;
  const int r = p % kPage;
  *reinterpret_cast<uint32_t*>(page + r * (D / 2) + l * 4) = packed;
  if ((l & 1) == 0) page[lay.scales_off + r * (D / 16) + (l >> 1)] = (uint8_t)sc;
  if (key != nullptr && l < DI / 16) {
    const uint4 kv = *reinterpret_cast<const uint4*>(key + (size_t)tok * DI + l * 16);
    *reinterpret_cast<uint4*>(page + lay.keys_off + r * DI + l * 16) = kv;
  }
  if (swa != nullptr) {
    *reinterpret_cast<uint4*>(swa + ((size_t)b * kWindow + (p % kWindow)) * D + l * 8) = raw;
  }
}

template <int D, int DI>
static hipError_t launch_qa(const CacheArgs& c, int n, const uint16_t* x, const int8_t* key,
                            const int32_t* seq, const int32_t* pos, uint16_t* swa,
                            hipStream_t st) {
  constexpr int TPB = kBlock / (D / 8);
  const int grid = (n + TPB - 1) / TPB;
  hipLaunchKernelGGL((quantize_append_kernel<D, DI>), dim3(grid), dim3(kBlock), 0, st,
                     (uint8_t*)c.pages, c.page_table, c.num_pages, c.max_pages, c.batch, n, x,
                     key, seq, pos, swa);
  return hipGetLastError();
}

hipError_t run_quantize_append(const CacheArgs& c, int n, const uint16_t* x, const int8_t* key,
                               const int32_t* seq, const int32_t* pos, uint16_t* swa,
                               hipStream_t st) {
  if (n == 0) return hipSuccess;
#define QA_CASE(D_, DI_) \
  if (c.D == D_ && c.Di == DI_) return launch_qa<D_, DI_>(c, n, x, key, seq, pos, swa, st);
  QA_CASE(128, 64) QA_CASE(128, 128) QA_CASE(256, 64) QA_CASE(256, 128)
  QA_CASE(512, 64) QA_CASE(512, 128)
#undef QA_CASE
  return hipErrorInvalidValue;
}

// Key scales of appended tokens: scale[i] goes to key_scales[pg][p % 64] for
// token i at (seq[i], pos[i]) with pg its page; tokens that do not map to a
// page are skipped, as in the append above.
__global__ __launch_bounds__(kBlock) void store_key_scales_kernel(
    const int32_t* __restrict__ page_table, int num_pages, int max_pages, int batch, int n,
    const float* __restrict__ scale, const int32_t* __restrict__ seq,
    const int32_t* __restrict__ pos, float* __restrict__ key_scales) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  const int b = seq[i], p = pos[i];
  if (b < 0 || b >= batch || p < 0 || p >= max_pages * kPage) return;
  const int pg = page_table[(size_t)b * max_pages + p / kPage];
  if (pg < 0 || pg >= num_pages) return;
  key_scales[(size_t)pg * kPage + p % kPage] = scale[i];
}

hipError_t run_store_key_scales(const CacheArgs& c, int n, const float* scale,
                                const int32_t* seq, const int32_t* pos, float* key_scales,
                                hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(store_key_scales_kernel, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0,
                     st, c.page_table, c.num_pages, c.max_pages, c.batch, n, scale, seq, pos,
                     key_scales);
  return hipGetLastError();
}

}  // namespace csa2
