// The per-token work of the FP4 append, shared by the standalone append
// kernel and the Full layer's fused append + score kernel.
//
// The FP4 main KV cache holds E2M1 elements with one E4M3 scale per 16
// channels (neodrop.ai V4.1-Flash report, 架构拆解 item 3); every layer keeps
// a 128-token window of recent tokens (zulogic "DeepSeek V4 1-Flash 架构拆解",
// section 4).  One token per D/8 lanes: each lane owns 8 consecutive
// channels (16 bytes of bf16), a lane pair owns one 16-channel group.
#pragma once

#include "common.h"

namespace csa2 {

struct AppendArgs {
  uint8_t* pages;
  const int32_t* page_table;
  int num_pages;
  int max_pages;
  int batch;
  int n_tokens;
  const uint16_t* x;          // [n][D] bf16 bits
  const int8_t* key;          // [n][Di] or NULL
  const int32_t* seq;
  const int32_t* pos;
  uint16_t* swa;              // [batch][128][D] or NULL
  // Fused with a Full layer's scoring: a token whose position is a scoring
  // candidate of its sequence (pos < min(L, max_ctx, 64*max_pages) - 128,
  // L = ctx_len[seq]) would race with the reads of that scoring, so it is
  // skipped.  NULL: no such restriction.
  const int32_t* ctx_len;
  int max_ctx;
};

template <int D>
__host__ __device__ constexpr int append_tokens_per_block() { return kBlock / (D / 8); }

// Lane l (< D/8) of token tok.  Every lane of a token takes the same early
// exits, so the group's lane-pair exchange stays inside live lanes.
template <int D, int DI>
__device__ __forceinline__ void append_token(const AppendArgs& a, int tok, int l) {
  constexpr PageLayout lay = page_layout(D, DI);
  if (tok >= a.n_tokens) return;
  const int b = a.seq[tok], p = a.pos[tok];
  bool ok = b >= 0 && b < a.batch && p >= 0 && p < a.max_pages * kPage;
  if (ok && a.ctx_len != nullptr) {
    int L = a.ctx_len[b];
    L = L < 0 ? 0 : L;
    L = L > a.max_ctx ? a.max_ctx : L;
    L = L > a.max_pages * kPage ? a.max_pages * kPage : L;
    ok = p >= L - kWindow;
  }
  const int pg = ok ? a.page_table[(size_t)b * a.max_pages + p / kPage] : -1;
  ok = ok && pg >= 0 && pg < a.num_pages;
  if (!ok) return;

  const uint4 raw = *reinterpret_cast<const uint4*>(a.x + (size_t)tok * D + l * 8);
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

  uint8_t* page = a.pages + (size_t)pg * lay.page_bytes;
  const int r = p % kPage;
  uint8_t* row = page + r * lay.row_bytes;
  *reinterpret_cast<uint32_t*>(row + l * 4) = packed;
  if ((l & 1) == 0) row[D / 2 + (l >> 1)] = (uint8_t)sc;
  if (a.key != nullptr && l < DI / 16) {
    const uint4 kv = *reinterpret_cast<const uint4*>(a.key + (size_t)tok * DI + l * 16);
    *reinterpret_cast<uint4*>(page + lay.keys_off + r * DI + l * 16) = kv;
  }
  if (a.swa != nullptr) {
    *reinterpret_cast<uint4*>(a.swa + ((size_t)b * kWindow + (p % kWindow)) * D + l * 8) = raw;
  }
}

// Block `blk` of an append grid: tokens blk*TPB .. blk*TPB + TPB - 1.
template <int D, int DI>
__device__ __forceinline__ void append_block(const AppendArgs& a, int blk) {
  constexpr int TPT = D / 8;
  append_token<D, DI>(a, blk * append_tokens_per_block<D>() + (int)threadIdx.x / TPT,
                      (int)threadIdx.x % TPT);
}

}  // namespace csa2
