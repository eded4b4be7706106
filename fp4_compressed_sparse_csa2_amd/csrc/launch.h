// Internal launch interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

struct CacheArgs {
  void* pages;
  const int32_t* page_table;
  int num_pages;
  int max_pages;
  int batch;
  int D;
  int Di;
};

hipError_t run_fill_zero(void* ws, size_t bytes, hipStream_t st);

struct AppendArgs;   // append.h
AppendArgs append_args(const CacheArgs& c, int n, const uint16_t* x, const int8_t* key,
                       const int32_t* seq, const int32_t* pos, uint16_t* swa);

// One selection call over per-sequence int32 scores, or float order keys
// (float_keys != 0; see select.hip).  The
// entries of sequence b are 0 <= i < n_b with n_b from ctx_len (candidates
// of a Full layer, i = position) or from pool_count (a Reindex layer's pool,
// output id = pool[b][i]).
struct SelectArgs {
  const int32_t* ctx_len;     // Full layer: candidates p_begin <= p < min(p_end, L_b - 128)
  int max_ctx;
  int max_pages;
  int p_begin;                // multiple of 64; entry i is position p_begin + i
  int p_end;
  const int32_t* pool;        // Reindex layer (non-NULL): [batch][P]
  const int32_t* pool_count;
  int P;
  int batch;
  int K;
  const int32_t* scores;      // [batch][stride]
  int stride;                 // multiple of 64
  uint32_t* hist1;            // [batch][kCtrlWords], zero outside a call
  uint2* cand;                // [batch][stride]
  uint32_t* chunk_counts;     // [batch][kMaxSelChunks]
  int32_t* out_idx;           // [batch][K]
  int32_t* out_count;         // [batch]
  int32_t* out_sel_scores;    // [batch][K] scores (float bits for float keys), or NULL
  int float_keys;             // 0: scores are int32 indexer scores; 1: value_key words
};
hipError_t run_select(const SelectArgs& a, int max_entries, hipStream_t st);

hipError_t run_quantize_append(const CacheArgs& c, int n, const uint16_t* x, const int8_t* key,
                               const int32_t* seq, const int32_t* pos, uint16_t* swa,
                               hipStream_t st);

// key_scales: NULL for int32 scores, else float [num_pages][64] per-token
// scales; the ranked values are then scaled_value(score, scale) and the
// score outputs carry float bits.
size_t index_topk_ws_bytes(int batch, int max_ctx, int K);
// append: NULL, or the tokens of a decode append (int32 scores only) fused
// into the scoring launch; tokens at scoring candidates are skipped.
hipError_t run_index_topk(const CacheArgs& c, const int32_t* ctx_len, int max_ctx,
                          const int8_t* q_idx, const float* key_scales, int K, int p_begin,
                          int p_end, int32_t* out_idx, int32_t* out_count, int32_t* out_scores,
                          int32_t* out_sel_scores, void* ws, hipStream_t st,
                          const AppendArgs* append = nullptr);

size_t reindex_ws_bytes(int batch, int P, int K);
hipError_t run_reindex(const CacheArgs& c, const int8_t* q_idx, const float* key_scales,
                       const int32_t* pool, const int32_t* pool_count, int P, int K,
                       int32_t* out_idx, int32_t* out_count, int32_t* out_scores, void* ws,
                       hipStream_t st);

// scale: float [n], or E4M3 bytes [n] when e4m3 (decoded exactly to fp32)
hipError_t run_store_key_scales(const CacheArgs& c, int n, const void* scale, bool e4m3,
                                const int32_t* seq, const int32_t* pos, float* key_scales,
                                hipStream_t st);

size_t topk_merge_ws_bytes(int batch, int n_parts, int K_in, int K);
// values: scores are float32 value bits (scaled indexer) instead of int32 scores
hipError_t run_topk_merge(int batch, int n_parts, int K_in, const int32_t* idx,
                          const int32_t* scores, const int32_t* counts, int K, int32_t* out_idx,
                          int32_t* out_count, int32_t* out_sel_scores, void* ws, hipStream_t st,
                          bool values = false);

// Contract-violation bits of csa2_validate_selection (the CSA2_SEL_* values).
constexpr uint32_t kBadLength = 1u, kBadCount = 2u, kBadPosition = 4u, kBadPage = 8u,
                   kNotAscending = 16u;
hipError_t run_validate_selection(const CacheArgs& c, const int32_t* ctx_len, const int32_t* idx,
                                  const int32_t* idx_count, int K, uint32_t* flags,
                                  hipStream_t st);

// Window-ring check bits of csa2_validate_window (the CSA2_WIN_* values).
constexpr uint32_t kWinNotF16 = 1u, kWinNotFinite = 2u;
hipError_t run_validate_window(const CacheArgs& c, const int32_t* ctx_len, const uint16_t* swa,
                               uint32_t* flags, hipStream_t st);

// One read of `bytes` (a multiple of 16) at src, XOR-folded into *sink.
hipError_t run_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);

hipError_t run_lse_merge(int n_parts, int batch, int H, int D, const float* outs,
                         const float* lses, float* out, float* lse, hipStream_t st);

size_t sparse_decode_ws_bytes(int batch, int H, int D, int K);
hipError_t run_sparse_decode(const CacheArgs& c, const int32_t* ctx_len, int H,
                             const uint16_t* q, float scale, const int32_t* idx,
                             const int32_t* idx_count, int K, const uint16_t* swa, float* out,
                             float* lse, void* ws, hipStream_t st);

}  // namespace csa2
