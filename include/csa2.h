/*
 * csa2.h -- C ABI of the CSA2 sparse-decode library for MI355X (gfx950).
 *
 * The decode step of compressed sparse attention over a shared FP4 global KV
 * cache, in four calls:
 *
 *   csa2_quantize_append  write tokens into the FP4 cache (+ indexer keys,
 *                         + the layer's 128-token window ring)
 *   csa2_index_topk       Full layer: int8 indexer scores over every cached
 *                         position outside the window, deterministic Top-K
 *   csa2_reindex          Reindex layer: rescore the Full layer's candidate
 *                         pool with this layer's own indexer query, Top-K'
 *   csa2_sparse_decode    attention of H query heads over the selected FP4
 *                         rows (dequantised on the fly) merged with the
 *                         layer's bf16 window; a Reuse layer calls it with
 *                         the indices of the layer it reuses
 *
 * Sources.  Layers are statically Full, Reindex or Reuse and share the main
 * KV and the indexer keys, reusing Top-K indices across layers; deeper
 * indexers refilter only the pool built by the first Full layer (neodrop.ai,
 * "DeepSeek 首次公开 V4.1-Flash 技术报告", section 架构拆解 item 2; zulogic,
 * "DeepSeek V4 1-Flash 架构拆解", section 3 mode table).  The main KV is FP4
 * E2M1 with one E4M3 scale per 16 channels (neodrop.ai, same page, 架构拆解
 * item 3).  Each layer keeps a 128-token sliding window that is merged with
 * the global cache (infernews.com, "DeepSeek V4.1 Flash 模型架構與推論優化
 * 技術規格剖析", section 2; zulogic, same page, section 4).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is DEVICE memory unless marked (host).  All
 *   buffers are owned by the caller; the library allocates nothing, frees
 *   nothing and keeps no state between calls, except the fixed per-device
 *   scratch of csa2_sparse_decode_noalloc.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Every call only enqueues work on it and returns; nothing synchronises.
 * - Return value: CSA2_OK, or a negative csa2_status for a host-side
 *   argument error (nothing is enqueued then) or a failed launch.  The
 *   library never reads device memory on the host, so contract violations
 *   that live in device data (an index out of range, a bad page id, a
 *   length beyond the page table) are not reported: the kernels skip such
 *   entries without touching memory outside the buffers, and results for
 *   the affected sequence are unspecified.
 * - Workspaces: calls that need scratch take (ws, ws_bytes), sized by the
 *   matching *_workspace_size query.  A workspace starts with per-sequence
 *   control words (batch of them) that must be zero when a call starts;
 *   the scratch after them is laid out from the call's batch and sizes.
 *   So a workspace must be zero-filled (csa2_workspace_init, or any zeroing
 *   allocation) before its first use, and again whenever it is handed to a
 *   call of another kind or with another `batch` than the call before it.
 *   Every call returns its control words to zero before it finishes, so
 *   later calls of the same kind and batch on the same stream need no
 *   re-initialisation, whatever their other sizes.  Two calls in flight on
 *   different streams need two workspaces.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_PAGE_TOKENS 64   /* token positions per cache page              */
#define CSA2_WINDOW 128       /* sliding-window length in tokens              */
#define CSA2_GROUP 16         /* channels per E4M3 scale                      */

typedef enum {
  CSA2_OK = 0,
  CSA2_E_NULL = -1,          /* a required pointer is NULL                    */
  CSA2_E_SHAPE = -2,         /* a size or count is out of range               */
  CSA2_E_UNSUPPORTED = -3,   /* head_dim / idx_dim / heads not supported      */
  CSA2_E_WORKSPACE = -4,     /* workspace NULL or smaller than required       */
  CSA2_E_HIP = -5,           /* a kernel launch failed                        */
  CSA2_E_SCRATCH = -6        /* request needs more than an allocation-free
                                call's fixed scratch                          */
} csa2_status;

/*
 * One owner ("Full") layer's global state.  All consumer layers read it.
 *
 * pages       device, num_pages * csa2_page_bytes(head_dim, idx_dim) bytes.
 *             Page layout (64 positions each), back to back:
 *               rows   [64][R], R = head_dim/2 + head_dim/16 bytes, the FP4
 *                      row of one token, contiguous:
 *                        codes  [head_dim/2]   E2M1 codes; channel 2j in the
 *                                              low nibble of byte j, 2j+1 in
 *                                              the high nibble
 *                        scales [head_dim/16]  E4M3 (OCP "FN") scale of
 *                                              channels 16g..16g+15 in byte g
 *               keys   [64][idx_dim]  int8 indexer keys
 *             (R = 288 at head_dim 512; a page is 26,624 bytes with idx_dim 128.)
 * page_table  device int32 [batch][max_pages_per_seq]: physical page of
 *             logical page i of sequence b (position p lives in page
 *             page_table[b][p/64], row p%64).  Contiguous caches use the
 *             identity table; the kernels have one code path.
 * head_dim    D, latent width of one KV row: 128, 256 or 512.
 * idx_dim     Di, indexer key width: 64 or 128.
 */
typedef struct {
  void* pages;
  const int32_t* page_table;
  int32_t num_pages;
  int32_t max_pages_per_seq;
  int32_t batch;
  int32_t head_dim;
  int32_t idx_dim;
} csa2_cache;

/* Bytes of one page: 64 * (D/2 + D/16 + Di).  0 for unsupported D/Di. */
size_t csa2_page_bytes(int32_t head_dim, int32_t idx_dim);

/* Human-readable name of a csa2_status value (static string). */
const char* csa2_status_string(int status);

/* Zero-fill `bytes` of workspace `ws` on `stream` with a fill kernel (no
 * memset node, so the call may be captured in a HIP graph). */
int csa2_workspace_init(void* ws, size_t bytes, void* stream);

/*
 * csa2_quantize_append -- FP4/E4M3 pack-and-quantise append.
 * Source: FP4 main KV = E2M1 codes with one E4M3 scale per 16 channels
 * (neodrop.ai V4.1-Flash report, 架构拆解 item 3); per-layer window of 128
 * tokens (zulogic "DeepSeek V4 1-Flash 架构拆解", section 4).
 *
 * For each token i < n_tokens, with b = seq[i], p = pos[i]:
 *   - per group of 16 channels: amax = max |x|; scale s = E4M3(amax/6),
 *     nearest with ties to the even code, saturating at 448; every channel
 *     gets the E2M1 code nearest to |x|/s (ties to the even code, sign bit
 *     = sign bit of x, all-zero magnitudes when s = 0);
 *   - the codes and scales go to row p of sequence b (layout above);
 *   - key_i8[i] (if key_i8 != NULL) goes to the indexer-key row of p;
 *   - x[i] (bf16 bits) goes to window slot p % 128 of swa[b] (if swa != NULL).
 *
 * x       device uint16 [n_tokens][D], bf16 bit patterns, finite values.
 * key_i8  device int8 [n_tokens][Di] or NULL.
 * seq,pos device int32 [n_tokens].  Tokens with b outside [0, batch), p
 *         outside [0, 64*max_pages_per_seq) or an out-of-range page id are
 *         skipped.  Two tokens of one call writing the same row or window
 *         slot race (either may win).
 * swa     device uint16 [batch][128][D] ring of this layer, or NULL.
 * Errors: CSA2_E_NULL (cache, pages, page_table, x, seq, pos when
 *         n_tokens > 0), CSA2_E_UNSUPPORTED (D, Di), CSA2_E_SHAPE
 *         (n_tokens < 0, batch/num_pages/max_pages_per_seq < 1).
 */
int csa2_quantize_append(const csa2_cache* cache, int32_t n_tokens,
                         const uint16_t* x, const int8_t* key_i8,
                         const int32_t* seq, const int32_t* pos,
                         uint16_t* swa, void* stream);

/*
 * csa2_index_topk -- Full layer: indexer scores and deterministic Top-K.
 * Source: shared indexer keys and Top-K addressing indices (neodrop.ai
 * V4.1-Flash report, 架构拆解 item 2); Full = the layer that builds the
 * indexer state and runs the sparse selection (zulogic, section 3 table).
 *
 * For each sequence b with L = ctx_len[b], n = max(0, L - 128) candidates:
 *   score[p] = sum_d q_idx[b][d] * key[b][p][d]   (int8 x int8 -> int32, exact)
 *   selected = the first min(K, n) positions p < n in the order
 *              (score descending, position ascending);
 *   out_idx[b]   = selected positions in ascending order, then -1 up to K;
 *   out_count[b] = min(K, n).
 *
 * ctx_len     device int32 [batch], 0 <= L <= 64*max_pages_per_seq.
 * max_ctx     (host) an upper bound of every ctx_len[b]; sizes the grid and
 *             the workspace.  Lengths above it are clamped to it.
 * q_idx       device int8 [batch][Di].
 * K           0 <= K <= 65536.
 * out_idx     device int32 [batch][K]; out_count device int32 [batch].
 * out_scores  device int32 [batch][max_ctx] or NULL: when given, receives
 *             the scores of positions p < n (other entries untouched).
 * ws          workspace of csa2_index_topk_workspace_size(batch, max_ctx, K).
 * Errors: CSA2_E_NULL, CSA2_E_UNSUPPORTED (Di), CSA2_E_SHAPE (K, max_ctx,
 *         batch), CSA2_E_WORKSPACE.
 */
size_t csa2_index_topk_workspace_size(int32_t batch, int32_t max_ctx, int32_t K);
int csa2_index_topk(const csa2_cache* cache, const int32_t* ctx_len, int32_t max_ctx,
                    const int8_t* q_idx, int32_t K,
                    int32_t* out_idx, int32_t* out_count, int32_t* out_scores,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_append_index_topk -- a decode step's append and the Full layer's
 * selection in one call: the same results as csa2_quantize_append(cache,
 * n_tokens, x, key_i8, seq, pos, swa) followed by csa2_index_topk(cache,
 * ctx_len, max_ctx, q_idx, K, ...), for tokens that lie in their sequence's
 * window (L - 128 <= pos, L = ctx_len[seq] clamped as in csa2_index_topk).
 * The append runs inside the scoring launch, which reads only positions
 * below L - 128, so the two cannot race; a token at a position below
 * L - 128 (a scoring candidate) is not written.  Arguments, limits, outputs
 * and errors as the two calls; ws is csa2_index_topk's workspace.
 */
int csa2_append_index_topk(const csa2_cache* cache, int32_t n_tokens, const uint16_t* x,
                           const int8_t* key_i8, const int32_t* seq, const int32_t* pos,
                           uint16_t* swa, const int32_t* ctx_len, int32_t max_ctx,
                           const int8_t* q_idx, int32_t K, int32_t* out_idx, int32_t* out_count,
                           int32_t* out_scores, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_reindex -- Reindex layer: refilter the owner's candidate pool.
 * Source: hierarchical sparse indexer, later indexer layers refilter only
 * inside the pool built by the first Full layer (neodrop.ai V4.1-Flash
 * report, 架构拆解 item 2); Reindex = reuse the KV, recompute the index /
 * candidates (zulogic, section 3 table).
 *
 * For each sequence b: the first c = pool_count[b] entries of pool[b] are
 * scored with this layer's q_idx[b] against the SHARED indexer keys; the
 * first min(K, c) in (score descending, position ascending) order are
 * written to out_idx[b] in ascending order, padded with -1 to K, and
 * out_count[b] = min(K, c).
 *
 * pool        device int32 [batch][P]: strictly ascending valid positions
 *             (the form csa2_index_topk returns); c <= P <= 65536.
 * K           0 <= K <= P.
 * out_scores  device int32 [batch][P] or NULL: scores of pool entries.
 * ws          workspace of csa2_reindex_workspace_size(batch, P, K).
 * Errors: as csa2_index_topk.
 */
size_t csa2_reindex_workspace_size(int32_t batch, int32_t P, int32_t K);
int csa2_reindex(const csa2_cache* cache, const int8_t* q_idx,
                 const int32_t* pool, const int32_t* pool_count, int32_t P, int32_t K,
                 int32_t* out_idx, int32_t* out_count, int32_t* out_scores,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_sparse_decode -- merged sparse attention of one layer.
 * Source: the global cache is merged with the window cache before decoding
 * (infernews.com V4.1 Flash page, section 2); each layer keeps its own
 * 128-token window (zulogic, section 4); Reuse layers attend with their own
 * queries over the reused indices (zulogic, section 3 table).
 *
 * For each sequence b (L = ctx_len[b], c = idx_count[b]) and head h < H:
 *   rows  = E2M1(code) * E4M3(scale) of positions idx[b][0..c) (exact), and
 *           the window positions [max(0, L-128), L) from swa[b][p % 128];
 *           each row is both key and value;
 *   l_j   = softmax_scale * <q[b][h], row_j>;
 *   out[b][h] = sum_j softmax(l)_j row_j   (one softmax over the union);
 *   lse[b][h] = max l + ln sum exp(l - max l)   (if lse != NULL).
 * With no rows at all (L = 0): out = 0, lse = -inf.
 *
 * q            device uint16 [batch][H][D] bf16 bits, H a multiple of 16,
 *              16 <= H <= 128.
 * idx          device int32 [batch][K]: c distinct positions in [0, L-128);
 *              entries at or beyond the count are ignored.  0 <= K <= 65536.
 * swa          device uint16 [batch][128][D] bf16 ring of this layer.  The
 *              window rows run through fp16 MFMA operands, so its live values
 *              must be finite and exactly representable in fp16: magnitude at
 *              most 65504, and a multiple of 2^-24 below 2^-14 (bf16 values
 *              from 2^-14 to 65280 always are).  csa2_validate_window reports
 *              rings outside this range.  NULL: no window rows (a context
 *              shard that holds none of the last 128 positions, see below).
 * out          device float [batch][H][D]; lse device float [batch][H] or NULL.
 * ws           workspace of csa2_sparse_decode_workspace_size(batch, H, D, K).
 * Selected positions whose page-table entry lies outside [0, num_pages)
 * are skipped, so a shard's cache view with -1 for the pages it does not
 * hold attends over its own rows only.
 * Errors: CSA2_E_NULL, CSA2_E_UNSUPPORTED (D, H), CSA2_E_SHAPE (K, batch),
 *         CSA2_E_WORKSPACE.
 */
size_t csa2_sparse_decode_workspace_size(int32_t batch, int32_t H, int32_t head_dim, int32_t K);
int csa2_sparse_decode(const csa2_cache* cache, const int32_t* ctx_len, int32_t H,
                       const uint16_t* q, float softmax_scale,
                       const int32_t* idx, const int32_t* idx_count, int32_t K,
                       const uint16_t* swa, float* out, float* lse,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_sparse_decode_noalloc -- csa2_sparse_decode without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, results, limits and errors as csa2_sparse_decode, minus
 * (ws, ws_bytes); the split partials go to a fixed scratch array the library
 * holds on each device, CSA2_NOALLOC_SCRATCH_BYTES bytes, for as long as the
 * process lives.  A call whose csa2_sparse_decode_workspace_size exceeds that
 * returns CSA2_E_SCRATCH before anything is enqueued.  The call allocates and
 * frees nothing; its first call on a device looks up that device's scratch
 * address (once, with the device current).  `stream` must belong to the
 * current device.  All calls on one device share its scratch, and nothing in
 * it needs to start at any value (every partial a call reads it wrote
 * first), but two calls that overlap in time on one device (different
 * streams, or host threads) race on it: serialise them.
 */
#define CSA2_NOALLOC_SCRATCH_BYTES (64u << 20)
int csa2_sparse_decode_noalloc(const csa2_cache* cache, const int32_t* ctx_len, int32_t H,
                               const uint16_t* q, float softmax_scale,
                               const int32_t* idx, const int32_t* idx_count, int32_t K,
                               const uint16_t* swa, float* out, float* lse, void* stream);

/*
 * csa2_validate_selection -- a debug-time check of the device-side contract
 * of csa2_sparse_decode's selection inputs, which the other calls do not
 * report (they skip offending entries and leave the sequence's results
 * unspecified).  For each sequence b, flags[b] (device uint32 [batch]) gets
 * the OR of:
 *   CSA2_SEL_BAD_LENGTH    ctx_len[b] outside [0, 64 * max_pages_per_seq]
 *   CSA2_SEL_BAD_COUNT     idx_count[b] outside [0, K]
 *   CSA2_SEL_BAD_POSITION  a counted index outside [0, L - 128) (the
 *                          candidates; window positions are not selectable)
 *   CSA2_SEL_BAD_PAGE      a counted index whose page-table entry is outside
 *                          [0, num_pages) (legal for a context shard's view)
 *   CSA2_SEL_NOT_ASCENDING the counted indices are not strictly ascending
 *                          (csa2_sparse_decode accepts any order of distinct
 *                          positions; in ascending order distinctness is
 *                          checked, in any other order it is not)
 * 0 means the inputs meet the contract.  Errors: CSA2_E_NULL, CSA2_E_SHAPE.
 */
#define CSA2_SEL_BAD_LENGTH 1u
#define CSA2_SEL_BAD_COUNT 2u
#define CSA2_SEL_BAD_POSITION 4u
#define CSA2_SEL_BAD_PAGE 8u
#define CSA2_SEL_NOT_ASCENDING 16u
int csa2_validate_selection(const csa2_cache* cache, const int32_t* ctx_len,
                            const int32_t* idx, const int32_t* idx_count, int32_t K,
                            uint32_t* flags, void* stream);

/*
 * csa2_validate_window -- a debug-time check of the window-ring contract of
 * csa2_sparse_decode (the ring's values are bf16 in the method; the decode
 * holds them as exact fp16 operands).  For each sequence b, flags[b] (device
 * uint32 [batch]) gets the OR, over the live slots of swa[b] (those of
 * positions [max(0, L - 128), L), L = ctx_len[b] clamped to the page table), of:
 *   CSA2_WIN_NOT_F16     a finite value that fp16 does not hold exactly
 *                        (magnitude above 65504, or too fine below 2^-14);
 *                        csa2_sparse_decode would round it
 *   CSA2_WIN_NOT_FINITE  an infinite or NaN value
 * Dead slots (L < 128) are not read.  Errors: CSA2_E_NULL, CSA2_E_SHAPE,
 * CSA2_E_UNSUPPORTED.
 * Source of the window: zulogic "DeepSeek V4 1-Flash 架构拆解", section 4;
 * infernews.com V4.1 Flash page, section 2.
 */
#define CSA2_WIN_NOT_F16 1u
#define CSA2_WIN_NOT_FINITE 2u
int csa2_validate_window(const csa2_cache* cache, const int32_t* ctx_len, const uint16_t* swa,
                         uint32_t* flags, void* stream);

/*
 * Context sharding of long sequences (several devices each holding a
 * contiguous range of a sequence's pages).  Each shard selects among its own
 * candidates under the Full layer's order; csa2_topk_merge turns the shard
 * lists into the one-device selection (exactly: an entry of the global Top-K
 * is beaten by fewer than K entries overall, hence by fewer than K in its
 * shard); each shard attends over the selected rows it holds (the tail shard
 * also over the window) and csa2_lse_merge combines the parts, which is the
 * one softmax over the union.  Selection rule: neodrop.ai V4.1-Flash report,
 * 架构拆解 item 2; one softmax over the merged caches: infernews.com V4.1
 * Flash page, section 2.
 */

/*
 * csa2_index_topk_range -- Full-layer selection restricted to the candidate
 * positions p_begin <= p < min(p_end, L - 128) of every sequence (entries,
 * order, tie rule and output form as csa2_index_topk).
 *
 * p_begin, p_end  (host) p_begin a multiple of 64, p_begin <= p_end.
 * out_sel_scores  device int32 [batch][K] or NULL: the score of each
 *                 selected position (aligned with out_idx), 0 past the count.
 * ws              workspace of csa2_index_topk_workspace_size(batch, max_ctx, K).
 * Errors: as csa2_index_topk, and CSA2_E_SHAPE for the range.
 */
int csa2_index_topk_range(const csa2_cache* cache, const int32_t* ctx_len, int32_t max_ctx,
                          const int8_t* q_idx, int32_t K, int32_t p_begin, int32_t p_end,
                          int32_t* out_idx, int32_t* out_count, int32_t* out_sel_scores,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_topk_merge -- the Top-K of n_parts shard selections of each sequence.
 *
 * idx      device int32 [n_parts][batch][K_in]: part s's positions of
 *          sequence b, strictly ascending; the parts of a sequence hold
 *          disjoint positions, in ascending order of part (part s below part
 *          s + 1), as csa2_index_topk_range returns them for ascending ranges.
 * scores   device int32 [n_parts][batch][K_in]: their scores.
 * counts   device int32 [n_parts][batch]: entries per part (clamped to
 *          [0, K_in]).
 * Output: out_idx[b] = the first min(K, total) of the union in (score
 * descending, position ascending) order, ascending, -1 padded to K;
 * out_count[b]; out_sel_scores (device int32 [batch][K] or NULL) their scores.
 * Limits: 1 <= n_parts <= 64, 0 <= K_in <= 65536, n_parts*K_in <= 524288,
 *         0 <= K <= min(65536, n_parts*K_in).
 * ws       workspace of csa2_topk_merge_workspace_size(batch, n_parts, K_in, K).
 * Errors: CSA2_E_NULL, CSA2_E_SHAPE, CSA2_E_WORKSPACE.
 */
size_t csa2_topk_merge_workspace_size(int32_t batch, int32_t n_parts, int32_t K_in, int32_t K);
int csa2_topk_merge(int32_t batch, int32_t n_parts, int32_t K_in, const int32_t* idx,
                    const int32_t* scores, const int32_t* counts, int32_t K,
                    int32_t* out_idx, int32_t* out_count, int32_t* out_sel_scores,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_lse_merge -- merge attention results over disjoint key sets.
 * For each row r = (b, h): M = max_s lses[s][r], w_s = exp(lses[s][r] - M)
 * (0 when lses[s][r] = -inf), out[r] = sum_s w_s outs[s][r] / sum_s w_s,
 * lse[r] = M + ln sum_s w_s (out = 0, lse = -inf when every part is empty).
 *
 * outs  device float [n_parts][batch][H][D]; lses device float [n_parts][batch][H]
 *       (csa2_sparse_decode's out and lse of each part).
 * out   device float [batch][H][D]; lse device float [batch][H] or NULL.
 * Limits: 1 <= n_parts <= 64, 1 <= H <= 128, D = head_dim in {128, 256, 512}.
 * Errors: CSA2_E_NULL, CSA2_E_SHAPE, CSA2_E_UNSUPPORTED.
 */
int csa2_lse_merge(int32_t n_parts, int32_t batch, int32_t H, int32_t head_dim,
                   const float* outs, const float* lses, float* out, float* lse, void* stream);

/*
 * Indexer keys with a per-token scale.  The owner layer's state holds the
 * indexer keys together with their scale (zulogic, "DeepSeek V4 1-Flash
 * 架构拆解", section 3, the owner-layer state diagram); the page gives no
 * formula, so the reading here is: every cached position p carries one fp32
 * scale s_p, and the ranked value is
 *   v_p = fl32(s_p * score_p)
 * (the int32 score is exact in float32; one round-to-nearest-even rounding),
 * with -0 taken as +0.  Order: value descending, position ascending; equal
 * values (including the two zeros) are ties that go to the lower position.
 * Scales must be finite; a non-finite scale gives an unspecified order for
 * its sequence (never an out-of-bounds access).
 *
 * key_scales  device float [num_pages][64]: the scale of page row r of
 *             physical page g at key_scales[64*g + r], beside the pages
 *             (caller-owned, filled by csa2_store_key_scales).
 */

/*
 * csa2_store_key_scales -- write the key scales of appended tokens.
 * scale[i] goes to the row of position pos[i] of sequence seq[i] (its page
 * from the page table); tokens whose (seq, pos) does not map to a page in
 * [0, num_pages) are skipped, as in csa2_quantize_append.
 * scale device float [n_tokens]; seq, pos device int32 [n_tokens].
 * Errors: CSA2_E_NULL, CSA2_E_UNSUPPORTED, CSA2_E_SHAPE.
 */
int csa2_store_key_scales(const csa2_cache* cache, int32_t n_tokens, const float* scale,
                          const int32_t* seq, const int32_t* pos, float* key_scales,
                          void* stream);

/*
 * csa2_store_key_scales_e4m3 -- the same with one E4M3 byte per token (the
 * OCP "FN" encoding of the cache's own scales): each byte is decoded exactly
 * to fp32 (an E4M3 value is a float32 value), so the ranking is that of the
 * decoded scales.  The NaN codes 0x7F / 0xFF decode to NaN, which the
 * ranking takes as a non-finite scale.
 * scale_e4m3 device uint8 [n_tokens]; other arguments and errors as above.
 */
int csa2_store_key_scales_e4m3(const csa2_cache* cache, int32_t n_tokens,
                               const uint8_t* scale_e4m3, const int32_t* seq, const int32_t* pos,
                               float* key_scales, void* stream);

/*
 * csa2_index_topk_scaled -- csa2_index_topk ranked by the scaled values v_p.
 * out_idx / out_count as csa2_index_topk (the first min(K, n) candidates in
 * (value descending, position ascending) order, ascending, -1 padded).
 * out_values      device float [batch][max_ctx] or NULL: v_p of every
 *                 candidate p < n (other entries untouched).
 * out_sel_values  device float [batch][K] or NULL: v_p of each selected
 *                 position (aligned with out_idx), 0 past the count.
 * ws              workspace of csa2_index_topk_workspace_size(batch, max_ctx, K).
 * Errors: as csa2_index_topk, and CSA2_E_NULL for key_scales.
 */
int csa2_index_topk_scaled(const csa2_cache* cache, const int32_t* ctx_len, int32_t max_ctx,
                           const int8_t* q_idx, const float* key_scales, int32_t K,
                           int32_t* out_idx, int32_t* out_count, float* out_values,
                           float* out_sel_values, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_reindex_scaled -- csa2_reindex ranked by the scaled values v_p of the
 * pool entries (this layer's q_idx against the shared keys and scales).
 * out_values  device float [batch][P] or NULL: v of each pool entry; an entry
 *             whose position has no page in [0, num_pages) gets -inf.
 * ws          workspace of csa2_reindex_workspace_size(batch, P, K).
 * Errors: as csa2_reindex, and CSA2_E_NULL for key_scales.
 */
int csa2_reindex_scaled(const csa2_cache* cache, const int8_t* q_idx, const float* key_scales,
                        const int32_t* pool, const int32_t* pool_count, int32_t P, int32_t K,
                        int32_t* out_idx, int32_t* out_count, float* out_values, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * csa2_stream_read -- a measurement aid, not a step of the method: reads
 * `bytes` of device memory at src once with 16-byte non-temporal loads (each
 * workgroup one contiguous 16 KB run) and XORs every word into *sink (device uint32; its old value is kept, so the
 * result is defined but of no use beyond keeping the loads).  Timing it
 * beside the method's calls gives the rate a plain read-only kernel reaches
 * on this memory, the reference against which the calls' achieved rates are
 * read: the method exists to cut the bytes one decode reads from HBM
 * (neodrop.ai V4.1-Flash page, section 架构拆解 introduction; zulogic,
 * section 9), and long-context decode is to be measured on its own
 * (zulogic, section 10).  bytes must be a multiple of 16 and src 16-byte
 * aligned.  Errors: CSA2_E_NULL, CSA2_E_SHAPE.
 */
int csa2_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * Context sharding with scaled keys: the same two steps as
 * csa2_index_topk_range + csa2_topk_merge, ranked by the values v_p.  The
 * merge is exact for the same reason (the order is total).
 *
 * csa2_index_topk_range_scaled -- csa2_index_topk_scaled over the candidate
 *   positions p_begin <= p < min(p_end, L - 128); out_sel_values (device
 *   float [batch][K] or NULL) holds the selected values.  Arguments, limits
 *   and errors as csa2_index_topk_range.
 * csa2_topk_merge_values -- csa2_topk_merge of shard lists whose scores are
 *   the float32 values (device float [n_parts][batch][K_in]); out_sel_values
 *   device float [batch][K] or NULL.  Limits, workspace and errors as
 *   csa2_topk_merge.
 */
int csa2_index_topk_range_scaled(const csa2_cache* cache, const int32_t* ctx_len,
                                 int32_t max_ctx, const int8_t* q_idx, const float* key_scales,
                                 int32_t K, int32_t p_begin, int32_t p_end, int32_t* out_idx,
                                 int32_t* out_count, float* out_sel_values, void* ws,
                                 size_t ws_bytes, void* stream);
int csa2_topk_merge_values(int32_t batch, int32_t n_parts, int32_t K_in, const int32_t* idx,
                           const float* values, const int32_t* counts, int32_t K,
                           int32_t* out_idx, int32_t* out_count, float* out_sel_values, void* ws,
                           size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
