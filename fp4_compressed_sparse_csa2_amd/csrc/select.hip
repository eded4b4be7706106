// Deterministic Top-K over int32 indexer scores: the selection kernels shared
// by csa2_index_topk (the Full layer's candidates 0 <= p < L - 128) and
// csa2_reindex (the entries of the Full layer's pool).
//
// The Full layer makes the sparse selection whose Top-K addressing indices
// later layers reuse, and deeper indexer layers refilter only the pool the
// Full layer built (neodrop.ai V4.1-Flash report, 架构拆解 item 2; zulogic
// "DeepSeek V4 1-Flash 架构拆解", section 3).  Order: score descending,
// position ascending.
//
// Input: the scores and, per sequence, a 2048-bin histogram of the top 11
// bits of the biased 22-bit key (built by the scoring kernel).  Two plans, no
// cross-block synchronisation inside a kernel (visibility comes from kernel
// boundaries):
//   single  - up to kSingleMax entries: one block per sequence holds them
//             all in registers (one 16-byte load row of 16 KB per step),
//             finds the K-th largest top digit t1, histograms the low digit
//             of the entries whose top digit is t1, fixes the exact
//             threshold and gives each selected entry its output slot from
//             one block scan of per-thread counts.
//   filter  - longer sequences: 4096-entry blocks keep their digit >= t1
//   + final   entries, in order, in their own slots; then one block per
//             sequence concatenates the slot lists (already in order),
//             histograms the low digit, fixes the threshold and emits.
// Both return the sequence's histogram to zero for the next call.
#include "common.h"
#include "launch.h"
#include "select.h"

namespace csa2 {

constexpr int kSelNT = 1024;                     // threads of the one-block-per-sequence kernels
constexpr int kSelWaves = kSelNT / 64;
constexpr int kListCap = 6144;                   // candidates the final kernel keeps in LDS
constexpr int kDirectPer = 8;                    // slots per thread in the final kernel's direct gather
constexpr int kFiltPer = 16;                     // entries per thread in the filter kernel
constexpr int kFiltChunk = kBlock * kFiltPer;    // 4096 entries per filter block

// Number of entries of sequence b.
__device__ __forceinline__ int sel_entries(const SelectArgs& a, int b) {
  if (a.pool_count != nullptr) {
    const int c = a.pool_count[b];
    return c < 0 ? 0 : (c > a.P ? a.P : c);
  }
  int L = a.ctx_len[b];
  L = L < 0 ? 0 : L;
  L = L > a.max_ctx ? a.max_ctx : L;
  L = L > a.max_pages * kPage ? a.max_pages * kPage : L;
  int hi = L > kWindow ? L - kWindow : 0;              // candidates end below the window
  hi = hi < a.p_end ? hi : a.p_end;
  return hi > a.p_begin ? hi - a.p_begin : 0;
}

// The j-th selected entry c = {key, entry} of sequence b: its id, and its
// score (or value) when the caller asked for them.  POOL (a Reindex layer):
// the entry index goes out, and map_pool turns the list into pool positions
// once it is complete (the one-block kernel holds the pool row in LDS and
// writes positions directly).  No output store depends on a load, so that the
// stores of an emission never wait for one another.
template <typename KT>
__device__ __forceinline__ void put_id(const SelectArgs& a, int b, int j, int32_t id,
                                       uint32_t key) {
  a.out_idx[(size_t)b * a.K + j] = id;
  if (a.out_sel_scores != nullptr) a.out_sel_scores[(size_t)b * a.K + j] = KT::out_word(key);
}
template <typename KT, bool POOL>
__device__ __forceinline__ void put_sel(const SelectArgs& a, int b, int j, uint2 c) {
  put_id<KT>(a, b, j, POOL ? (int32_t)c.y : a.p_begin + (int32_t)c.y, c.x);
}

// The first `written` outputs of sequence b (entry indices, put_sel<.., true>
// by this block) replaced by their pool positions.  All threads call.
template <int NT>
__device__ __forceinline__ void map_pool(const SelectArgs& a, int b, int written) {
  __syncthreads();                               // the block's output stores are visible
  int32_t* out = a.out_idx + (size_t)b * a.K;
  const int32_t* pool = a.pool + (size_t)b * a.P;
  for (int j = threadIdx.x; j < written; j += NT) out[j] = pool[out[j]];
}

// K = 0 or every entry selected: the first min(K, n) entries in order, then -1.
template <typename KT, bool POOL>
__device__ __forceinline__ void select_all(const SelectArgs& a, int b, int n, int nt) {
  int32_t* out = a.out_idx + (size_t)b * a.K;
  const int32_t* row = a.scores + (size_t)b * a.stride;
  for (int i = threadIdx.x; i < a.K; i += nt) {
    out[i] = i >= n ? -1 : (POOL ? a.pool[(size_t)b * a.P + i] : a.p_begin + i);
    if (a.out_sel_scores != nullptr)
      a.out_sel_scores[(size_t)b * a.K + i] = i < n ? KT::stored_out(row[i]) : 0;
  }
  if (threadIdx.x == 0) a.out_count[b] = n < a.K ? n : a.K;
}

// ------------------------------------------------------------------ single
// Up to kSingleMax entries, all held in registers by a block of kSingleNT
// threads.  Thread t holds entries 4096j + 4t + k (j < 4, k < 4): row j of
// the block's loads reads 16 KB of consecutive scores, 1 KB per wave
// instruction (rows past the last entry are not loaded).  With the top digit t1 from
// the scoring kernel's histogram, the entries whose top digit is t1
// histogram their second digit in LDS (float keys: then those on the
// threshold's top 22 bits their third), which fixes the threshold key tau and
// how many entries equal to it are taken.  One block scan of each thread's
// per-row (above, tie) counts then gives every selected entry its output slot
// in entry order: no candidate list is built.  POOL: the pool row is staged in
// LDS (its loads in flight with the scores') and the slots get pool positions.
constexpr int kSingleNT = 1024;                      // threads of the one-block kernel
constexpr int kSingleWaves = kSingleNT / 64;
constexpr int kRegRow = 4 * kSingleNT;                // entries per load row
constexpr int kRegRows = kSingleMax / kRegRow;        // 4 rows of 4096 entries
static_assert(kRegRow <= 0xFFFF, "a row prefix fits a packed half");

template <typename KT, bool POOL>
__global__ __launch_bounds__(kSingleNT) void select_single_kernel(SelectArgs a) {
  __shared__ uint32_t hist2[kBins];
  __shared__ __attribute__((aligned(16))) int32_t pool_lds[POOL ? kSingleMax : 1];   // pool row
  __shared__ int scan_scratch[kSingleWaves];
  __shared__ int row_scan[kRegRows][kSingleWaves];
  __shared__ int sh_t1, sh_above1, sh_t2, sh_above2, sh_t3, sh_above3;

  const int b = blockIdx.x;
  const int n = sel_entries(a, b);
  const int K = a.K;
  if (K == 0 || n <= K) {
    select_all<KT, POOL>(a, b, n, kSingleNT);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* h1 = a.hist1 + (size_t)b * kCtrlWords;
  const int32_t* row = a.scores + (size_t)b * a.stride;
  const int nrows = (n + kRegRow - 1) / kRegRow;        // load rows holding entries

  // POOL: with P a multiple of 4 and a 16-byte aligned pool, the row is read
  // in rows of 16-byte loads like the scores (entries 4096j + 4t .. +3; a
  // load that starts below n <= P then ends inside the row), else entry by
  // entry
  constexpr int kPoolPer = POOL ? kSingleMax / kSingleNT : 1;
  int32_t pv[kPoolPer];
  const int32_t* prow = POOL ? a.pool + (size_t)b * a.P : nullptr;
  const bool pool16 =
      POOL && (a.P & 3) == 0 && (reinterpret_cast<uintptr_t>(a.pool) & 15u) == 0u;
  if constexpr (POOL) {
    if (pool16) {
#pragma unroll
      for (int j = 0; j < kRegRows; ++j) {
        if (j >= nrows) break;
        const int e0 = j * kRegRow + 4 * tid;
        const int4 q = *reinterpret_cast<const int4*>(prow + (e0 < n ? e0 : 0));
        pv[4 * j] = q.x;
        pv[4 * j + 1] = q.y;
        pv[4 * j + 2] = q.z;
        pv[4 * j + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPoolPer; ++i) {
        const int e = tid + i * kSingleNT;
        pv[i] = prow[e < n ? e : 0];
      }
    }
  }
  // Entry indices of a load are multiples of 4 and the row stride a multiple
  // of 64, so a load that starts below n lies inside the row; loads that
  // start at or past n read entry 0 instead and are masked.
  uint4 v[kRegRows];
#pragma unroll
  for (int j = 0; j < kRegRows; ++j) {
    if (j >= nrows) break;
    const int e0 = j * kRegRow + 4 * tid;
    v[j] = *reinterpret_cast<const uint4*>(row + (e0 < n ? e0 : 0));
  }
  const DigitBins<kSingleNT> bins = load_digit_bins<kSingleNT, kHistReps>(h1);
  for (int i = tid; i < kBins; i += kSingleNT) hist2[i] = 0u;
  if constexpr (POOL) {
    if (pool16) {
#pragma unroll
      for (int j = 0; j < kRegRows; ++j) {
        if (j >= nrows) break;
        const int e0 = j * kRegRow + 4 * tid;
        if (e0 < n)
          *reinterpret_cast<int4*>(pool_lds + e0) =
              make_int4(pv[4 * j], pv[4 * j + 1], pv[4 * j + 2], pv[4 * j + 3]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPoolPer; ++i) {
        const int e = tid + i * kSingleNT;
        if (e < n) pool_lds[e] = pv[i];
      }
    }
  }
  find_digit_in<kSingleNT>(bins, K, scan_scratch, &sh_t1, &sh_above1);
  const bool have_t1 = sh_t1 >= 0;
  const uint32_t t1 = (uint32_t)sh_t1;
  {
    // every thread has read its bins (before find_digit_in's barriers):
    // return the histogram replicas to zero for the next call now, so that
    // the stores drain while the entries are classified
    uint4* h4 = reinterpret_cast<uint4*>(h1);
    for (int i = tid; i < kCtrlHist2 / 4; i += kSingleNT) h4[i] = make_uint4(0u, 0u, 0u, 0u);
  }

  // keys of the held entries (rows past n are skipped, block-uniformly) and
  // 4-bit masks of the live ones, and of those whose top digit is t1
  uint32_t key[kRegRows][4];
  uint32_t live[kRegRows];
#pragma unroll
  for (int j = 0; j < kRegRows; ++j) {
    live[j] = 0u;
    if (j >= nrows) continue;
    const int w[4] = {(int)v[j].x, (int)v[j].y, (int)v[j].z, (int)v[j].w};
    const int lim = n - j * kRegRow - 4 * tid;          // live entries of the four
    live[j] = lim >= 4 ? 0xFu : (lim > 0 ? (1u << lim) - 1u : 0u);
    uint32_t at_t1 = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      key[j][k] = KT::key(w[k]);
      at_t1 |= (key[j][k] >> KT::kTopShift) == t1 ? 1u << k : 0u;
    }
    at_t1 = have_t1 ? at_t1 & live[j] : 0u;
    if (at_t1 != 0u) {                                  // second digit, few entries
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if ((at_t1 >> k) & 1u) atomicAdd(&hist2[KT::mid(key[j][k])], 1u);
    }
  }
  __syncthreads();
  find_digit<kSingleNT>(hist2, K - sh_above1, scan_scratch, &sh_t2, &sh_above2);
  uint32_t tau = have_t1 ? (t1 << 11) | (uint32_t)sh_t2 : 0xFFFFFFFFu;
  int need_ties = K - sh_above1 - sh_above2;
  if constexpr (KT::kThree) {
    // third digit: histogram (in hist2, whose bins every thread has read) of
    // the entries whose top 22 bits are the threshold's
    for (int i = tid; i < kBins; i += kSingleNT) hist2[i] = 0u;
    __syncthreads();
    const uint32_t pre = have_t1 && sh_t2 >= 0 ? tau : 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < kRegRows; ++j) {
      if (j >= nrows) continue;
      uint32_t at = 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k) at |= (key[j][k] >> KT::kLowBits) == pre ? 1u << k : 0u;
      at &= live[j];
      if (at != 0u) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if ((at >> k) & 1u) atomicAdd(&hist2[KT::low(key[j][k])], 1u);
      }
    }
    __syncthreads();
    find_digit<kSingleNT>(hist2, need_ties, scan_scratch, &sh_t3, &sh_above3);
    tau = sh_t3 >= 0 ? (pre << KT::kLowBits) | (uint32_t)sh_t3 : 0xFFFFFFFFu;
    need_ties = sh_t3 >= 0 ? need_ties - sh_above3 : 0;
  }

  // per row: masks of this thread's entries above tau and equal to it, and
  // their counts packed as above + (ties << 16) (a row prefix is at most
  // kRegRow, so the halves never carry)
  uint32_t gt[kRegRows], tie[kRegRows];
  int cnt[kRegRows], inc[kRegRows];
#pragma unroll
  for (int j = 0; j < kRegRows; ++j) {
    gt[j] = tie[j] = 0u;
    cnt[j] = inc[j] = 0;
    if (j >= nrows) continue;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      gt[j] |= key[j][k] > tau ? 1u << k : 0u;
      tie[j] |= key[j][k] == tau ? 1u << k : 0u;
    }
    gt[j] &= live[j];
    tie[j] &= live[j];
    cnt[j] = __builtin_popcount(gt[j]) + (__builtin_popcount(tie[j]) << 16);
    inc[j] = wave_inclusive_scan(cnt[j]);
  }
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < kRegRows; ++j) row_scan[j][wave] = inc[j];
  }
  __syncthreads();
  int before[kRegRows], tot[kRegRows];
#pragma unroll
  for (int j = 0; j < kRegRows; ++j) {
    before[j] = tot[j] = 0;
    if (j >= nrows) continue;
    const int2 bt = waves_before_and_total<kSingleNT>(row_scan[j]);
    before[j] = bt.x;
    tot[j] = bt.y;
  }
  // emit: the selected entries of a thread's row take consecutive slots,
  // starting after every selection before them in entry order; ties are
  // taken in entry order until need_ties of them are
  int g0 = 0, t0 = 0;                                 // over the rows before j
#pragma unroll
  for (int j = 0; j < kRegRows; ++j) {
    if (j >= nrows) continue;
    const int pre = before[j] + inc[j] - cnt[j];      // this thread's row prefix
    const int gb = g0 + (pre & 0xFFFF), tb = t0 + (pre >> 16);
    uint32_t sel = gt[j];
    int r = tb;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool t = (tie[j] >> k) & 1u;
      sel |= (t && r < need_ties) ? 1u << k : 0u;
      r += t ? 1 : 0;
    }
    const int slot0 = gb + (tb < need_ties ? tb : need_ties);
    if (sel != 0u) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int slot = slot0 + __builtin_popcount(sel & ((1u << k) - 1u));
        if (((sel >> k) & 1u) && slot < K) {
          const int e = j * kRegRow + 4 * tid + k;
          put_id<KT>(a, b, slot, POOL ? pool_lds[e] : a.p_begin + e, key[j][k]);
        }
      }
    }
    g0 += tot[j] & 0xFFFF;
    t0 += tot[j] >> 16;
  }
  const int taken = g0 + (t0 < need_ties ? t0 : need_ties);
  const int written = taken < K ? taken : K;
  int32_t* out = a.out_idx + (size_t)b * K;
  for (int j = written + tid; j < K; j += kSingleNT) {
    out[j] = -1;
    if (a.out_sel_scores != nullptr) a.out_sel_scores[(size_t)b * K + j] = 0;
  }
  if (tid == 0) a.out_count[b] = written;
}

// ------------------------------------------------------------------ filter
// Block = 4096 entries of one sequence.  Keeps the entries whose top digit is
// at least t1 in entry order in the chunk's own slot list, counts them, and
// adds the low digits of those whose top digit equals t1 to the sequence's
// low-digit histogram.
template <typename KT>
__global__ __launch_bounds__(kBlock) void select_filter_kernel(SelectArgs a) {
  __shared__ int scan_scratch[kBlock / 64];
  __shared__ int sh_t1, sh_above1;

  const int b = blockIdx.y;
  const int n = sel_entries(a, b);
  const int chunk = blockIdx.x, chunk0 = chunk * kFiltChunk;
  if (a.K == 0 || n <= a.K || chunk0 >= n) return;
  const int32_t* row = a.scores + (size_t)b * a.stride;
  uint32_t* ctrl = a.hist1 + (size_t)b * kCtrlWords;

  // the block's share of the histogram, then this thread's 16 scores, all in
  // flight together: the score loads are unconditional (a thread past n
  // reads the row's first 16 entries, inside the row, and keeps none), so
  // that no branch holds them and their use
  const DigitBins<kBlock> bins = load_digit_bins<kBlock, kHistReps>(ctrl);
  const int p0 = chunk0 + (int)threadIdx.x * kFiltPer;
  uint4 sv[kFiltPer / 4];
  {
    const uint4* src = reinterpret_cast<const uint4*>(row + (p0 < n ? p0 : 0));
#pragma unroll
    for (int i = 0; i < kFiltPer / 4; ++i) sv[i] = src[i];
  }
  find_digit_in<kBlock>(bins, a.K, scan_scratch, &sh_t1, &sh_above1);
  const uint32_t t1 = (uint32_t)sh_t1;
  if (chunk == 0 && threadIdx.x == 0) {  // for the final stage (every block finds the same)
    ctrl[kCtrlTop] = (uint32_t)sh_t1;
    ctrl[kCtrlTop + 1] = (uint32_t)sh_above1;
  }

  uint32_t key[kFiltPer];
  uint32_t keep = 0;                     // bit e: entry p0 + e is kept
#pragma unroll
  for (int i = 0; i < kFiltPer / 4; ++i) {
    const int w[4] = {(int)sv[i].x, (int)sv[i].y, (int)sv[i].z, (int)sv[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t kk = KT::key(w[k]);
      key[4 * i + k] = kk;
      keep |= (p0 + 4 * i + k < n && (kk >> KT::kTopShift) >= t1) ? 1u << (4 * i + k) : 0u;
    }
  }
  int chunk_total;
  int slot = block_exclusive_scan<kBlock>(__builtin_popcount(keep), scan_scratch, &chunk_total);
  uint2* dst = a.cand + (size_t)b * a.stride + chunk0;
#pragma unroll
  for (int e = 0; e < kFiltPer; ++e) {
    if ((keep >> e) & 1u) {
      dst[slot++] = make_uint2(key[e], (uint32_t)(p0 + e));
      if ((key[e] >> KT::kTopShift) == t1) atomicAdd(&ctrl[kCtrlHist2 + KT::mid(key[e])], 1u);
    }
  }
  if (threadIdx.x == 0) a.chunk_counts[(size_t)b * kMaxSelChunks + chunk] = (uint32_t)chunk_total;
}

// ------------------------------------------------------------------ final
// One block per sequence.  The top digit comes from the filter, the second
// from its low-digit histogram (one block scan), so every candidate is
// classified once: above the threshold key tau, equal to it (the first
// need_ties of those, in entry order, are selected) or below.
// Direct plan (at most 16 chunks, none with more kept than its wave holds):
// wave w requests the first 64*SPL slots of chunk w (SPL = 4, 8, 12 or 16
// per lane, chosen by the host from the expected share of K per chunk) together
// with the counts and the histogram, before any of them is known, and places its
// chunk's picks from registers after one barrier.  Otherwise the slot lists
// are concatenated in LDS (the overflow read from the lists themselves) and
// emitted in order.
// Float keys take a third digit from an LDS histogram of the candidates
// whose top 22 bits are the threshold's, counted from registers (direct) or
// from the concatenated list (general).
template <int SPL, typename KT, bool POOL>
__global__ __launch_bounds__(kSelNT) void select_final_kernel(SelectArgs a) {
  constexpr int spl = SPL;
  static_assert(kSelWaves * 64 * SPL <= 0xFFFF, "direct-plan counts fit a packed half");
  __shared__ int offs[kMaxSelChunks + 1];
  __shared__ uint2 list[kListCap];
  __shared__ int scan_scratch[kSelWaves];
  __shared__ int2 wave_tot[kSelWaves];
  __shared__ int sh[7];
  __shared__ uint32_t hist3[KT::kThree ? kBins : 1];

  const int b = blockIdx.x;
  const int n = sel_entries(a, b);
  const int K = a.K;
  if (K == 0 || n <= K) {
    select_all<KT, POOL>(a, b, n, kSelNT);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (KT::kThree)                      // visible after find_digit_in's barriers
    for (int i = tid; i < kBins; i += kSelNT) hist3[i] = 0u;
  uint32_t* h1 = a.hist1 + (size_t)b * kCtrlWords;
  uint32_t* h2 = h1 + kCtrlHist2;
  const uint32_t* counts = a.chunk_counts + (size_t)b * kMaxSelChunks;
  const uint2* cand_row = a.cand + (size_t)b * a.stride;
  int32_t* out = a.out_idx + (size_t)b * K;
  const int n_chunks = (n + kFiltChunk - 1) / kFiltChunk;
  const bool few = n_chunks <= kSelWaves;

  // this lane's spl slots of chunk `wave` (slots past the row's end read
  // entry 0 and are never used), the chunk counts, the filter's top digit
  // and the low-digit histogram, together
  uint4 sv[spl / 2];
  int my_count = 0;
  if (few) {
    if (wave < n_chunks) {
#pragma unroll
      for (int j = 0; j < spl / 2; ++j) {
        const int e = wave * kFiltChunk + spl * lane + 2 * j;
        sv[j] = *reinterpret_cast<const uint4*>(cand_row + (e < a.stride ? e : 0));
      }
    }
    my_count = lane < n_chunks ? (int)counts[lane] : 0;
  }
  // the top digit and the count above it as the filter found them, then the
  // second digit from the filter's histogram
  const int top_t1 = (int)h1[kCtrlTop], top_above1 = (int)h1[kCtrlTop + 1];
  const DigitBins<kSelNT> bins2 = load_digit_bins<kSelNT>(h2);
  if (tid == 0) {                                // visible after find_digit_in's barriers
    sh[0] = top_t1;
    sh[1] = top_above1;
    sh[6] = 0;                                   // the largest chunk count (general plan)
  }
  find_digit_in<kSelNT>(bins2, top_t1 >= 0 ? K - top_above1 : 1, scan_scratch, &sh[2], &sh[3]);
  {
    // every control word has been read (the top digit into registers, the
    // histogram before find_digit_in's barriers): zero them for the next
    // call now, while the candidates are classified
    uint4* h4 = reinterpret_cast<uint4*>(h1);
    for (int i = tid; i < kCtrlWords / 4; i += kSelNT) h4[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  // both digits exist whenever the histograms hold the sequence's n > K
  // entries; if they do not (a workspace that was not zeroed), nothing is
  // selected
  const bool have_tau = sh[0] >= 0 && sh[2] >= 0;
  uint32_t tau = have_tau ? ((uint32_t)sh[0] << 11) | (uint32_t)sh[2] : 0xFFFFFFFFu;
  int need_ties = have_tau ? K - sh[1] - sh[3] : 0;
  // float keys: tau so far is the threshold's top 22 bits; count the third
  // digit of the candidates that share them (count(f) visits each candidate
  // once), then fix the full threshold.  All threads must call.
  auto third_digit = [&](auto count) {
    if constexpr (KT::kThree) {
      const uint32_t pre = tau;
      count([&](uint32_t key) {
        if ((key >> KT::kLowBits) == pre) atomicAdd(&hist3[KT::low(key)], 1u);
      });
      __syncthreads();
      find_digit<kSelNT>(hist3, have_tau ? need_ties : 1, scan_scratch, &sh[4], &sh[5]);
      const bool ok = have_tau && sh[4] >= 0;
      tau = ok ? (pre << KT::kLowBits) | (uint32_t)sh[4] : 0xFFFFFFFFu;
      need_ties = ok ? need_ties - sh[5] : 0;
    }
  };

  int cmax = 0, off = 0;
  if (few) {
#pragma unroll
    for (int c = 0; c < kSelWaves; ++c) {
      const int v = __builtin_amdgcn_readlane(my_count, c);
      cmax = v > cmax ? v : cmax;
      off += c < wave ? v : 0;
    }
  }
  int written;
  if (few && cmax <= 64 * spl) {
    // ---- direct: wave w holds chunk w's candidates spl*lane .. spl*lane+spl-1
    const int cnt = wave < n_chunks ? __builtin_amdgcn_readlane(my_count, wave) : 0;
    uint2 e[spl];
#pragma unroll
    for (int j = 0; j < spl / 2; ++j) {
      e[2 * j] = make_uint2(sv[j].x, sv[j].y);
      e[2 * j + 1] = make_uint2(sv[j].z, sv[j].w);
    }
    third_digit([&](auto add) {
#pragma unroll
      for (int k = 0; k < spl; ++k)
        if (spl * lane + k < cnt) add(e[k].x);
    });
    uint32_t gtm = 0, tiem = 0;
#pragma unroll
    for (int k = 0; k < spl; ++k) {
      const bool live = spl * lane + k < cnt;
      gtm |= (live && e[k].x > tau) ? 1u << k : 0u;
      tiem |= (live && e[k].x == tau) ? 1u << k : 0u;
    }
    // in-wave prefix counts of this lane's picks (at most spl each)
    const uint32_t ng = __builtin_popcount(gtm), nt = __builtin_popcount(tiem);
    int gpre = 0, tpre = 0, gw = 0, tw = 0;
#pragma unroll
    for (int bit = 0; (1 << bit) <= spl; ++bit) {
      const uint64_t bg = __ballot((ng >> bit) & 1u), bt = __ballot((nt >> bit) & 1u);
      gpre += lanes_below(bg) << bit;
      tpre += lanes_below(bt) << bit;
      gw += (int)__popcll(bg) << bit;
      tw += (int)__popcll(bt) << bit;
    }
    // the waves' counts packed as above + (ties << 16) (at most 16 x 64 x
    // SPL = 16384 each), summed by DPP; scan_scratch's last reader passed a
    // barrier above
    if (lane == 0) scan_scratch[wave] = gw + (tw << 16);
    __syncthreads();
    const int2 bt = waves_before_and_total<kSelNT>(scan_scratch);
    int g = gpre + (bt.x & 0xFFFF), t = tpre + (bt.x >> 16);
    const int G = bt.y & 0xFFFF, T = bt.y >> 16;
#pragma unroll
    for (int k = 0; k < spl; ++k) {
      if ((gtm >> k) & 1u) {
        const int slot = g + (t < need_ties ? t : need_ties);
        if (slot < K) put_sel<KT, POOL>(a, b, slot, e[k]);
        ++g;
      } else if ((tiem >> k) & 1u) {
        if (t < need_ties && g + t < K) put_sel<KT, POOL>(a, b, g + t, e[k]);
        ++t;
      }
    }
    const int ties = T < need_ties ? T : need_ties;
    const int nsel = G + (ties > 0 ? ties : 0);
    written = nsel < K ? nsel : K;
  } else {
    // ---- general: concatenate the slot lists (offsets first)
    int total = 0, vmax = 0;
    for (int c0 = 0; c0 < n_chunks; c0 += kSelNT) {
      const int c = c0 + tid;
      const int v = c < n_chunks ? (int)counts[c] : 0;
      int round_total;
      const int pre = block_exclusive_scan<kSelNT>(v, scan_scratch, &round_total);
      if (c < n_chunks) offs[c] = total + pre;
      total += round_total;
      vmax = v > vmax ? v : vmax;
    }
    vmax = wave_inclusive_max(vmax);
    if (lane == 63) atomicMax(&sh[6], vmax);
    if (tid == 0) offs[n_chunks] = total;
    __syncthreads();
    // direct gather: a power-of-two group of tpc threads per chunk, each
    // taking the chunk's slots j, j + tpc, .. (kDirectPer of them), when no
    // chunk holds more than that
    const int np2 = n_chunks > 1 ? 1 << (32 - __builtin_clz((unsigned)(n_chunks - 1))) : 1;
    const int tpc = np2 <= kSelNT ? kSelNT / np2 : 0;
    if (n_chunks <= 2 * kSelWaves) {
      // few chunks: each wave walks whole chunks, its lanes over consecutive
      // candidates
      for (int c = wave; c < n_chunks; c += kSelWaves) {
        const int o = offs[c], cnt = offs[c + 1] - o;
        for (int i = lane; i < cnt && o + i < kListCap; i += 64)
          list[o + i] = cand_row[(size_t)c * kFiltChunk + i];
      }
    } else if (tpc > 0 && sh[6] <= tpc * kDirectPer) {
      const int c = tid / tpc, j = tid % tpc;
      if (c < n_chunks) {
        const int o = offs[c], cn = offs[c + 1] - o;
        uint2 v[kDirectPer];
#pragma unroll
        for (int m = 0; m < kDirectPer; ++m) {
          const int i = j + tpc * m;
          v[m] = cand_row[i < cn ? (size_t)c * kFiltChunk + i : 0];
        }
#pragma unroll
        for (int m = 0; m < kDirectPer; ++m) {
          const int i = j + tpc * m;
          if (i < cn && o + i < kListCap) list[o + i] = v[m];
        }
      }
    } else {
      // many small chunks: list slot f (< kListCap) comes from the chunk c
      // with offs[c] <= f < offs[c + 1], the largest c whose offset is at
      // most f, found by binary lifting over the offsets.  A thread's kPer
      // searches go step by step together (their LDS reads issued at once,
      // one wait per step), then every slot's load is issued at once
      // (clamped addresses, no branches), instead of one search and one
      // chunk after another
      constexpr int kPer = (kListCap + kSelNT - 1) / kSelNT;
      const int lim = total < kListCap ? total : kListCap;
      int c[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) c[q] = 0;            // offs[0] = 0 <= f
      // steps top, top/2, .., 1 reach any chunk below n_chunks
      const int top = n_chunks > 1 ? 1 << (31 - __builtin_clz((unsigned)(n_chunks - 1))) : 0;
      for (int step = top; step > 0; step >>= 1) {
        int o[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int cand = c[q] + step;
          o[q] = offs[cand < n_chunks ? cand : n_chunks];
        }
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int cand = c[q] + step;
          c[q] = (cand < n_chunks && o[q] <= tid + q * kSelNT) ? cand : c[q];
        }
      }
      int ofs[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) ofs[q] = offs[c[q]];
      uint2 v[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int f = tid + q * kSelNT;
        v[q] = cand_row[f < lim ? (size_t)c[q] * kFiltChunk + (f - ofs[q]) : 0];
      }
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int f = tid + q * kSelNT;
        if (f < lim) list[f] = v[q];
      }
    }
    __syncthreads();
    // entry f of the concatenated slot lists (already in entry order)
    auto get = [&](int f) -> uint2 {
      if (f < kListCap) return list[f];
      int lo = 0, hi = n_chunks - 1;        // largest c with offs[c] <= f
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offs[mid] <= f) lo = mid; else hi = mid - 1;
      }
      return cand_row[(size_t)lo * kFiltChunk + (f - offs[lo])];
    };
    third_digit([&](auto add) {
      for (int f = tid; f < total; f += kSelNT) add(get(f).x);
    });
    auto put = [&](int j, uint2 c) { put_sel<KT, POOL>(a, b, j, c); };
    written = total <= kListCap
                  ? emit_in_order<kSelNT>([&](int f) -> uint2 { return list[f]; }, total, tau,
                                          need_ties, K, wave_tot, put)
                  : emit_in_order<kSelNT>(get, total, tau, need_ties, K, wave_tot, put);
  }
  if constexpr (POOL) map_pool<kSelNT>(a, b, written);
  for (int j = written + tid; j < K; j += kSelNT) {
    out[j] = -1;
    if (a.out_sel_scores != nullptr) a.out_sel_scores[(size_t)b * K + j] = 0;
  }
  if (tid == 0) a.out_count[b] = written;
}

// ------------------------------------------------------------------ host
template <typename KT, bool POOL>
static hipError_t run_select_keys(const SelectArgs& a, int max_entries, hipStream_t st) {
  if (max_entries <= kSingleMax) {
    hipLaunchKernelGGL((select_single_kernel<KT, POOL>), dim3(a.batch), dim3(kSingleNT), 0, st,
                       a);
    return hipGetLastError();
  }
  const int chunks = (max_entries + kFiltChunk - 1) / kFiltChunk;
  hipLaunchKernelGGL(select_filter_kernel<KT>, dim3(chunks, a.batch), dim3(kBlock), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // candidate slots per lane in the direct plan: K's expected share of a
  // chunk, with 25% to spare, against 64 lanes x SPL
  const long long share = (long long)a.K * kFiltChunk * 5;       // x 4 * max_entries
  const long long unit = (long long)max_entries * 4 * 64;
  if (share <= unit * 4)
    hipLaunchKernelGGL((select_final_kernel<4, KT, POOL>), dim3(a.batch), dim3(kSelNT), 0, st, a);
  else if (share <= unit * 8)
    hipLaunchKernelGGL((select_final_kernel<8, KT, POOL>), dim3(a.batch), dim3(kSelNT), 0, st, a);
  else if (share <= unit * 12)
    hipLaunchKernelGGL((select_final_kernel<12, KT, POOL>), dim3(a.batch), dim3(kSelNT), 0, st,
                       a);
  else
    hipLaunchKernelGGL((select_final_kernel<16, KT, POOL>), dim3(a.batch), dim3(kSelNT), 0, st,
                       a);
  return hipGetLastError();
}

hipError_t run_select(const SelectArgs& a, int max_entries, hipStream_t st) {
  if (a.pool != nullptr)
    return a.float_keys ? run_select_keys<FloatKeys, true>(a, max_entries, st)
                        : run_select_keys<IntKeys, true>(a, max_entries, st);
  return a.float_keys ? run_select_keys<FloatKeys, false>(a, max_entries, st)
                      : run_select_keys<IntKeys, false>(a, max_entries, st);
}

}  // namespace csa2
