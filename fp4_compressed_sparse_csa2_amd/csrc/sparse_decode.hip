// csa2_sparse_decode: attention of H query heads over the selected FP4 rows
// (gathered through the page table, dequantised on the fly) merged with the
// layer's 128-token bf16 window, in one softmax.
//
// The global cache and the window cache are merged before decoding
// (infernews.com V4.1 Flash page, section 2); each layer keeps its own
// 128-token window (zulogic "DeepSeek V4 1-Flash 架构拆解", section 4); a
// Reuse layer attends with its own queries over reused indices (same page,
// section 3).  One latent row per token is both key and value.
//
// Work: a sequence's tokens form 64-token tiles -- two tiles of window rows,
// then ceil(K/64) tiles of selected FP4 rows.  A block owns one
// (sequence, group of 16 heads) and a run of consecutive tiles (a split);
// 4 waves.  All splits of one (sequence, head group) land on one XCD.
//
// The block starts by issuing every load that depends on nothing: its
// queries, its first window rows, the positions of its first four FP4 tiles
// and (when it fits in LDS) the sequence's page table.  The queries are
// converted once per block to exact f16 copies of q * 2^e (e per head) and
// staged in LDS.  The FP4 rows of a short run are all requested at once; a
// long run is a pipeline (while tile f computes, the rows of f+1, the page
// of f+3 and the position of f+4 are in flight).  Per tile, with gather lane
// (c, g) of wave w holding token 16w + c and channels [gD/4, (g+1)D/4):
//   1. dequantise its channels (FP4 -> exact E2M1 with the hardware
//      converter at scale 1.0, then an exact f16 multiply by the E4M3 scale;
//      window rows bf16 -> f16, exact) and write them to the LDS tile;
//   2. S^T for the wave's 16 tokens and the 16 heads on MFMA 16x16x32 f16
//      straight from those registers (the contraction visits the channels in
//      the order the lanes hold them, the same for the queries); tile max per
//      head through LDS;
//   3. online softmax in the exp2 domain against a reference maximum that
//      moves only when a weight would exceed 2^8, P (f16) to LDS;
//   4. wave w accumulates O[16 heads][D/4 slice] += P X with MFMA, the X
//      operand read token-major from the LDS tile by ds_read_b64_tr_b16.
// A split writes (m, l, unnormalised O); a combine kernel merges the splits
// of each (sequence, head) by their LSE, every load of a thread in flight at
// once.
#include "common.h"
#include "launch.h"

namespace csa2 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;

// Transposed LDS read: within each 16-lane group, lane i receives element
// (i % 4) of the 8 bytes addressed by lanes 4k + i/4, k = 0..3.
__device__ __forceinline__ half4 lds_read_tr(const _Float16* p) {
  return __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p));
}

constexpr int kTile = 64;                  // tokens per tile
constexpr int kHG = 16;                    // heads per block
constexpr int kPStride = kTile + 8;        // P tile row stride (halfs)
constexpr int kWinTiles = kWindow / kTile; // window tiles per sequence
constexpr int kMaxSplits = 64;
constexpr int kPtCache = 2048;             // page-table entries cached in LDS (131072 positions)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;              // softmax reference moves past this (log2 units)
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Dequantise 16 channels: 8 code bytes (two words) and their E4M3 scale s,
// given as the f16 pair {s, s}.  The hardware converter decodes E2M1 exactly
// at scale 1.0; the product with the E4M3 scale (<= 5 significant bits in
// total) is exact in f16.
__device__ __forceinline__ void dequant16(uint32_t w0, uint32_t w1, half2v s2, half8& lo,
                                          half8& hi) {
  uint4 u0, u1;
  u0.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 0) * s2);
  u0.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 1) * s2);
  u0.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 2) * s2);
  u0.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 3) * s2);
  u1.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 0) * s2);
  u1.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 1) * s2);
  u1.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 2) * s2);
  u1.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 3) * s2);
  lo = __builtin_bit_cast(half8, u0);
  hi = __builtin_bit_cast(half8, u1);
}

// Four E4M3 scale bytes (sign cleared) as two f16 pairs, exactly, by the
// hardware FP8 converter at scale 1.0.
__device__ __forceinline__ void e4m3x4_to_f16(uint32_t w, half2v& s01, half2v& s23) {
  s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w & 0x7F7F7F7Fu, 1.0f, false);
  s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w & 0x7F7F7F7Fu, 1.0f, true);
}

__device__ __forceinline__ half8 bf16x8_to_f16(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  half8 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = (_Float16)bf16_to_f32(w[k] & 0xFFFFu);
    o[2 * k + 1] = (_Float16)bf16_to_f32(w[k] >> 16);
  }
  return o;
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (one head, the 16 tokens a
// wave holds), with the gfx950 cross-row swaps instead of LDS permutes.
__device__ __forceinline__ float max_across_rows(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ uint32_t umax_across_rows(uint32_t v) {
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((uint32_t)a[0], (uint32_t)a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)c[0], (uint32_t)c[1]);
}
__device__ __forceinline__ float sum_across_rows(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// One thread's quarter of an FP4 row: D/8 code bytes and D/64 scale bytes.
template <int D>
struct RowPart {
  uint4 c[D / 128];
  uint2 s;
};

// Loads one thread's quarter of the row rowkey = (page << 6) | row; a negative
// rowkey loads row 0 of page 0 instead (always present), so that the loads of
// a pipeline stage are issued without branches.
template <int D>
__device__ __forceinline__ void load_row_part(RowPart<D>& r, const uint8_t* pages,
                                              long long rowkey, int page_bytes, int scales_off,
                                              int quarter) {
  const long long rk = rowkey < 0 ? 0 : rowkey;
  const uint8_t* page = pages + (size_t)(rk >> 6) * page_bytes;
  const int row = (int)(rk & 63);
  const uint4* cp = reinterpret_cast<const uint4*>(page + row * (D / 2) + quarter * (D / 8));
#pragma unroll
  for (int i = 0; i < D / 128; ++i) r.c[i] = cp[i];
  const uint8_t* sp = page + scales_off + row * (D / 16) + quarter * (D / 64);
  if constexpr (D == 512) {
    r.s = *reinterpret_cast<const uint2*>(sp);
  } else if constexpr (D == 256) {
    r.s = make_uint2(*reinterpret_cast<const uint32_t*>(sp), 0u);
  } else {
    r.s = make_uint2(*reinterpret_cast<const uint16_t*>(sp), 0u);
  }
}

// PTC: the sequence's page table (max_pages <= kPtCache) is staged in LDS.
template <int D, bool PTC>
__global__ __launch_bounds__(kBlock, 2) void sparse_decode_kernel(
    const uint8_t* __restrict__ pages, const int32_t* __restrict__ page_table, int num_pages,
    int max_pages, int scales_off, int page_bytes, const int32_t* __restrict__ ctx_len, int H,
    const uint16_t* __restrict__ q, float scale, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ idx_count, int K, const uint16_t* __restrict__ swa,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float2* __restrict__ part_ml, int batch, int n_splits, int split_tiles) {
  // X row stride: D halves + 24 (48 bytes), so that rows sit 48 bytes apart
  // modulo 256: the dequant writes (16 consecutive rows per 16 lanes) and the
  // transposed reads (4 rows x 32 bytes) touch distinct banks.
  constexpr int XS = D + 24;
  constexpr int QS = D + 8;                 // row stride of the staged queries
  constexpr int KQ = D / 32;                // MFMA k-steps over D for QK
  constexpr int NB = D / 64;                // 16-dim blocks per wave for PV
  constexpr int DQ = D / 4;                 // channels per lane in the gather
  constexpr int QPL = D / 16 / 8;           // uint4 of one head's query per lane in staging
  static_assert(kHG * QS <= kTile * XS, "query staging fits in the X tile");
  __shared__ __attribute__((aligned(16))) _Float16 X[kTile * XS];
  __shared__ __attribute__((aligned(16))) _Float16 Pt[kHG * kPStride];
  __shared__ __attribute__((aligned(16))) float red_max[kHG][4];
  __shared__ float red_sum[4][kHG];
  __shared__ int q_exp[kHG];
  __shared__ int pt_lds[PTC ? kPtCache : 1];

  // ---- block -> (group = (sequence, split), head group); the head groups of
  // a group share an XCD, so all but the first read its rows from L2
  const int n_hg = H / kHG;
  const int groups = batch * n_splits;
  const int xcd = blockIdx.x & 7, r8 = blockIdx.x >> 3;
  const int hg = r8 % n_hg;
  const int grp = (r8 / n_hg) * 8 + xcd;
  if (grp >= groups) return;
  const int b = grp / n_splits, split = grp % n_splits;
  const int unit = b * n_hg + hg;

  // per-sequence scalars, used only after every prologue load is issued
  const int L_raw = ctx_len[b];
  const int cnt_raw = idx_count[b];
  // This block's tiles as fixed by the plan alone: window tiles [wa, wb0)
  // and FP4 tiles [fa, fb0) of the ceil(K/64) a sequence can have.  With one
  // split a block takes them all; with several, splits 0 and 1 take one
  // window tile each and split s >= 2 takes FP4 tiles
  // [(s-2)*split_tiles, (s-1)*split_tiles).  The sequence's length and Top-K
  // count trim them later.
  const int tiles_k = (K + kTile - 1) / kTile;
  int wa = 0, wb0 = 0, fa = 0, fb0 = 0;
  if (n_splits == 1) {
    wb0 = kWinTiles;
    fb0 = tiles_k;
  } else if (split < kWinTiles) {
    wa = split;
    wb0 = split + 1;
  } else {
    fa = (split - kWinTiles) * split_tiles;
    fb0 = min(fa + split_tiles, tiles_k);
  }
  if (swa == nullptr) wb0 = wa;                          // no window rows at all

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;
  // gather: lane (lc, lg) of wave w holds token 16w + lc of the tile,
  // channels [lg*D/4, (lg+1)*D/4)
  const int tok = wave * 16 + lc;

  const int32_t* pt = page_table + (size_t)b * max_pages;
  const int32_t* idx_row = idx + (size_t)b * K;
  const uint16_t* swa_b = swa != nullptr ? swa + (size_t)b * kWindow * D : nullptr;

  // ---- prologue: every load is issued before any result is used
  // window rows by ring slot: window tile t holds slots 64t .. 64t+63 (the
  // softmax does not depend on the order of the window's tokens); slot s
  // holds a token of the window iff s < min(L, 128)
  uint4 wreg[DQ / 8];
  auto load_win = [&](int t) {
    const uint4* src =
        reinterpret_cast<const uint4*>(swa_b + (size_t)(t * kTile + tok) * D + lg * DQ);
#pragma unroll
    for (int i = 0; i < DQ / 8; ++i) wreg[i] = src[i];
  };
  if (wa < wb0) load_win(wa);
  // positions of the first FP4 tiles: unconditional loads of clamped entries
  // of the index row; which of them are real is decided from the count
  auto pos_load = [&](int f) -> int {
    const int j = f * kTile + tok;
    return idx_row[j < K ? j : K - 1];
  };
  int p0 = -1, p1 = -1, p2 = -1, p3 = -1;
  if (fa < fb0) {
    p0 = pos_load(fa);
    p1 = pos_load(fa + 1);
    p2 = pos_load(fa + 2);
    p3 = pos_load(fa + 3);
  }
  int ptv[PTC ? kPtCache / kBlock : 1];
  if (PTC && fa < fb0) {
#pragma unroll
    for (int i = 0; i < kPtCache / kBlock; ++i) {
      const int e = i * kBlock + tid;
      if (i * kBlock < max_pages) ptv[i] = pt[e < max_pages ? e : 0];
    }
  }

  // ---- queries, staged once per block: wave w converts heads 4w .. 4w+3
  // (16 lanes per head) to exact f16 copies of q * 2^e, e chosen per head so
  // that the largest |q| lands in [2^14, 2^15); the staging aliases X
  _Float16* Qs = X;
  {
    const int hq = wave * 4 + lg;                        // head within the group
    const uint16_t* src = q + ((size_t)b * H + hg * kHG + hq) * D + lc * (D / 16);
    uint4 qraw[QPL];
    uint32_t qmax = 0;
#pragma unroll
    for (int i = 0; i < QPL; ++i) {
      qraw[i] = reinterpret_cast<const uint4*>(src)[i];
      const uint32_t w[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) qmax = max(qmax, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) qmax = max(qmax, (uint32_t)__shfl_xor((int)qmax, m, 16));
    int qexp = 0;
    if (qmax != 0u) {
      int ex;
      frexpf(bf16_to_f32(qmax), &ex);     // max|q| in [2^(ex-1), 2^ex)
      qexp = 15 - ex;
    }
    if (lc == 0) q_exp[hq] = qexp;
    _Float16* dst = Qs + hq * QS + lc * (D / 16);
#pragma unroll
    for (int i = 0; i < QPL; ++i) {
      const uint32_t w[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
      half8 h;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[2 * k] = (_Float16)ldexpf(bf16_to_f32(w[k] & 0xFFFFu), qexp);
        h[2 * k + 1] = (_Float16)ldexpf(bf16_to_f32(w[k] >> 16), qexp);
      }
      *reinterpret_cast<half8*>(dst + 8 * i) = h;
    }
  }
  if (PTC && fa < fb0) {
#pragma unroll
    for (int i = 0; i < kPtCache / kBlock; ++i)
      if (i * kBlock < max_pages) pt_lds[i * kBlock + tid] = ptv[i];
  }
  __syncthreads();
  // QK operands.  The contraction over D may visit the channels in any order
  // as long as X and Q agree: k-step kk takes, in lane row lg, channels
  // lg*D/4 + 8kk .. +8, which are exactly the channels a gather lane holds,
  // so the X operand comes straight from the dequantised registers.
  // qf[kk]: head lc, channels lg*D/4 + 8kk .. +8.
  half8 qf[KQ];
#pragma unroll
  for (int kk = 0; kk < KQ; ++kk)
    qf[kk] = *reinterpret_cast<const half8*>(Qs + lc * QS + lg * DQ + 8 * kk);
  // logits in log2 units: scale2 * (q~ . x) for head lc
  const float scale2 = ldexpf(scale, -q_exp[lc]) * kLog2e;
  __syncthreads();                      // the staging area becomes the X tile

  const int L = L_raw < 0 ? 0 : (L_raw > max_pages * kPage ? max_pages * kPage : L_raw);
  const int n_glob = L > kWindow ? L - kWindow : 0;     // selectable positions
  const int cnt = cnt_raw < 0 ? 0 : (cnt_raw > K ? K : cnt_raw);
  const int n_win = swa == nullptr ? 0 : (L < kWindow ? L : kWindow);
  const int wb = min(wb0, (n_win + kTile - 1) / kTile);  // tiles that hold tokens
  const int fb = min(fb0, (cnt + kTile - 1) / kTile);
  const int nf = fb > fa ? fb - fa : 0;
  auto pos_ok = [&](int f) -> bool { return f < fb && f * kTile + tok < cnt; };
  bool ok3 = pos_ok(fa + 3);

  // page of a selected position (-1 if it is not a selectable position)
  auto page_of = [&](int p) -> int {
    const bool in = p >= 0 && p < n_glob;
    const int pi = in ? p / kPage : 0;
    const int v = PTC ? pt_lds[pi] : pt[pi];
    return in ? v : -1;
  };
  auto rowkey_of = [&](int p, int pg) -> long long {
    return (p >= 0 && pg >= 0 && pg < num_pages) ? ((long long)pg << 6) | (p & (kPage - 1)) : -1;
  };
  int pg2 = -1;
  long long rk0 = -1, rk1 = -1;
  RowPart<D> cur, nxt;
  if (fa < fb) {
    p0 = pos_ok(fa) ? p0 : -1;
    p1 = pos_ok(fa + 1) ? p1 : -1;
    p2 = pos_ok(fa + 2) ? p2 : -1;
    const int pg0 = page_of(p0), pg1 = page_of(p1);
    pg2 = page_of(p2);
    rk0 = rowkey_of(p0, pg0);
    rk1 = rowkey_of(p1, pg1);
    load_row_part<D>(cur, pages, rk0, page_bytes, scales_off, lg);
  }

  // running softmax state of head lc (every lane of the head holds the same);
  // acc[nb] holds O^T[dims wave*DQ + 16nb + 4lg + i][head lc]
  float m_q = -INFINITY, l_q = 0.0f;
  floatx4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // ---- the rest of a tile once this wave's S^T (tokens 16*wave + 4lg + i,
  // head lc) is known and the tile's rows are being written to X; bit i of
  // vbits marks token 16*wave + 4lg + i as real
  auto finish_tile = [&](floatx4 s, uint32_t vbits) {
    float lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = ((vbits >> i) & 1u) ? s[i] * scale2 : -INFINITY;
      lmax = fmaxf(lmax, s[i]);
    }
    lmax = max_across_rows(lmax);
    if (lg == 0) red_max[lc][wave] = lmax;
    __syncthreads();                    // also: the whole X tile is written

    // online softmax of head lc with a lazily moved reference: the weights
    // are exp2(s - m_ref), and m_ref moves (rescaling l and O) only when a
    // tile's maximum exceeds it by more than kLazy, so the weights stay below
    // 2^kLazy (f16 holds them to the same relative precision) and the
    // rescale of the accumulators is rare.  All waves take the same decision
    // from the same maxima.
    const float4 rm = *reinterpret_cast<const float4*>(&red_max[lc][0]);
    const float mt = fmaxf(fmaxf(rm.x, rm.y), fmaxf(rm.z, rm.w));
    const bool first = m_q == -INFINITY;                 // l and O are still zero
    const float m_new = (first || mt > m_q + kLazy) ? mt : m_q;
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = first ? 1.0f : exp2f(m_q - m_use);
    float psum = 0.f;
    half4 ph;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 p16 = (_Float16)exp2f(s[i] - m_use);
      ph[i] = p16;
      psum += (float)p16;               // the weights the PV product actually uses
    }
    l_q = l_q * alpha + sum_across_rows(psum);
    m_q = m_new;
    *reinterpret_cast<half4*>(Pt + lc * kPStride + wave * 16 + lg * 4) = ph;
    if (__ballot(alpha != 1.0f)) {      // wave-uniform: skipped once the maxima settle
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] *= alpha;
    }
    __syncthreads();

    // O^T[wave's D/4 dims][16 heads] += X^T P^T
#pragma unroll
    for (int kb = 0; kb < kTile / 32; ++kb) {
      const half8 pb = *reinterpret_cast<const half8*>(Pt + lc * kPStride + kb * 32 + lg * 8);
      const int tok0 = kb * 32 + lg * 8 + (lc >> 2);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = wave * DQ + nb * 16 + 4 * (lc & 3);
        const half4 b0 = lds_read_tr(X + tok0 * XS + col);
        const half4 b1 = lds_read_tr(X + (tok0 + 4) * XS + col);
        const half8 xt = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xt, pb, acc[nb], 0, 0, 0);
      }
    }
    __syncthreads();
  };

  _Float16* xrow = X + tok * XS + lg * DQ;

  // ---- window tiles (their rows were requested in the prologue)
#pragma unroll 1
  for (int t = wa; t < wb; ++t) {
    const bool ok = t * kTile + tok < n_win;
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      const half8 x = ok ? bf16x8_to_f16(wreg[kk]) : half8{};
      *reinterpret_cast<half8*>(xrow + 8 * kk) = x;
      if (kk & 1) s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, qf[kk], s1, 0, 0, 0);
      else        s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, qf[kk], s0, 0, 0, 0);
    }
    const uint32_t vbits = (uint32_t)(__ballot(ok) >> (4 * lg)) & 0xFu;
    if (t + 1 < wb) load_win(t + 1);    // in flight while this tile computes
    finish_tile(s0 + s1, vbits);
  }

  // ---- FP4 tiles
  auto fp4_tile = [&](const RowPart<D>& rp, long long rk) {
    // the E4M3 scales of this lane's groups as f16; a token that is not
    // real gets scale 0, so that its X row is exactly zero whatever the
    // bytes it loaded (its weight in P is zero as well)
    const bool ok = rk >= 0;
    half2v sc[4];
    e4m3x4_to_f16(ok ? rp.s.x : 0u, sc[0], sc[1]);
    if constexpr (D / 64 > 4) e4m3x4_to_f16(ok ? rp.s.y : 0u, sc[2], sc[3]);
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < DQ / 16; ++g) {
      const uint4 c4 = rp.c[g / 2];
      const uint32_t w0 = (g & 1) ? c4.z : c4.x, w1 = (g & 1) ? c4.w : c4.y;
      const half2v sp = sc[g / 2];
      const half2v s2 = (g & 1) ? __builtin_shufflevector(sp, sp, 1, 1)
                                : __builtin_shufflevector(sp, sp, 0, 0);
      half8 lo, hi;
      dequant16(w0, w1, s2, lo, hi);
      *reinterpret_cast<half8*>(xrow + 16 * g) = lo;
      *reinterpret_cast<half8*>(xrow + 16 * g + 8) = hi;
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, qf[2 * g], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, qf[2 * g + 1], s1, 0, 0, 0);
    }
    const uint32_t vbits = (uint32_t)(__ballot(ok) >> (4 * lg)) & 0xFu;
    finish_tile(s0 + s1, vbits);
  };
  if (nf > 0 && nf <= 4) {
    // a short run: every row of the run is requested at once
    const long long rk3 = rowkey_of(ok3 ? p3 : -1, page_of(ok3 ? p3 : -1));
    const long long rk2 = rowkey_of(p2, pg2);
    RowPart<D> r1, r2, r3;
    if (nf > 1) load_row_part<D>(r1, pages, rk1, page_bytes, scales_off, lg);
    if (nf > 2) load_row_part<D>(r2, pages, rk2, page_bytes, scales_off, lg);
    if (nf > 3) load_row_part<D>(r3, pages, rk3, page_bytes, scales_off, lg);
    fp4_tile(cur, rk0);
    if (nf > 1) fp4_tile(r1, rk1);
    if (nf > 2) fp4_tile(r2, rk2);
    if (nf > 3) fp4_tile(r3, rk3);
  } else {
    // a long run: a pipeline position -> page -> row address -> rows, so that
    // tile f computes while the rows of f+1, the page of f+3 and the position
    // of f+4 are on their way
#pragma unroll 1
    for (int f = fa; f < fb; ++f) {
      load_row_part<D>(nxt, pages, rk1, page_bytes, scales_off, lg);
      const long long rk2 = rowkey_of(p2, pg2);
      const int pg3 = page_of(ok3 ? p3 : -1);
      const int p4 = pos_load(f + 4);          // consumed next iteration
      const bool ok4 = pos_ok(f + 4);
      fp4_tile(cur, rk0);
      rk0 = rk1;
      rk1 = rk2;
      p2 = ok3 ? p3 : -1;
      pg2 = pg3;
      p3 = p4;
      ok3 = ok4;
      cur = nxt;
    }
  }

  // ---- finish: total l of head lc across waves (every wave saw the same m)
  if (lg == 0) red_sum[wave][lc] = l_q;
  __syncthreads();
  const float l_tot = red_sum[0][lc] + red_sum[1][lc] + red_sum[2][lc] + red_sum[3][lc];
  const int head = hg * kHG + lc;
  if (n_splits == 1) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.0f;
    float* orow = out + ((size_t)b * H + head) * D + wave * DQ + 4 * lg;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<floatx4*>(orow + nb * 16) = acc[nb] * inv;
    if (wave == 0 && lg == 0 && lse != nullptr)
      lse[(size_t)b * H + head] = l_tot > 0.f ? (m_q + log2f(l_tot)) * kLn2 : -INFINITY;
    return;
  }

  // ---- split partials: (m, l) per head and the unnormalised O, stored
  // non-temporally (read once, by the combine kernel)
  const size_t prow = ((size_t)unit * n_splits + split) * kHG + lc;   // partial row of head lc
  float* orow = part_o + prow * D + wave * DQ + 4 * lg;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    __builtin_nontemporal_store(acc[nb], reinterpret_cast<floatx4*>(orow + nb * 16));
  if (wave == 0 && lg == 0) part_ml[prow] = make_float2(m_q, l_tot);
}

// LSE merge of the split partials.  Block = (unit, HPB heads); thread = one
// float4 of one head's output; every load of a batch of 16 splits is issued
// before any is used.
template <int D>
__global__ __launch_bounds__(kBlock) void sparse_combine_kernel(
    const float* __restrict__ part_o, const float2* __restrict__ part_ml, int H, int n_splits,
    float* __restrict__ out, float* __restrict__ lse) {
  constexpr int T4 = D / 4;                 // threads per head
  constexpr int HPB = kBlock / T4;          // heads per block
  constexpr int SB = 16;                    // splits per batch of loads
  const int n_hg = H / kHG;
  const int unit = blockIdx.x / (kHG / HPB);
  const int h = (blockIdx.x % (kHG / HPB)) * HPB + (int)threadIdx.x / T4;
  const int d4 = (int)threadIdx.x % T4;
  const int b = unit / n_hg, hg = unit % n_hg;
  const size_t ubase = (size_t)unit * n_splits;
  const size_t ostep = (size_t)kHG * D / 4;             // float4s from one split to the next
  const float4* src = reinterpret_cast<const float4*>(part_o + (ubase * kHG + h) * D) + d4;

  float M = -INFINITY, Lsum = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < n_splits; s0 += SB) {
    float2 ml[SB];
    float4 x[SB];
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      if (s0 + i < n_splits) {
        ml[i] = part_ml[(ubase + s0 + i) * kHG + h];
        const floatx4 t =       // partials are read once: non-temporal
            __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(src + (s0 + i) * ostep));
        x[i] = make_float4(t.x, t.y, t.z, t.w);
      } else {
        ml[i] = make_float2(-INFINITY, 0.f);
        x[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float mb = M;
#pragma unroll
    for (int i = 0; i < SB; ++i)
      if (ml[i].y > 0.f) mb = fmaxf(mb, ml[i].x);
    if (mb == -INFINITY) continue;                      // nothing with weight yet
    const float r = M == -INFINITY ? 0.f : exp2f(M - mb);
    Lsum *= r;
    a.x *= r;
    a.y *= r;
    a.z *= r;
    a.w *= r;
    M = mb;
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const float w = ml[i].y > 0.f ? exp2f(ml[i].x - M) : 0.f;
      Lsum += w * ml[i].y;
      a.x += w * x[i].x;
      a.y += w * x[i].y;
      a.z += w * x[i].z;
      a.w += w * x[i].w;
    }
  }
  const float il = Lsum > 0.f ? 1.0f / Lsum : 0.0f;
  const size_t orow = (size_t)b * H + hg * kHG + h;
  reinterpret_cast<float4*>(out + orow * D)[d4] = make_float4(a.x * il, a.y * il, a.z * il, a.w * il);
  if (d4 == 0 && lse != nullptr) lse[orow] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ host
struct DecodePlan {
  int n_splits, split_tiles;
};

#ifndef CSA2_DECODE_MIN_SPLIT_TILES
#define CSA2_DECODE_MIN_SPLIT_TILES 3
#endif

// Splits: with at least 256 (sequence, head group) units one block per unit
// takes all of a sequence's tiles.  Otherwise two one-tile splits take the window tiles
// and FP4 runs of split_tiles tiles fill the rest, enough of them to keep the
// grid near one resident wave of blocks (two per CU on 256 CUs) but at least
// CSA2_DECODE_MIN_SPLIT_TILES tiles per run, so that the partials stay small
// next to the work, and at most kMaxSplits splits.
static DecodePlan plan_decode(int batch, int H, int K) {
  const int tiles = (K + kTile - 1) / kTile;             // FP4 tiles
  const int units = batch * (H / kHG);
  if (units >= 256 || tiles == 0) return DecodePlan{1, tiles + kWinTiles};
  int tps = (tiles * units + 511) / 512;
  if (tps < CSA2_DECODE_MIN_SPLIT_TILES) tps = CSA2_DECODE_MIN_SPLIT_TILES;
  const int min_tps = (tiles + kMaxSplits - kWinTiles - 1) / (kMaxSplits - kWinTiles);
  if (tps < min_tps) tps = min_tps;
  if (tps > tiles) tps = tiles;
  return DecodePlan{kWinTiles + (tiles + tps - 1) / tps, tps};
}

struct DecodeWs {
  size_t part_o, part_ml, total;
};
static DecodeWs decode_ws(int batch, int H, int D, int K) {
  const DecodePlan pl = plan_decode(batch, H, K);
  const size_t units = (size_t)batch * (H / kHG);
  const size_t rows = units * pl.n_splits * kHG;
  auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  DecodeWs w;
  w.part_ml = 0;
  w.part_o = a256(rows * 8);
  w.total = pl.n_splits > 1 ? w.part_o + a256(rows * D * 4) : 256;
  return w;
}

size_t sparse_decode_ws_bytes(int batch, int H, int D, int K) {
  return decode_ws(batch, H, D, K).total;
}

template <int D>
static void launch_decode(const CacheArgs& c, const int32_t* ctx_len, int H, const uint16_t* q,
                          float scale, const int32_t* idx, const int32_t* idx_count, int K,
                          const uint16_t* swa, float* out, float* lse, uint8_t* ws,
                          hipStream_t st) {
  const PageLayout lay = page_layout(D, c.Di);
  const DecodePlan pl = plan_decode(c.batch, H, K);
  const DecodeWs w = decode_ws(c.batch, H, D, K);
  const int units = c.batch * (H / kHG);
  const int groups = c.batch * pl.n_splits;
  const int blocks = ((groups + 7) / 8) * 8 * (H / kHG);
  auto kern = c.max_pages <= kPtCache ? sparse_decode_kernel<D, true>
                                      : sparse_decode_kernel<D, false>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kBlock), 0, st, (const uint8_t*)c.pages,
                     c.page_table, c.num_pages, c.max_pages, lay.scales_off, lay.page_bytes,
                     ctx_len, H, q, scale, idx, idx_count, K, swa, out, lse,
                     reinterpret_cast<float*>(ws + w.part_o),
                     reinterpret_cast<float2*>(ws + w.part_ml), c.batch, pl.n_splits,
                     pl.split_tiles);
  if (pl.n_splits > 1) {
    constexpr int HPB = kBlock / (D / 4);
    hipLaunchKernelGGL((sparse_combine_kernel<D>), dim3(units * (kHG / HPB)), dim3(kBlock), 0, st,
                       reinterpret_cast<const float*>(ws + w.part_o),
                       reinterpret_cast<const float2*>(ws + w.part_ml), H, pl.n_splits, out, lse);
  }
}

hipError_t run_sparse_decode(const CacheArgs& c, const int32_t* ctx_len, int H,
                             const uint16_t* q, float scale, const int32_t* idx,
                             const int32_t* idx_count, int K, const uint16_t* swa, float* out,
                             float* lse, void* ws, hipStream_t st) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  switch (c.D) {
    case 128: launch_decode<128>(c, ctx_len, H, q, scale, idx, idx_count, K, swa, out, lse, w, st); break;
    case 256: launch_decode<256>(c, ctx_len, H, q, scale, idx, idx_count, K, swa, out, lse, w, st); break;
    case 512: launch_decode<512>(c, ctx_len, H, q, scale, idx, idx_count, K, swa, out, lse, w, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace csa2
