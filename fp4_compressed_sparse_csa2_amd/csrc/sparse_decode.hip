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
// (sequence, group of HG heads) and a run of consecutive tiles (a split);
// 4 waves.  HG is 64 where the heads allow it, so that every dequantised
// row feeds four head blocks of MFMAs (the dequantisation and the LDS
// round trip of the X tile are paid once per 64 heads, not once per 16);
// small batches take 16-head groups and token splits instead, to fill the
// chip.  All splits of one (sequence, head group) land on one XCD.
//
// The block starts by issuing every load that depends on nothing: its
// queries, its first window rows, the positions of its first four FP4 tiles
// and (when it fits in LDS) the sequence's page table.  The queries are
// converted once per block to exact f16 copies of q * 2^e (e per head) and
// kept in registers (HG/16 head blocks x D/32 k-steps of MFMA operands).  The
// FP4 rows of a short run are all requested at once; a long run is a
// pipeline (while tile f computes, the rows of f+1, the page of f+3 and the
// position of f+4 are in flight).  Per tile, with gather lane (c, g) of wave
// w holding token 16w + c and channels [gD/4, (g+1)D/4) -- one contiguous
// run of its FP4 row (codes, then the scales after the codes):
//   1. dequantise its channels (FP4 -> exact E2M1 with the hardware
//      converter at scale 1.0, then an exact f16 multiply by the E4M3 scale;
//      window rows bf16 -> f16) and write them to the LDS tile;
//   2. S^T for the wave's 16 tokens and each head block on MFMA 16x16x32 f16
//      straight from those registers (the contraction visits the channels in
//      the order the lanes hold them, the same for the queries); tile max per
//      head through LDS;
//   3. online softmax in the exp2 domain against a reference maximum that
//      moves only when a weight would exceed 2^8, P (f16) to LDS;
//   4. wave w accumulates O[HG heads][D/4 slice] += P X with MFMA, each X
//      operand read token-major from the LDS tile by ds_read_b64_tr_b16 and
//      used for every head block.
// A split writes (m, l, unnormalised O); a combine kernel merges the splits
// of each (sequence, head) by their LSE, every load of a thread in flight at
// once.
#include <stdlib.h>

#include "common.h"
#include "launch.h"

namespace csa2 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;

// Transposed LDS read: within each 16-lane group, lane i receives element
// (i % 4) of the 8 bytes addressed by lanes 4k + i/4, k = 0..3.
__device__ __forceinline__ half4 lds_read_tr(const _Float16* p) {
  return __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p));
}

constexpr int kTile = 64;                  // tokens per tile
constexpr int kPStride = kTile + 8;        // P tile row stride (halfs)
constexpr int kWinTiles = kWindow / kTile; // window tiles per sequence
constexpr int kMaxSplits = 64;
constexpr int kPtCache = 1024;             // page-table entries cached in LDS (65536 positions)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;              // softmax reference moves past this (log2 units)
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// 2^x by the hardware instruction alone (no range reduction): the arguments
// here are at most kLazy (a softmax weight against its reference) or at most
// 0 (a rescale factor); -inf gives 0, and results below the float range
// flush to 0, which only drops weights below 2^-126 of the largest.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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
__device__ __forceinline__ float sum_across_rows(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// The tiles of split `split`: window tiles [wa, wb0) and FP4 tiles [fa, fb0)
// of the kWinTiles + ceil(K/64) a sequence can have (its length and Top-K
// count trim them later).  One split takes them all.  With win_sep, splits
// 0 and 1 take one window tile each and split s >= 2 the FP4 run
// [(s-2)*split_tiles, (s-1)*split_tiles); otherwise split s takes the run
// [s*split_tiles, (s+1)*split_tiles) of the list window tiles, then FP4 tiles.
struct TileRange {
  int wa, wb0, fa, fb0;
};
__device__ __forceinline__ TileRange split_range(int split, int n_splits, int split_tiles,
                                                 int tiles_k, int win_sep) {
  if (n_splits == 1) return TileRange{0, kWinTiles, 0, tiles_k};
  if (win_sep) {
    if (split < kWinTiles) return TileRange{split, split + 1, 0, 0};
    const int fa = (split - kWinTiles) * split_tiles;
    return TileRange{0, 0, fa, min(fa + split_tiles, tiles_k)};
  }
  const int ls = split * split_tiles;
  const int le = min(ls + split_tiles, kWinTiles + tiles_k);
  return TileRange{min(ls, kWinTiles), min(le, kWinTiles), max(ls - kWinTiles, 0),
                   max(le - kWinTiles, 0)};
}

// One thread's quarter of an FP4 row: D/8 code bytes and D/64 scale bytes.
template <int D>
struct RowPart {
  uint4 c[D / 128];
  uint2 s;
};

// Loads one thread's quarter of the row rowkey = (page << 6) | row; a negative
// rowkey loads row 0 of page 0 instead (always present), so that the loads of
// a pipeline stage are issued without branches.  A row is R = D/2 + D/16
// contiguous bytes (codes, then scales); quarter g takes code bytes
// [gD/8, (g+1)D/8) and scale bytes D/2 + [gD/64, (g+1)D/64).  At D = 128 a
// row start is only 8-byte aligned, so the codes go in two 8-byte loads.
template <int D>
__device__ __forceinline__ void load_row_part(RowPart<D>& r, const uint8_t* pages,
                                              long long rowkey, int page_bytes, int quarter) {
  constexpr int R = D / 2 + D / 16;
  const long long rk = rowkey < 0 ? 0 : rowkey;
  const uint8_t* row = pages + (size_t)(rk >> 6) * page_bytes + (int)(rk & 63) * R;
  const uint8_t* cp = row + quarter * (D / 8);
  const uint8_t* sp = row + D / 2 + quarter * (D / 64);
  if constexpr (D == 512) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.c[i] = reinterpret_cast<const uint4*>(cp)[i];
    r.s = *reinterpret_cast<const uint2*>(sp);
  } else if constexpr (D == 256) {
#pragma unroll
    for (int i = 0; i < 2; ++i) r.c[i] = reinterpret_cast<const uint4*>(cp)[i];
    r.s = make_uint2(*reinterpret_cast<const uint32_t*>(sp), 0u);
  } else {
    const uint2 a = reinterpret_cast<const uint2*>(cp)[0], b = reinterpret_cast<const uint2*>(cp)[1];
    r.c[0] = make_uint4(a.x, a.y, b.x, b.y);
    r.s = make_uint2(*reinterpret_cast<const uint16_t*>(sp), 0u);
  }
}

// PTC: the sequence's page table (max_pages <= kPtCache) is staged in LDS.
// HG: heads per block (16, 32 or 64).  With 64 heads the query operands and
// accumulators take about 400 registers, so a block holds its CU alone (one
// wave per SIMD); with 16, two blocks share a CU.
template <int D, int HG, bool PTC>
__global__ __launch_bounds__(kBlock, HG == 16 ? 2 : 1) void sparse_decode_kernel(
    const uint8_t* __restrict__ pages, const int32_t* __restrict__ page_table, int num_pages,
    int max_pages, int page_bytes, const int32_t* __restrict__ ctx_len, int H,
    const uint16_t* __restrict__ q, float scale, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ idx_count, int K, const uint16_t* __restrict__ swa,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float2* __restrict__ part_ml, int batch, int n_splits, int split_tiles, int win_sep) {
  // X row stride: D halves + 24 (48 bytes), so that rows sit 48 bytes apart
  // modulo 256: the dequant writes (16 consecutive rows per 16 lanes) and the
  // transposed reads (4 rows x 32 bytes) touch distinct banks.
  constexpr int XS = D + 24;
  constexpr int QS = D + 8;                 // row stride of the staged queries
  constexpr int KQ = D / 32;                // MFMA k-steps over D for QK
  constexpr int NB = D / 64;                // 16-dim blocks per wave for PV
  constexpr int DQ = D / 4;                 // channels per lane in the gather
  constexpr int QPL = D / 16 / 8;           // uint4 of one head's query per lane in staging
  constexpr int HB = HG / 16;               // head blocks
  static_assert(HG * QS <= kTile * XS, "query staging fits in the X tile");
  __shared__ __attribute__((aligned(16))) _Float16 X[kTile * XS];
  __shared__ __attribute__((aligned(16))) _Float16 Pt[HG * kPStride];
  __shared__ __attribute__((aligned(16))) float red_max[HG][4];
  __shared__ float red_sum[4][HG];
  __shared__ int q_exp[HG];
  __shared__ int pt_lds[PTC ? kPtCache : 1];

  // ---- block -> (group = (sequence, split), head group); the head groups of
  // a group share an XCD, so all but the first read its rows from L2
  const int n_hg = H / HG;
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
  // this block's tiles as fixed by the plan alone
  const int tiles_k = (K + kTile - 1) / kTile;
  const TileRange tr = split_range(split, n_splits, split_tiles, tiles_k, win_sep);
  const int wa = tr.wa, fa = tr.fa, fb0 = tr.fb0;
  const int wb0 = swa == nullptr ? wa : tr.wb0;           // no window rows at all                          // no window rows at all

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;
  // gather: lane (lc, lg) of wave w holds token 16w + lc of the tile,
  // channels [lg*D/4, (lg+1)*D/4)
  const int tok = wave * 16 + lc;

  const int32_t* pt = page_table + (size_t)b * max_pages;
  const int32_t* idx_row = idx + (size_t)b * K;
  const uint16_t* swa_b = swa != nullptr ? swa + (size_t)b * kWindow * D : nullptr;

  // ---- prologue: every load is issued before any result is used
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

  // ---- queries: every load issued now; converted (below) once the rows of
  // the first FP4 tile are requested
  uint4 qraw[HB][QPL];
#pragma unroll
  for (int round = 0; round < HB; ++round) {
    const int hq = round * 16 + wave * 4 + lg;           // head within the group
    const uint16_t* src = q + ((size_t)b * H + hg * HG + hq) * D + lc * (D / 16);
#pragma unroll
    for (int i = 0; i < QPL; ++i) qraw[round][i] = reinterpret_cast<const uint4*>(src)[i];
  }
  if (PTC) {
    if (fa < fb0) {
#pragma unroll
      for (int i = 0; i < kPtCache / kBlock; ++i)
        if (i * kBlock < max_pages) pt_lds[i * kBlock + tid] = ptv[i];
    }
    __syncthreads();                    // the page table is in LDS
  }

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
  // the first FP4 tile's rows, requested unconditionally (a block with no
  // FP4 tile loads row 0 of page 0 and never uses it), so that no branch
  // makes the query conversion below wait for them
  p0 = pos_ok(fa) ? p0 : -1;
  p1 = pos_ok(fa + 1) ? p1 : -1;
  p2 = pos_ok(fa + 2) ? p2 : -1;
  int pg2 = page_of(p2);
  long long rk0 = rowkey_of(p0, page_of(p0)), rk1 = rowkey_of(p1, page_of(p1));
  RowPart<D> cur, nxt;
  load_row_part<D>(cur, pages, rk0, page_bytes, lg);

  // queries, staged once per block: per round, wave w converts 4 heads (16
  // lanes per head) to exact f16 copies of q * 2^e, e chosen per head so
  // that the largest |q| lands in [2^14, 2^15); the staging aliases X
  _Float16* Qs = X;
#pragma unroll
  for (int round = 0; round < HB; ++round) {
    const int hq = round * 16 + wave * 4 + lg;           // head within the group
    uint32_t qmax = 0;
#pragma unroll
    for (int i = 0; i < QPL; ++i) {
      const uint32_t w[4] = {qraw[round][i].x, qraw[round][i].y, qraw[round][i].z,
                             qraw[round][i].w};
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
      const uint32_t w[4] = {qraw[round][i].x, qraw[round][i].y, qraw[round][i].z,
                             qraw[round][i].w};
      half8 h;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[2 * k] = (_Float16)ldexpf(bf16_to_f32(w[k] & 0xFFFFu), qexp);
        h[2 * k + 1] = (_Float16)ldexpf(bf16_to_f32(w[k] >> 16), qexp);
      }
      *reinterpret_cast<half8*>(dst + 8 * i) = h;
    }
  }
  __syncthreads();
  // QK operands.  The contraction over D may visit the channels in any order
  // as long as X and Q agree: k-step kk takes, in lane row lg, channels
  // lg*D/4 + 8kk .. +8, which are exactly the channels a gather lane holds,
  // so the X operand comes straight from the dequantised registers.
  // qf[hb][kk]: head 16hb + lc, channels lg*D/4 + 8kk .. +8.
  half8 qf[HB][KQ];
  float scale2[HB];                       // logits in log2 units: scale2 * (q~ . x)
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk)
      qf[hb][kk] = *reinterpret_cast<const half8*>(Qs + (hb * 16 + lc) * QS + lg * DQ + 8 * kk);
    scale2[hb] = ldexpf(scale, -q_exp[hb * 16 + lc]) * kLog2e;
  }
  __syncthreads();                      // the staging area becomes the X tile

  // running softmax state of head 16hb + lc (every lane of the head holds
  // the same); acc[hb][nb] holds O^T[dims wave*DQ + 16nb + 4lg + i][head 16hb + lc]
  float m_q[HB], l_q[HB];
  floatx4 acc[HB][NB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    m_q[hb] = -INFINITY;
    l_q[hb] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[hb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- the rest of a tile once this wave's S^T (tokens 16*wave + 4lg + i,
  // head 16hb + lc) is known and the tile's rows are being written to X; bit
  // i of vbits marks token 16*wave + 4lg + i as real
  auto finish_tile = [&](floatx4 (&s)[HB], uint32_t vbits) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float lmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[hb][i] = ((vbits >> i) & 1u) ? s[hb][i] * scale2[hb] : -INFINITY;
        lmax = fmaxf(lmax, s[hb][i]);
      }
      lmax = max_across_rows(lmax);
      if (lg == 0) red_max[hb * 16 + lc][wave] = lmax;
    }
    __syncthreads();                    // also: the whole X tile is written

    // online softmax of head 16hb + lc with a lazily moved reference: the
    // weights are exp2(s - m_ref), and m_ref moves (rescaling l and O) only
    // when a tile's maximum exceeds it by more than kLazy, so the weights
    // stay below 2^kLazy (f16 holds them to the same relative precision) and
    // the rescale of the accumulators is rare.  All waves take the same
    // decision from the same maxima.
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const float4 rm = *reinterpret_cast<const float4*>(&red_max[hb * 16 + lc][0]);
      const float mt = fmaxf(fmaxf(rm.x, rm.y), fmaxf(rm.z, rm.w));
      const bool first = m_q[hb] == -INFINITY;           // l and O are still zero
      const bool moves = !first && mt > m_q[hb] + kLazy;
      const float m_new = (first || moves) ? mt : m_q[hb];
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      float alpha = 1.0f;
      if (__ballot(moves)) alpha = moves ? fast_exp2(m_q[hb] - m_use) : 1.0f;
      float psum = 0.f;
      half4 ph;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 p16 = (_Float16)fast_exp2(s[hb][i] - m_use);
        ph[i] = p16;
        psum += (float)p16;             // the weights the PV product actually uses
      }
      l_q[hb] = l_q[hb] * alpha + sum_across_rows(psum);
      m_q[hb] = m_new;
      *reinterpret_cast<half4*>(Pt + (hb * 16 + lc) * kPStride + wave * 16 + lg * 4) = ph;
      if (__ballot(alpha != 1.0f)) {    // wave-uniform: skipped once the maxima settle
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[hb][nb] *= alpha;
      }
    }
    __syncthreads();

    // O^T[wave's D/4 dims][HG heads] += X^T P^T
#pragma unroll
    for (int kb = 0; kb < kTile / 32; ++kb) {
      half8 pb[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
        pb[hb] = *reinterpret_cast<const half8*>(Pt + (hb * 16 + lc) * kPStride + kb * 32 + lg * 8);
      const int tok0 = kb * 32 + lg * 8 + (lc >> 2);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = wave * DQ + nb * 16 + 4 * (lc & 3);
        const half4 b0 = lds_read_tr(X + tok0 * XS + col);
        const half4 b1 = lds_read_tr(X + (tok0 + 4) * XS + col);
        const half8 xt = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          acc[hb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xt, pb[hb], acc[hb][nb], 0, 0, 0);
      }
    }
    __syncthreads();
  };

  _Float16* xrow = X + tok * XS + lg * DQ;

  // ---- window tiles: window tile t holds ring slots 64t .. 64t+63 (the
  // softmax does not depend on the order of the window's tokens); slot s
  // holds a token of the window iff s < min(L, 128).  A lane's D/4 channels
  // of bf16 come in chunks of 16-byte loads (four, or two with 64 heads), the
  // next chunk in flight while one is converted.
  constexpr int WC = HG == 16 ? (DQ / 8 >= 4 ? 4 : DQ / 8) : 2;   // uint4 per chunk
  constexpr int NWC = DQ / 8 / WC;                       // chunks per row part
#pragma unroll 1
  for (int t = wa; t < wb; ++t) {
    const bool ok = t * kTile + tok < n_win;
    const uint4* src = reinterpret_cast<const uint4*>(swa_b + (size_t)(t * kTile + tok) * D + lg * DQ);
    uint4 wc[2][WC];
#pragma unroll
    for (int i = 0; i < WC; ++i) wc[0][i] = src[i];
    floatx4 s[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) s[hb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NWC; ++c) {
      if (c + 1 < NWC) {
#pragma unroll
        for (int i = 0; i < WC; ++i) wc[(c + 1) & 1][i] = src[(c + 1) * WC + i];
      }
#pragma unroll
      for (int i = 0; i < WC; ++i) {
        const int kk = c * WC + i;
        const half8 x = ok ? bf16x8_to_f16(wc[c & 1][i]) : half8{};
        *reinterpret_cast<half8*>(xrow + 8 * kk) = x;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          s[hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, qf[hb][kk], s[hb], 0, 0, 0);
      }
    }
    const uint32_t vbits = (uint32_t)(__ballot(ok) >> (4 * lg)) & 0xFu;
    finish_tile(s, vbits);
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
    floatx4 s[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) s[hb] = floatx4{0.f, 0.f, 0.f, 0.f};
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
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        s[hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, qf[hb][2 * g], s[hb], 0, 0, 0);
        s[hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, qf[hb][2 * g + 1], s[hb], 0, 0, 0);
      }
    }
    const uint32_t vbits = (uint32_t)(__ballot(ok) >> (4 * lg)) & 0xFu;
    finish_tile(s, vbits);
  };
  if (HG == 16 && nf > 0 && nf <= 4) {
    // a short run: every row of the run is requested at once (16-head blocks
    // only; with 64 heads the registers hold one row part in flight)
    const long long rk3 = rowkey_of(ok3 ? p3 : -1, page_of(ok3 ? p3 : -1));
    const long long rk2 = rowkey_of(p2, pg2);
    RowPart<D> r1, r2, r3;
    if (nf > 1) load_row_part<D>(r1, pages, rk1, page_bytes, lg);
    if (nf > 2) load_row_part<D>(r2, pages, rk2, page_bytes, lg);
    if (nf > 3) load_row_part<D>(r3, pages, rk3, page_bytes, lg);
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
      load_row_part<D>(nxt, pages, rk1, page_bytes, lg);
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

  // ---- finish: total l of each head across waves (every wave saw the same m)
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
    if (lg == 0) red_sum[wave][hb * 16 + lc] = l_q[hb];
  __syncthreads();
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int hl = hb * 16 + lc;                         // head within the group
    const float l_tot = red_sum[0][hl] + red_sum[1][hl] + red_sum[2][hl] + red_sum[3][hl];
    const int head = hg * HG + hl;
    if (n_splits == 1) {
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.0f;
      float* orow = out + ((size_t)b * H + head) * D + wave * DQ + 4 * lg;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        *reinterpret_cast<floatx4*>(orow + nb * 16) = acc[hb][nb] * inv;
      if (wave == 0 && lg == 0 && lse != nullptr)
        lse[(size_t)b * H + head] = l_tot > 0.f ? (m_q[hb] + log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
      // split partials: (m, l) per head and the unnormalised O, stored
      // non-temporally (read once, by the combine kernel)
      const size_t prow = ((size_t)unit * n_splits + split) * HG + hl;   // partial row of the head
      float* orow = part_o + prow * D + wave * DQ + 4 * lg;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        __builtin_nontemporal_store(acc[hb][nb], reinterpret_cast<floatx4*>(orow + nb * 16));
      if (wave == 0 && lg == 0) part_ml[prow] = make_float2(m_q[hb], l_tot);
    }
  }
}

// The 64-head block: 8 waves (two per SIMD), so that the query operands of
// 64 heads and the accumulators of 64 heads x D fit the registers without
// spilling.  Wave w = (tq, hh) = (w % 4, w / 4):
//   QK  for the 16 tokens 16tq.. of a tile and the 32 heads 32hh.., with its
//       own dequantised registers as the X operand (the two head halves of a
//       token quarter dequantise the same rows; the first writes the X
//       tile).  Splitting the channels instead would dequantise every
//       element once, but the partial logits of all 64 heads it keeps
//       (16 more registers) push the wave past 256 registers;
//   PV  for all 64 heads over the D/8 dims D/8*w.. (each X operand read from
//       the tile once and used for the four head blocks).
// The online softmax state of every head is kept by every wave (the same
// decisions from the same maxima), the weight sums by the waves that form
// the weights.
//
// The FP4 rows do not pass through registers: a prologue turns the block's
// selected positions into row keys (page << 6 | row) in LDS, and the rows of
// tile f+2 are copied from HBM into a three-stage LDS ring by the gfx950
// global-to-LDS loads (16 bytes per lane, each row one contiguous R-byte run)
// while tile f computes; the gather lanes read their codes and scales from
// the ring.  Barriers are plain s_barrier after the wave's own LDS accesses
// completed: the ring's copies are waited for by count (vmcnt), not by a
// fence that would wait for every copy in flight.
constexpr int kBlock8 = 512;
constexpr int kStages = 3;           // LDS ring stages of FP4 tiles
constexpr int kMaxRunTiles = 32;     // FP4 tiles of one 64-head block at most (row-key table)

// Reads of a ring row written out here because the compiler cannot tell
// the ring stages apart: before a plain LDS read of the ring it waits for
// every global-to-LDS copy still in flight, the prefetch of the next two
// tiles included, which would leave the ring nothing to overlap.  The caller
// has waited for this tile's copies (vmcnt) and passed the block barrier.
// Each read waits for its own data (one LDS wait per call).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
// Two 8-byte code words at p and p + 8.
__device__ __forceinline__ void ring_codes2(const uint8_t* p, uint2& c0, uint2& c1) {
  uint64_t a, b;
  asm volatile("ds_read_b64 %0, %2\n\tds_read_b64 %1, %2 offset:8\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(a), "=&v"(b)
               : "v"(lds_addr(p))
               : "memory");
  c0 = make_uint2((uint32_t)a, (uint32_t)(a >> 32));
  c1 = make_uint2((uint32_t)b, (uint32_t)(b >> 32));
}
// NB scale bytes (2, 4 or 8) at p, as two words (the second 0 below 8).
template <int NB>
__device__ __forceinline__ void ring_scales(const uint8_t* p, uint32_t& s0, uint32_t& s1) {
  s1 = 0u;
  if constexpr (NB == 8) {
    uint64_t v;
    asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v) : "v"(lds_addr(p)) : "memory");
    s0 = (uint32_t)v;
    s1 = (uint32_t)(v >> 32);
  } else if constexpr (NB == 4) {
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(s0) : "v"(lds_addr(p)) : "memory");
  } else {
    static_assert(NB == 2, "2, 4 or 8 scale bytes");
    asm volatile("ds_read_u16 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(s0) : "v"(lds_addr(p)) : "memory");
  }
}

// N LDS words (at the byte addresses a[]), read with one LDS wait and
// without the compiler's wait for the copies in flight (see ring_read).
template <int N>
__device__ __forceinline__ void lds_words(const uint32_t (&a)[N], int (&w)[N]) {
  static_assert(N >= 1 && N <= 3, "one to three words");
  if constexpr (N == 1) {
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(w[0]) : "v"(a[0]) : "memory");
  } else if constexpr (N == 2) {
    asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(w[0]), "=&v"(w[1]) : "v"(a[0]), "v"(a[1]) : "memory");
  } else {
    asm volatile(
        "ds_read_b32 %0, %3\n\tds_read_b32 %1, %4\n\tds_read_b32 %2, %5\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]) : "v"(a[0]), "v"(a[1]), "v"(a[2]) : "memory");
  }
}

// Every LDS access of this wave has completed, then the block barrier.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// At most N vector-memory operations of this wave still in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS geometry of one staged FP4 tile: 64 rows of PSPR slots of CB bytes (a
// row's R bytes in its first R/CB slots; D = 512 pads a row to 19 slots so
// that the 16 rows a gather lane group reads start in distinct banks).  One
// global-to-LDS instruction fills 64 consecutive slots.
template <int D>
struct Ring {
  static constexpr int R = D / 2 + D / 16;
  static constexpr int CB = (R % 16 == 0) ? 16 : 4;   // bytes per lane and copy
  static constexpr int SPR = R / CB;                   // slots holding a row
  static constexpr int PSPR = D == 512 ? SPR + 1 : SPR;
  static constexpr int NCOPY = PSPR;                   // copies per tile (64 slots each)
  static constexpr int STAGE = kTile * PSPR * CB;      // bytes per stage
};

template <int D>
__global__ __launch_bounds__(kBlock8, 1) void sparse_decode64_kernel(
    const uint8_t* __restrict__ pages, const int32_t* __restrict__ page_table, int num_pages,
    int max_pages, int page_bytes, const int32_t* __restrict__ ctx_len, int H,
    const uint16_t* __restrict__ q, float scale, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ idx_count, int K, const uint16_t* __restrict__ swa,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float2* __restrict__ part_ml, int batch, int n_splits, int split_tiles, int win_sep) {
  using RG = Ring<D>;
  constexpr int HG = 64;
  constexpr int R = RG::R;
  constexpr int XS = D + 24;                // X row stride (halfs), see sparse_decode_kernel
  constexpr int QS = D + 8;
  constexpr int KQ = D / 32;                // MFMA k-steps over D
  constexpr int DE = D / 4;                 // channels per gather lane
  constexpr int NG = DE / 16;               // scale groups per gather lane
  constexpr int DW = D / 8;                 // PV dims per wave
  constexpr int NDB = DW / 16;              // 16-dim blocks per wave in PV
  constexpr int QPL = D / 16 / 8;
  constexpr int RT = kMaxRunTiles * kTile;  // row keys held
  static_assert(HG * QS <= kTile * XS, "query staging fits in the X tile");
  __shared__ __attribute__((aligned(16))) _Float16 X[kTile * XS];
  __shared__ __attribute__((aligned(16))) _Float16 Pt[HG * kPStride];
  __shared__ __attribute__((aligned(16))) uint8_t ring[kStages * RG::STAGE];
  __shared__ int rk_lds[RT];
  __shared__ __attribute__((aligned(16))) float red_max[HG][4];
  __shared__ float red_sum[4][HG];
  __shared__ int q_exp[HG];

  const int n_hg = H / HG;
  const int groups = batch * n_splits;
  const int xcd = blockIdx.x & 7, r8 = blockIdx.x >> 3;
  const int hg = r8 % n_hg;
  const int grp = (r8 / n_hg) * 8 + xcd;
  if (grp >= groups) return;
  const int b = grp / n_splits, split = grp % n_splits;
  const int unit = b * n_hg + hg;

  const int L_raw = ctx_len[b];
  const int cnt_raw = idx_count[b];
  const int tiles_k = (K + kTile - 1) / kTile;
  const TileRange tr = split_range(split, n_splits, split_tiles, tiles_k, win_sep);
  const int wa = tr.wa, fa = tr.fa, fb0 = tr.fb0;
  const int wb0 = swa == nullptr ? wa : tr.wb0;           // no window rows at all

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lg = lane >> 4, lc = lane & 15;
  const int tq = wave & 3, hh = wave >> 2;
  const int tok = tq * 16 + lc;             // gather token of this lane in a tile
  const int ch0 = lg * DE;                  // first channel of this gather lane

  const int32_t* pt = page_table + (size_t)b * max_pages;
  const int32_t* idx_row = idx + (size_t)b * K;
  const uint16_t* swa_b = swa != nullptr ? swa + (size_t)b * kWindow * D : nullptr;

  // ---- prologue.  Loads that depend on nothing first: the selected
  // positions of the block's FP4 tiles (RT / 512 per thread), the queries.
  constexpr int PPT = RT / kBlock8;         // positions per thread
  const int n_pos = (fb0 - fa) * kTile;     // entries of the index row this block covers
  int pos[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int e = i * kBlock8 + tid;
    const int j = fa * kTile + e;
    pos[i] = e < n_pos ? idx_row[j < K ? j : K - 1] : -1;
  }

  // queries: two rounds of 32 heads (16 lanes per head)
  _Float16* Qs = X;
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    const int hq = round * 32 + wave * 4 + lg;
    const uint16_t* src = q + ((size_t)b * H + hg * HG + hq) * D + lc * (D / 16);
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
      frexpf(bf16_to_f32(qmax), &ex);
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
  lds_sync();
  // qf[j][kk]: head 32hh + 16j + lc, channels ch0 + 8kk .. +8 (the gather
  // lane's channels, in the order it holds them); scale2[j]: its logits in
  // log2 units
  half8 qf[2][KQ];
  float scale2[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int hl = hh * 32 + j * 16 + lc;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk)
      qf[j][kk] = *reinterpret_cast<const half8*>(Qs + hl * QS + ch0 + 8 * kk);
    scale2[j] = ldexpf(scale, -q_exp[hl]) * kLog2e;
  }

  const int L = L_raw < 0 ? 0 : (L_raw > max_pages * kPage ? max_pages * kPage : L_raw);
  const int n_glob = L > kWindow ? L - kWindow : 0;
  const int cnt = cnt_raw < 0 ? 0 : (cnt_raw > K ? K : cnt_raw);
  const int n_win = swa == nullptr ? 0 : (L < kWindow ? L : kWindow);
  const int wb = min(wb0, (n_win + kTile - 1) / kTile);
  const int fb = min(fb0, (cnt + kTile - 1) / kTile);

  // row keys of the block's FP4 tiles: -1 for an entry past the count, a
  // position outside the candidates or a page outside the pool
  if (fa < fb) {
    int pg[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int e = i * kBlock8 + tid;
      const int p = pos[i];
      const bool in = e < n_pos && fa * kTile + e < cnt && p >= 0 && p < n_glob;
      pos[i] = in ? p : -1;
      pg[i] = pt[in ? p / kPage : 0];
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int e = i * kBlock8 + tid;
      const int p = pos[i];
      const bool ok = p >= 0 && pg[i] >= 0 && pg[i] < num_pages;
      if (e < n_pos) rk_lds[e] = ok ? (pg[i] << 6) | (p & (kPage - 1)) : -1;
    }
  }
  lds_sync();                               // the staging area becomes the X tile; row keys set

  // copies of tile f's rows into ring stage (f - fa) % kStages: this wave
  // issues copies c = wave, wave + 8, ... (< NCOPY) of the tile
  const int n_mine = (RG::NCOPY - wave + 7) / 8;  // copies per tile of this wave
  constexpr int NC = (RG::NCOPY + 7) / 8;   // copies per wave and tile at most
  auto copy_tile = [&](int f) {
    uint8_t* stage = ring + ((f - fa) % kStages) * RG::STAGE;
    // this wave's first slot of the tile, hidden from the compiler so that
    // the slot arithmetic below is redone per call rather than kept in
    // registers across the tile loop (where they would be spilled, and a
    // spill reload waits for every copy in flight)
    int k0 = wave * 64 + lane;
    asm volatile("" : "+v"(k0));
    // the row keys of this wave's copies first, then the copies
    uint32_t ra[NC];
    int rks[NC];
#pragma unroll
    for (int c0 = 0; c0 < NC; ++c0) {
      const int c = c0 * 8 + wave;
      const int row = c < RG::NCOPY ? (k0 + 512 * c0) / RG::PSPR : 0;
      ra[c0] = lds_addr(&rk_lds[(f - fa) * kTile + row]);
    }
    lds_words<NC>(ra, rks);
#pragma unroll
    for (int c0 = 0; c0 < NC; ++c0) {
      const int c = c0 * 8 + wave;
      if (c < RG::NCOPY) {
        const int k = k0 + 512 * c0;                       // slot of the tile (c * 64 + lane)
        const int row = k / RG::PSPR, part = k - row * RG::PSPR;
        const int rk = rks[c0];
        const bool live = rk >= 0 && part < RG::SPR;       // else page 0, row 0 (pad slots,
        const int in_page = (rk & 63) * R + part * RG::CB; // invalid rows: never read)
        const uint8_t* src = pages + (live ? (size_t)(rk >> 6) * page_bytes + in_page : 0);
#if defined(__HIP_DEVICE_COMPILE__)
        // (the host pass of hipcc rejects the 16-byte form of this builtin)
        __builtin_amdgcn_global_load_lds(
            (const void*)src,
            (__attribute__((address_space(3))) void*)(stage + c * 64 * RG::CB), RG::CB, 0, 0);
#endif
      }
    }
  };
  // waits until this wave's copies of tile f have landed, given that the
  // copies of `later` (0..2) later tiles were issued after them
  auto wait_tile = [&](int later) {
    const int n = later * n_mine;
    if (n == 0) wait_vm<0>();
    else if (n == 1) wait_vm<1>();
    else if (n == 2) wait_vm<2>();
    else if (n == 3) wait_vm<3>();
    else if (n == 4) wait_vm<4>();
    else if (n == 6) wait_vm<6>();
    else wait_vm<0>();
  };
  if (fa < fb) copy_tile(fa);
  if (fa + 1 < fb) copy_tile(fa + 1);

  // softmax state: m_q[hb] of head 16hb + lc, for all 64 heads; l_q[j] the
  // weight sum over this wave's tokens of head 32hh + 16j + lc.
  // acc[hb][db] holds O^T[dims DW*wave + 16db + 4lg + i][head 16hb + lc].
  float m_q[4], l_q[2];
  floatx4 acc[4][NDB];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    m_q[hb] = -INFINITY;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[hb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  l_q[0] = l_q[1] = 0.0f;

  // the rest of a tile once the X tile is being written and this wave's S^T
  // (tokens 16tq + 4lg + i, heads 32hh + 16j + lc) is known
  auto finish_tile = [&](floatx4 (&s)[2], uint32_t vbits) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float lmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[j][i] = ((vbits >> i) & 1u) ? s[j][i] * scale2[j] : -INFINITY;
        lmax = fmaxf(lmax, s[j][i]);
      }
      lmax = max_across_rows(lmax);
      if (lg == 0) red_max[hh * 32 + j * 16 + lc][tq] = lmax;
    }
    lds_sync();                             // the X tile and the tile maxima are written

    float alpha[4], m_use[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const float4 rm = *reinterpret_cast<const float4*>(&red_max[hb * 16 + lc][0]);
      const float mt = fmaxf(fmaxf(rm.x, rm.y), fmaxf(rm.z, rm.w));
      const bool first = m_q[hb] == -INFINITY;
      const bool moves = !first && mt > m_q[hb] + kLazy;
      const float m_new = (first || moves) ? mt : m_q[hb];
      m_use[hb] = m_new == -INFINITY ? 0.0f : m_new;
      alpha[hb] = 1.0f;
      if (__ballot(moves)) alpha[hb] = moves ? fast_exp2(m_q[hb] - m_use[hb]) : 1.0f;
      m_q[hb] = m_new;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int hb = hh * 2 + j;
      const float mu = hh ? m_use[2 + j] : m_use[j];
      const float al = hh ? alpha[2 + j] : alpha[j];
      float psum = 0.f;
      half4 ph;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 p16 = (_Float16)fast_exp2(s[j][i] - mu);
        ph[i] = p16;
        psum += (float)p16;
      }
      l_q[j] = l_q[j] * al + sum_across_rows(psum);
      *reinterpret_cast<half4*>(Pt + (hb * 16 + lc) * kPStride + tq * 16 + lg * 4) = ph;
    }
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      if (__ballot(alpha[hb] != 1.0f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[hb][db] *= alpha[hb];
      }
    }
    lds_sync();                             // P is written

#pragma unroll
    for (int kb = 0; kb < kTile / 32; ++kb) {
      const int tok0 = kb * 32 + lg * 8 + (lc >> 2);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = wave * DW + db * 16 + 4 * (lc & 3);
        const half4 b0 = lds_read_tr(X + tok0 * XS + col);
        const half4 b1 = lds_read_tr(X + (tok0 + 4) * XS + col);
        const half8 xt = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const half8 pb =
              *reinterpret_cast<const half8*>(Pt + (hb * 16 + lc) * kPStride + kb * 32 + lg * 8);
          acc[hb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xt, pb, acc[hb][db], 0, 0, 0);
        }
      }
    }
  };

  _Float16* xrow = X + tok * XS + ch0;
  const bool writer = hh == 0;              // the first head half writes the X tile

  // window tiles: each lane converts its D/8 channels of bf16 (16-byte
  // loads, two in flight while two are converted) into the X tile and the
  // QK operands
#pragma unroll 1
  for (int t = wa; t < wb; ++t) {
    const bool ok = t * kTile + tok < n_win;
    const uint4* src = reinterpret_cast<const uint4*>(swa_b + (size_t)(t * kTile + tok) * D + ch0);
    constexpr int WC = 2;
    uint4 wv[2][WC];
#pragma unroll
    for (int i = 0; i < WC; ++i) wv[0][i] = src[i];
    floatx4 s[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    if (t > wa) lds_sync();                 // the previous tile's PV is done with X and P
#pragma unroll
    for (int c = 0; c < KQ / WC; ++c) {
      if (c + 1 < KQ / WC) {
#pragma unroll
        for (int i = 0; i < WC; ++i) wv[(c + 1) & 1][i] = src[(c + 1) * WC + i];
      }
#pragma unroll
      for (int i = 0; i < WC; ++i) {
        const int kk = c * WC + i;
        const half8 x = ok ? bf16x8_to_f16(wv[c & 1][i]) : half8{};
        if (writer) *reinterpret_cast<half8*>(xrow + 8 * kk) = x;
        s[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, qf[0][kk], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, qf[1][kk], s[1], 0, 0, 0);
      }
    }
    const uint32_t vbits = (uint32_t)(__ballot(ok) >> (4 * lg)) & 0xFu;
    finish_tile(s, vbits);
  }

  // FP4 tiles from the ring: tile f+2 is requested, tile f's copies waited
  // for, then every wave reads its rows from stage (f - fa) % 3
  const uint8_t* my_row = ring + tok * RG::PSPR * RG::CB;
#pragma unroll 1
  for (int f = fa; f < fb; ++f) {
    if (f + 2 < fb) copy_tile(f + 2);
    wait_tile(min(2, fb - 1 - f));
    lds_sync();                             // tile f is in LDS everywhere; X and P are free
    const uint8_t* rowp = my_row + ((f - fa) % kStages) * RG::STAGE;
    // row keys of this lane's token and of the tokens 16tq + 4lg + i its
    // logits belong to (-1: no row)
    int rk_mine;
    intx4 rk_q;
    {
      const uint32_t base = lds_addr(&rk_lds[(f - fa) * kTile + tq * 16]);
      asm volatile("ds_read_b32 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(rk_mine), "=&v"(rk_q)
                   : "v"(base + 4 * lc), "v"(base + 16 * lg)
                   : "memory");
    }
    const bool ok = rk_mine >= 0;
    // this lane's NG scale bytes (at D/2 + ch0/16) and code bytes (at ch0/2)
    uint32_t sw0, sw1;
    ring_scales<NG>(rowp + D / 2 + ch0 / 16, sw0, sw1);
    half2v sc[4];
    e4m3x4_to_f16(ok ? sw0 : 0u, sc[0], sc[1]);
    if constexpr (NG > 4) e4m3x4_to_f16(ok ? sw1 : 0u, sc[2], sc[3]);
    floatx4 s[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    uint2 cv[2];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if ((g & 1) == 0) ring_codes2(rowp + ch0 / 2 + 8 * g, cv[0], cv[1]);
      const uint2 v = cv[g & 1];
      const half2v spair = sc[g / 2];
      const half2v s2 = (g & 1) ? __builtin_shufflevector(spair, spair, 1, 1)
                                : __builtin_shufflevector(spair, spair, 0, 0);
      half8 lo, hi;
      dequant16(v.x, v.y, s2, lo, hi);
      if (writer) {
        *reinterpret_cast<half8*>(xrow + 16 * g) = lo;
        *reinterpret_cast<half8*>(xrow + 16 * g + 8) = hi;
      }
      s[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, qf[0][2 * g], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, qf[1][2 * g], s[1], 0, 0, 0);
      s[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, qf[0][2 * g + 1], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, qf[1][2 * g + 1], s[1], 0, 0, 0);
    }
    const uint32_t vbits = (rk_q.x >= 0 ? 1u : 0u) | (rk_q.y >= 0 ? 2u : 0u) |
                           (rk_q.z >= 0 ? 4u : 0u) | (rk_q.w >= 0 ? 8u : 0u);
    finish_tile(s, vbits);
  }

  // finish: l of each head summed over the four token quarters
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (lg == 0) red_sum[tq][hh * 32 + j * 16 + lc] = l_q[j];
  lds_sync();
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int hl = hb * 16 + lc;
    const float l_tot = red_sum[0][hl] + red_sum[1][hl] + red_sum[2][hl] + red_sum[3][hl];
    const int head = hg * HG + hl;
    if (n_splits == 1) {
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.0f;
      float* orow = out + ((size_t)b * H + head) * D + wave * DW + 4 * lg;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<floatx4*>(orow + db * 16) = acc[hb][db] * inv;
      if (wave == 0 && lg == 0 && lse != nullptr)
        lse[(size_t)b * H + head] = l_tot > 0.f ? (m_q[hb] + log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
      const size_t prow = ((size_t)unit * n_splits + split) * HG + hl;
      float* orow = part_o + prow * D + wave * DW + 4 * lg;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        __builtin_nontemporal_store(acc[hb][db], reinterpret_cast<floatx4*>(orow + db * 16));
      if (wave == 0 && lg == 0) part_ml[prow] = make_float2(m_q[hb], l_tot);
    }
  }
}

// LSE merge of the split partials.  Block = (unit, HPB heads); thread = V
// float4s of one head's output (T4 float4s apart); every load of a batch of
// SB splits is issued before any is used.  V > 1 for few splits, so that a
// thread still has several loads in flight and the grid fits the chip at once.
template <int D, int HG, int V>
__global__ __launch_bounds__(kBlock) void sparse_combine_kernel(
    const float* __restrict__ part_o, const float2* __restrict__ part_ml, int H, int n_splits,
    float* __restrict__ out, float* __restrict__ lse) {
  constexpr int T4 = D / 4 / V;             // threads per head
  constexpr int HPB = kBlock / T4;          // heads per block
  constexpr int SB = 16 / V;                // splits per batch of loads
  static_assert(HPB <= HG && HG % HPB == 0, "a block's heads lie in one head group");
  const int n_hg = H / HG;
  const int unit = blockIdx.x / (HG / HPB);
  const int h = (blockIdx.x % (HG / HPB)) * HPB + (int)threadIdx.x / T4;
  const int d4 = (int)threadIdx.x % T4;
  const int b = unit / n_hg, hg = unit % n_hg;
  const size_t ubase = (size_t)unit * n_splits;
  const size_t ostep = (size_t)HG * D / 4;              // float4s from one split to the next
  const float4* src = reinterpret_cast<const float4*>(part_o + (ubase * HG + h) * D) + d4;

  float M = -INFINITY, Lsum = 0.f;
  float4 a[V];
#pragma unroll
  for (int v = 0; v < V; ++v) a[v] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < n_splits; s0 += SB) {
    float2 ml[SB];
    float4 x[SB][V];
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      if (s0 + i < n_splits) {
        ml[i] = part_ml[(ubase + s0 + i) * HG + h];
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const floatx4 t =     // partials are read once: non-temporal
              __builtin_nontemporal_load(
                  reinterpret_cast<const floatx4*>(src + (s0 + i) * ostep + v * T4));
          x[i][v] = make_float4(t.x, t.y, t.z, t.w);
        }
      } else {
        ml[i] = make_float2(-INFINITY, 0.f);
#pragma unroll
        for (int v = 0; v < V; ++v) x[i][v] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float mb = M;
#pragma unroll
    for (int i = 0; i < SB; ++i)
      if (ml[i].y > 0.f) mb = fmaxf(mb, ml[i].x);
    if (mb == -INFINITY) continue;                      // nothing with weight yet
    const float r = M == -INFINITY ? 0.f : exp2f(M - mb);
    Lsum *= r;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      a[v].x *= r;
      a[v].y *= r;
      a[v].z *= r;
      a[v].w *= r;
    }
    M = mb;
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const float w = ml[i].y > 0.f ? exp2f(ml[i].x - M) : 0.f;
      Lsum += w * ml[i].y;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        a[v].x += w * x[i][v].x;
        a[v].y += w * x[i][v].y;
        a[v].z += w * x[i][v].z;
        a[v].w += w * x[i][v].w;
      }
    }
  }
  const float il = Lsum > 0.f ? 1.0f / Lsum : 0.0f;
  const size_t orow = (size_t)b * H + hg * HG + h;
#pragma unroll
  for (int v = 0; v < V; ++v)
    reinterpret_cast<float4*>(out + orow * D)[d4 + v * T4] =
        make_float4(a[v].x * il, a[v].y * il, a[v].z * il, a[v].w * il);
  if (d4 == 0 && lse != nullptr) lse[orow] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ host
struct DecodePlan {
  int hg;                 // heads per block
  int n_splits, split_tiles;
  int win_sep;            // window tiles in splits of their own (see split_range)
};

#ifndef CSA2_DECODE_MIN_SPLIT_TILES
#define CSA2_DECODE_MIN_SPLIT_TILES 3
#endif

// A positive integer from the environment, or 0.
static int env_int(const char* name) {
  const char* v = getenv(name);
  if (v == nullptr) return 0;
  const int x = atoi(v);
  return x > 0 ? x : 0;
}

// Head group: 64 heads per block (the 8-wave kernel) when H is a multiple
// of 64 and the batch has at least 64 (sequence, 64-head) units; otherwise
// 16 heads per block (four times the dequantisation per row, four times the
// blocks).  Splits keep the grid near one resident wave of blocks (256 CUs,
// one 64-head block or two 16-head blocks each):
//   16 heads: when the units fill the resident blocks, one block per unit
//     takes all of a sequence's tiles; otherwise two one-tile splits take the
//     window tiles and FP4 runs of split_tiles tiles (at least
//     CSA2_DECODE_MIN_SPLIT_TILES, so that the partials stay small next to
//     the work) fill the rest;
//   64 heads: equal runs over the window-then-FP4 tile list, as many as fill
//     the resident blocks, each at most kMaxRunTiles FP4 tiles (the block's
//     row-key table).
// At most kMaxSplits splits.  The environment variables
// CSA2_DECODE_HEADS_PER_BLOCK (16 or 64) and CSA2_DECODE_SPLIT_TILES (> 0:
// split with runs of that many tiles; at least the sequence's tile count: no
// split) override the choice (tuning and tests); they are read on every
// call, by the workspace-size query and the launch alike.
static DecodePlan plan_decode(int batch, int H, int K) {
  const int F = (K + kTile - 1) / kTile;                 // FP4 tiles
  const int T = F + kWinTiles;                           // all tiles of a sequence
  int hg = (H % 64 == 0 && batch * (H / 64) >= 64) ? 64 : 16;
  const int e_hg = env_int("CSA2_DECODE_HEADS_PER_BLOCK");
  if (e_hg == 16 || (e_hg == 64 && H % 64 == 0)) hg = e_hg;
  const int units = batch * (H / hg);
  const int e_tps = env_int("CSA2_DECODE_SPLIT_TILES");
  if (hg == 16) {
    const int resident = 512;
    if (F == 0 || (e_tps == 0 && units >= resident) || e_tps >= T) return DecodePlan{16, 1, T, 1};
    int tps = e_tps;
    if (tps == 0) {
      tps = (F * units + resident - 1) / resident;
      if (tps < CSA2_DECODE_MIN_SPLIT_TILES) tps = CSA2_DECODE_MIN_SPLIT_TILES;
    }
    const int min_tps = (F + kMaxSplits - kWinTiles - 1) / (kMaxSplits - kWinTiles);
    if (tps < min_tps) tps = min_tps;
    if (tps > F) tps = F;
    return DecodePlan{16, kWinTiles + (F + tps - 1) / tps, tps, 1};
  }
  const int resident = 256;
  int tps = e_tps;
  if (tps == 0) {
    const int want = units >= resident ? 1 : (resident + units - 1) / units;   // splits per unit
    tps = (T + want - 1) / want;
  }
  if (tps > kMaxRunTiles) tps = kMaxRunTiles;
  if (tps < (T + kMaxSplits - 1) / kMaxSplits) tps = (T + kMaxSplits - 1) / kMaxSplits;
  if (tps >= T && F <= kMaxRunTiles) return DecodePlan{64, 1, T, 0};
  return DecodePlan{64, (T + tps - 1) / tps, tps, 0};
}

struct DecodeWs {
  size_t part_o, part_ml, total;
};
static DecodeWs decode_ws(int batch, int H, int D, int K) {
  const DecodePlan pl = plan_decode(batch, H, K);
  const size_t rows = (size_t)batch * H * pl.n_splits;   // partial rows (unit, split, head)
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

template <int D, int HG>
static void launch_decode_hg(const CacheArgs& c, const DecodePlan& pl, const int32_t* ctx_len,
                             int H, const uint16_t* q, float scale, const int32_t* idx,
                             const int32_t* idx_count, int K, const uint16_t* swa, float* out,
                             float* lse, uint8_t* ws, hipStream_t st) {
  const PageLayout lay = page_layout(D, c.Di);
  const DecodeWs w = decode_ws(c.batch, H, D, K);
  const int units = c.batch * (H / HG);
  const int groups = c.batch * pl.n_splits;
  const int blocks = ((groups + 7) / 8) * 8 * (H / HG);
  float* part_o = reinterpret_cast<float*>(ws + w.part_o);
  float2* part_ml = reinterpret_cast<float2*>(ws + w.part_ml);
  if constexpr (HG == 64) {
    hipLaunchKernelGGL(sparse_decode64_kernel<D>, dim3(blocks), dim3(kBlock8), 0, st,
                       (const uint8_t*)c.pages,
                       c.page_table, c.num_pages, c.max_pages, lay.page_bytes, ctx_len, H, q,
                       scale, idx, idx_count, K, swa, out, lse, part_o, part_ml, c.batch,
                       pl.n_splits, pl.split_tiles, pl.win_sep);
  } else {
    auto kern = c.max_pages <= kPtCache ? sparse_decode_kernel<D, 16, true>
                                        : sparse_decode_kernel<D, 16, false>;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kBlock), 0, st, (const uint8_t*)c.pages,
                       c.page_table, c.num_pages, c.max_pages, lay.page_bytes, ctx_len, H, q,
                       scale, idx, idx_count, K, swa, out, lse, part_o, part_ml, c.batch,
                       pl.n_splits, pl.split_tiles, pl.win_sep);
  }
  if (pl.n_splits > 1) {
    // few splits: four float4s per thread (two where a block of four would
    // span more than one head group)
    constexpr int VF = kBlock * 16 / D <= HG ? 4 : 2;
    const float* po = reinterpret_cast<const float*>(ws + w.part_o);
    const float2* pm = reinterpret_cast<const float2*>(ws + w.part_ml);
    if (pl.n_splits <= 4) {
      constexpr int HPB = kBlock * VF * 4 / D;
      hipLaunchKernelGGL((sparse_combine_kernel<D, HG, VF>), dim3(units * (HG / HPB)),
                         dim3(kBlock), 0, st, po, pm, H, pl.n_splits, out, lse);
    } else {
      constexpr int HPB = kBlock * 4 / D;
      hipLaunchKernelGGL((sparse_combine_kernel<D, HG, 1>), dim3(units * (HG / HPB)),
                         dim3(kBlock), 0, st, po, pm, H, pl.n_splits, out, lse);
    }
  }
}

template <int D>
static void launch_decode(const CacheArgs& c, const int32_t* ctx_len, int H, const uint16_t* q,
                          float scale, const int32_t* idx, const int32_t* idx_count, int K,
                          const uint16_t* swa, float* out, float* lse, uint8_t* ws,
                          hipStream_t st) {
  const DecodePlan pl = plan_decode(c.batch, H, K);
  if (pl.hg == 64)
    launch_decode_hg<D, 64>(c, pl, ctx_len, H, q, scale, idx, idx_count, K, swa, out, lse, ws, st);
  else
    launch_decode_hg<D, 16>(c, pl, ctx_len, H, q, scale, idx, idx_count, K, swa, out, lse, ws, st);
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
