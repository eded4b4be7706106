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
// Block = (sequence, group of 16 heads, token split), 4 waves.  Per 64-token
// tile:
//   1. all threads gather/dequantise the tile into LDS as f16 [64][D+8]
//      (FP4 -> exact E2M1 with the hardware converter at scale 1.0, then an
//      exact f16 multiply by the E4M3 scale; window rows bf16 -> f16);
//   2. wave w computes S^T = X[16w..16w+16) Q^T with MFMA 16x16x32 f16
//      (queries pre-scaled per head by a power of two so that their f16 copy
//      is exact), tile max per head through LDS;
//   3. online softmax in the exp2 domain, P (f16) to LDS;
//   4. wave w accumulates O[16 heads][D/4 slice] += P X with MFMA, the X
//      operand read token-contiguous by ds_read_b64_tr_b16.
// Splits write (m, l, unnormalised O) and a combine kernel merges them.
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
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Dequantise 16 channels: 8 code bytes (two words) with E4M3 scale byte sc.
__device__ __forceinline__ void dequant16(uint32_t w0, uint32_t w1, uint32_t sc, half8& lo,
                                          half8& hi) {
  const _Float16 s = (_Float16)e4m3_value(sc & 0x7Fu);
  const half2v s2 = {s, s};
  half2v r[8];
  r[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 0) * s2;
  r[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 1) * s2;
  r[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 2) * s2;
  r[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 3) * s2;
  r[4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 0) * s2;
  r[5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 1) * s2;
  r[6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 2) * s2;
  r[7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 3) * s2;
  lo = half8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
  hi = half8{r[4][0], r[4][1], r[5][0], r[5][1], r[6][0], r[6][1], r[7][0], r[7][1]};
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

template <int D>
__global__ __launch_bounds__(kBlock, 2) void sparse_decode_kernel(
    const uint8_t* __restrict__ pages, const int32_t* __restrict__ page_table, int num_pages,
    int max_pages, int scales_off, int page_bytes, const int32_t* __restrict__ ctx_len, int H,
    const uint16_t* __restrict__ q, float scale, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ idx_count, int K, const uint16_t* __restrict__ swa,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float2* __restrict__ part_ml, int batch, int n_splits, int split_tokens) {
  constexpr int XS = D + 8;                 // LDS row stride (halfs) of the X tile
  constexpr int KQ = D / 32;                // MFMA k-steps over D for QK
  constexpr int NB = D / 64;                // 16-dim blocks per wave for PV
  constexpr int DQ = D / 4;                 // channels per thread in the gather
  __shared__ __attribute__((aligned(16))) _Float16 X[kTile * XS];
  __shared__ __attribute__((aligned(16))) _Float16 Pt[kHG * kPStride];
  __shared__ float red_max[4][kHG];
  __shared__ float red_sum[4][kHG];
  __shared__ uint8_t valid[kTile];

  // ---- block -> (sequence, split, head group), head groups of a unit share an XCD
  const int n_hg = H / kHG;
  const int units = batch * n_splits;
  const int grp = blockIdx.x / (8 * n_hg), rem = blockIdx.x % (8 * n_hg);
  const int hg = rem / 8;
  const int unit = grp * 8 + rem % 8;
  if (unit >= units) return;
  const int b = unit / n_splits, split = unit % n_splits;

  int L = ctx_len[b];
  L = L < 0 ? 0 : (L > max_pages * kPage ? max_pages * kPage : L);
  const int n_glob = L > kWindow ? L - kWindow : 0;     // selectable positions
  int cnt = idx_count[b];
  cnt = cnt < 0 ? 0 : (cnt > K ? K : cnt);
  const int n_win = L < kWindow ? L : kWindow;
  const int n_tok = cnt + n_win;
  const int t_begin = split * split_tokens;
  const int t_end = min(t_begin + split_tokens, n_tok);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;

  // ---- queries: lane holds head lc, dims 32kk + 8lg .. +8, as exact f16 of q*2^e
  const int head_q = hg * kHG + lc;
  const uint16_t* qrow = q + ((size_t)b * H + head_q) * D;
  uint4 qraw[KQ];
  uint32_t qmax = 0;
#pragma unroll
  for (int kk = 0; kk < KQ; ++kk) {
    qraw[kk] = *reinterpret_cast<const uint4*>(qrow + kk * 32 + lg * 8);
    const uint32_t w[4] = {qraw[kk].x, qraw[kk].y, qraw[kk].z, qraw[kk].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) qmax = max(qmax, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
  }
  qmax = max(qmax, (uint32_t)__shfl_xor((int)qmax, 16, 64));
  qmax = max(qmax, (uint32_t)__shfl_xor((int)qmax, 32, 64));
  int qexp = 0;
  if (qmax != 0u) {
    int ex;
    frexpf(bf16_to_f32(qmax), &ex);     // max|q| in [2^(ex-1), 2^ex)
    qexp = 15 - ex;                     // scaled max in [2^14, 2^15)
  }
  half8 qf[KQ];
#pragma unroll
  for (int kk = 0; kk < KQ; ++kk) {
    const uint32_t w[4] = {qraw[kk].x, qraw[kk].y, qraw[kk].z, qraw[kk].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      qf[kk][2 * k] = (_Float16)ldexpf(bf16_to_f32(w[k] & 0xFFFFu), qexp);
      qf[kk][2 * k + 1] = (_Float16)ldexpf(bf16_to_f32(w[k] >> 16), qexp);
    }
  }
  // logits in log2 units: scale2 * (q~ . x)
  const float scale2 = ldexpf(scale, -qexp) * kLog2e;

  // running softmax state: per lane for head lc (QK layout) and for heads
  // 4lg+i (PV layout); identical inputs give identical values in both.
  float m_q = -INFINITY, l_q = 0.0f;
  float m_o[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  floatx4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int32_t* pt = page_table + (size_t)b * max_pages;
  const int32_t* idx_row = idx + (size_t)b * K;
  const uint16_t* swa_b = swa + (size_t)b * kWindow * D;
  const int g_tok = tid >> 2;            // gather: token of the tile
  const int g_q = tid & 3;               // gather: quarter of the channels

  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    // ---- 1. gather + dequantise the tile
    {
      const int j = t0 + g_tok;
      _Float16* xrow = X + g_tok * XS + g_q * DQ;
      bool ok = false;
      if (j < t_end && j < cnt) {
        const int p = idx_row[j];
        const int pg = (p >= 0 && p < n_glob) ? pt[p / kPage] : -1;
        if (pg >= 0 && pg < num_pages) {
          ok = true;
          const uint8_t* page = pages + (size_t)pg * page_bytes;
          const int r = p % kPage;
          const uint4* cp = reinterpret_cast<const uint4*>(page + r * (D / 2) + g_q * (DQ / 2));
          const uint8_t* sp = page + scales_off + r * (D / 16) + g_q * (DQ / 16);
          uint4 cw[DQ / 32];
#pragma unroll
          for (int i = 0; i < DQ / 32; ++i) cw[i] = cp[i];
          uint8_t sb[DQ / 16];
#pragma unroll
          for (int i = 0; i < DQ / 16; ++i) sb[i] = sp[i];
#pragma unroll
          for (int g = 0; g < DQ / 16; ++g) {
            const uint4 c4 = cw[g / 2];
            const uint32_t w0 = (g & 1) ? c4.z : c4.x, w1 = (g & 1) ? c4.w : c4.y;
            const uint32_t sc = sb[g];
            half8 lo, hi;
            dequant16(w0, w1, sc, lo, hi);
            *reinterpret_cast<half8*>(xrow + 16 * g) = lo;
            *reinterpret_cast<half8*>(xrow + 16 * g + 8) = hi;
          }
        }
      } else if (j < t_end) {
        const int p = L - n_win + (j - cnt);
        ok = true;
        const uint4* src =
            reinterpret_cast<const uint4*>(swa_b + (size_t)(p % kWindow) * D + g_q * DQ);
#pragma unroll
        for (int i = 0; i < DQ / 8; ++i) *reinterpret_cast<half8*>(xrow + 8 * i) = bf16x8_to_f16(src[i]);
      }
      if (!ok) {
#pragma unroll
        for (int i = 0; i < DQ / 8; ++i) *reinterpret_cast<half8*>(xrow + 8 * i) = half8{};
      }
      if (g_q == 0) valid[g_tok] = ok ? 1 : 0;
    }
    __syncthreads();

    // ---- 2. S^T for tokens 16*wave .. +16 of the tile, all 16 heads
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
    const _Float16* xa = X + (wave * 16 + lc) * XS + lg * 8;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      const half8 a = *reinterpret_cast<const half8*>(xa + kk * 32);
      s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qf[kk], s, 0, 0, 0);
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = wave * 16 + lg * 4 + i;
      s[i] = valid[tt] ? s[i] * scale2 : -INFINITY;
      lmax = fmaxf(lmax, s[i]);
    }
    lmax = fmaxf(lmax, __shfl_xor(lmax, 16, 64));
    lmax = fmaxf(lmax, __shfl_xor(lmax, 32, 64));
    if (lg == 0) red_max[wave][lc] = lmax;
    __syncthreads();

    // ---- 3. online softmax
    {
      float mt = fmaxf(fmaxf(red_max[0][lc], red_max[1][lc]), fmaxf(red_max[2][lc], red_max[3][lc]));
      const float m_new = fmaxf(m_q, mt);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = exp2f(m_q - m_use);
      float psum = 0.f;
      half4 ph;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = exp2f(s[i] - m_use);
        const _Float16 p16 = (_Float16)pv;
        ph[i] = p16;
        psum += (float)p16;             // the weights the PV product actually uses
      }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      l_q = l_q * alpha + psum;
      m_q = m_new;
      *reinterpret_cast<half4*>(Pt + lc * kPStride + wave * 16 + lg * 4) = ph;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = lg * 4 + i;
        const float mt_o =
            fmaxf(fmaxf(red_max[0][h], red_max[1][h]), fmaxf(red_max[2][h], red_max[3][h]));
        const float mn = fmaxf(m_o[i], mt_o);
        const float mu = mn == -INFINITY ? 0.0f : mn;
        const float al = exp2f(m_o[i] - mu);
        m_o[i] = mn;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb][i] *= al;
      }
    }
    __syncthreads();

    // ---- 4. O[16 heads][wave's D/4] += P X
#pragma unroll
    for (int kb = 0; kb < kTile / 32; ++kb) {
      const half8 a = *reinterpret_cast<const half8*>(Pt + lc * kPStride + kb * 32 + lg * 8);
      const int tok0 = kb * 32 + lg * 8 + (lc >> 2);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = wave * DQ + nb * 16 + 4 * (lc & 3);
        const half4 b0 = lds_read_tr(X + tok0 * XS + col);
        const half4 b1 = lds_read_tr(X + (tok0 + 4) * XS + col);
        const half8 bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bb, acc[nb], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- finish: total l per head across waves (every wave saw the same m)
  if (lg == 0) red_sum[wave][lc] = l_q;
  __syncthreads();
  float l_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = lg * 4 + i;
    l_o[i] = red_sum[0][h] + red_sum[1][h] + red_sum[2][h] + red_sum[3][h];
  }
  if (n_splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = hg * kHG + lg * 4 + i;
      const float inv = l_o[i] > 0.f ? 1.0f / l_o[i] : 0.0f;
      float* orow = out + ((size_t)b * H + head) * D + wave * DQ + lc;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) orow[nb * 16] = acc[nb][i] * inv;
    }
    if (wave == 0 && lg == 0 && lse != nullptr) {
      const float lt = red_sum[0][lc] + red_sum[1][lc] + red_sum[2][lc] + red_sum[3][lc];
      lse[(size_t)b * H + hg * kHG + lc] = lt > 0.f ? (m_q + log2f(lt)) * kLn2 : -INFINITY;
    }
  } else {
    const size_t pbase = ((size_t)b * n_splits + split) * H;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = hg * kHG + lg * 4 + i;
      float* orow = part_o + (pbase + head) * D + wave * DQ + lc;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) orow[nb * 16] = acc[nb][i];
    }
    if (wave == 0 && lg == 0) {
      const float lt = red_sum[0][lc] + red_sum[1][lc] + red_sum[2][lc] + red_sum[3][lc];
      part_ml[pbase + hg * kHG + lc] = make_float2(m_q, lt);
    }
  }
}

// LSE-merge of the split partials: one block per (sequence, head).
__global__ __launch_bounds__(128) void sparse_combine_kernel(const float* __restrict__ part_o,
                                                             const float2* __restrict__ part_ml,
                                                             int H, int D, int n_splits,
                                                             float* __restrict__ out,
                                                             float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, part_ml[((size_t)b * n_splits + s) * H + h].x);
  const float Mu = M == -INFINITY ? 0.0f : M;
  float Lsum = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    const float2 ml = part_ml[((size_t)b * n_splits + s) * H + h];
    Lsum += ml.y > 0.f ? exp2f(ml.x - Mu) * ml.y : 0.f;
  }
  const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.0f;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < n_splits; ++s) {
      const size_t r = ((size_t)b * n_splits + s) * H + h;
      const float2 ml = part_ml[r];
      if (ml.y > 0.f) acc += exp2f(ml.x - Mu) * part_o[r * D + d];
    }
    out[((size_t)b * H + h) * D + d] = acc * inv;
  }
  if (threadIdx.x == 0 && lse != nullptr)
    lse[(size_t)b * H + h] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ host
static int plan_splits(int batch, int H, int K) {
  const int tiles = (K + kWindow + kTile - 1) / kTile;
  const int per_seq_blocks = H / kHG;
  int want = (512 + batch * per_seq_blocks - 1) / (batch * per_seq_blocks);
  if (want < 1) want = 1;
  int tiles_per_split = (tiles + want - 1) / want;
  if (tiles_per_split < 1) tiles_per_split = 1;
  return (tiles + tiles_per_split - 1) / tiles_per_split;
}
static int split_tokens_for(int n_splits, int K) {
  const int tiles = (K + kWindow + kTile - 1) / kTile;
  return ((tiles + n_splits - 1) / n_splits) * kTile;
}

size_t sparse_decode_ws_bytes(int batch, int H, int D, int K) {
  const int ns = plan_splits(batch, H, K);
  if (ns == 1) return 256;
  const size_t o = (size_t)batch * ns * H * D * 4;
  const size_t ml = (size_t)batch * ns * H * 8;
  return ((o + 255) & ~(size_t)255) + ml;
}

template <int D>
static void launch_decode(const CacheArgs& c, const int32_t* ctx_len, int H, const uint16_t* q,
                          float scale, const int32_t* idx, const int32_t* idx_count, int K,
                          const uint16_t* swa, float* out, float* lse, float* po, float2* pml,
                          int ns, int st_tok, hipStream_t st) {
  const PageLayout lay = page_layout(D, c.Di);
  const int units = c.batch * ns;
  const int blocks = ((units + 7) / 8) * 8 * (H / kHG);
  hipLaunchKernelGGL((sparse_decode_kernel<D>), dim3(blocks), dim3(kBlock), 0, st,
                     (const uint8_t*)c.pages, c.page_table, c.num_pages, c.max_pages,
                     lay.scales_off, lay.page_bytes, ctx_len, H, q, scale, idx, idx_count, K, swa,
                     out, lse, po, pml, c.batch, ns, st_tok);
}

hipError_t run_sparse_decode(const CacheArgs& c, const int32_t* ctx_len, int H,
                             const uint16_t* q, float scale, const int32_t* idx,
                             const int32_t* idx_count, int K, const uint16_t* swa, float* out,
                             float* lse, void* ws, hipStream_t st) {
  const int ns = plan_splits(c.batch, H, K);
  const int st_tok = split_tokens_for(ns, K);
  float* po = nullptr;
  float2* pml = nullptr;
  if (ns > 1) {
    const size_t o = (size_t)c.batch * ns * H * c.D * 4;
    po = static_cast<float*>(ws);
    pml = reinterpret_cast<float2*>(static_cast<uint8_t*>(ws) + ((o + 255) & ~(size_t)255));
  }
  switch (c.D) {
    case 128: launch_decode<128>(c, ctx_len, H, q, scale, idx, idx_count, K, swa, out, lse, po, pml, ns, st_tok, st); break;
    case 256: launch_decode<256>(c, ctx_len, H, q, scale, idx, idx_count, K, swa, out, lse, po, pml, ns, st_tok, st); break;
    case 512: launch_decode<512>(c, ctx_len, H, q, scale, idx, idx_count, K, swa, out, lse, po, pml, ns, st_tok, st); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  hipLaunchKernelGGL(sparse_combine_kernel, dim3(c.batch * H), dim3(128), 0, st, po, pml, H, c.D,
                     ns, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
