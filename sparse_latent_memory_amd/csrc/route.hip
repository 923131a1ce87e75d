// Stage 2: routing - cosine scores of Qr against the pooled router-key bank,
// mean over router heads, max over query tokens, max per document, top-k -
// and the device side of context assembly.
//
// Method: "EverMind-AI/MSA: Memory Sparse Attention for 100M-Token Contexts"
// (hysenlabs.com), section "How MSA compresses and routes documents"; stage 2
// of "EverMind Releases Memory-Sparse Attention Code for Long-Context AI
// Models" (toolmesh.ai), section "Architectural Design and Inference".
//
// Kernels, in launch order:
//  1. scan     stream the bank once from HBM, one 16-row tile per wave step.
//              bf16, at most 8 query tokens: every workgroup first builds the
//              normalised query as MFMA A-fragments in LDS (each token split
//              into a bf16 head and a bf16 remainder row, so the query keeps
//              ~16 mantissa bits); v_mfma_f32_16x16x32_bf16 then computes the
//              query dot products and the 16x16 Gram matrix of the tile
//              (A = B = bank fragment), whose diagonal is every row's squared
//              norm per head, so no cross-lane reduction runs on the VALU.
//              Otherwise (fp32, or more tokens) a prep kernel writes fp32
//              unit queries and the scan is a per-row wave reduction.
//              Output: row_score[b, j] = max over query b's tokens.
//  2. block    per 256-document block: per-document max -> doc_scores, block
//              top-k by a bitonic sort in LDS -> candidates.
//  3. final    one workgroup per query selects the exact top-k: the k-th
//              largest block maximum T bounds the global k-th key from below
//              and only the k blocks whose maximum is >= T can hold winners,
//              so at most k*k keys are sorted; a radix select over
//              wave-private histograms covers what that path does not
//              (k > 64, more than 4096 blocks).  With device-side assembly it
//              also writes the copy plan.
//  4. gather   (device-side assembly only) copy the selected documents'
//              pooled K/V rows from mapped pinned host memory into mem_kv.
// Keys are (order-preserving score bits << 32) | (0xffffffff - doc id), so one
// unsigned comparison orders by score descending, then id ascending.
#include "msa_internal.h"

#include <algorithm>

namespace msa {
namespace {

constexpr int kDocsPerBlock = 256;
constexpr int kWaves = 4;            // waves per workgroup in the scan / top-k kernels
constexpr int kSortCap = kMaxTopK;   // keys the final selection can sort in LDS
constexpr int kFastTopK = 64;        // k up to this uses the block-maximum bound (<= k*k survivors)
constexpr int kWideChains = 1;       // query tiles in flight per wave in the wide scan (4 measured no faster)

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// --------------------------------------------------------------------------
// 1a. fp32 unit queries for the VALU scan: qhat[m, h*dr + i] =
//     qr[m,h,i] / max(|qr[m,h]|, eps) / Hr.
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void prep_unit_kernel(const T *__restrict__ qr, float *__restrict__ qhat, int M,
                                                        int Hr, int dr) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int mh = blockIdx.x * kWaves + wave; mh < M * Hr; mh += gridDim.x * kWaves) {
    const T *src = qr + (int64_t)mh * dr;
    float ss = 0.f;
    for (int i = lane; i < dr; i += 64) {
      const float x = Elt<T>::get(src, i);
      ss += x * x;
    }
    ss = wave_sum(ss);
    const float scale = 1.0f / (fmaxf(sqrtf(ss), kEps) * (float)Hr);
    for (int i = lane; i < dr; i += 64) qhat[(int64_t)mh * dr + i] = Elt<T>::get(src, i) * scale;
  }
}

// --------------------------------------------------------------------------
// 1b. bf16 MFMA scan with the query preparation fused in
// --------------------------------------------------------------------------
// A-fragment f = h*KS + s, lane l holds A[row = l%16][k = 32 s + 8 (l/16) + e]
// (e < 8) of head h.  Row 2m is the bf16 rounding of unit query token m, row
// 2m+1 the bf16 rounding of its remainder; rows of absent tokens are zero.
// Lane l owns bank row (tile*16 + l%16) and the same k slice, so one load
// instruction of the wave reads 16 rows x 64 contiguous bytes.  Heads are
// loaded in groups of HG, one group ahead of the MFMAs that consume them.
#ifndef MSA_SCAN_HG
#define MSA_SCAN_HG 1
#endif
#ifndef MSA_SCAN_PIPE      // 1: keep the head-group loop rolled (fewer registers)
#define MSA_SCAN_PIPE 0
#endif
#ifndef MSA_SCAN_NT        // 1: non-temporal bank loads (the bank is read once per call)
#define MSA_SCAN_NT 0
#endif
#ifndef MSA_SCAN_CHUNKED   // 1: contiguous tile range per wave; 0: tiles strided over waves
#define MSA_SCAN_CHUNKED 0
#endif
#ifndef MSA_SCAN_GRID_MULT // workgroups launched per resident workgroup slot
#define MSA_SCAN_GRID_MULT 1
#endif
#if MSA_SCAN_NT
#define SCAN_LD ld16_nt
#else
#define SCAN_LD ld16
#endif

template <int HR, int KS, int HG>
__global__ __launch_bounds__(256) void scan_mfma_kernel(const uint16_t *__restrict__ kr,
                                                        const uint16_t *__restrict__ qr,
                                                        float *__restrict__ row_score, int64_t n_pool, int B,
                                                        int Tq) {
  constexpr int NF = HR * KS;                     // fragments per 16-row tile per lane
  constexpr int DR = KS * 32;                     // router head dim
  constexpr int ROW = HR * DR;                    // elements per bank row
  constexpr int NG = HR / HG;                     // head groups per tile
  constexpr int GF = HG * KS;                     // fragments per head group
  __shared__ u32x4 afrag[NF * 64];
  __shared__ float qscale[8 * HR];
  const int M = B * Tq;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  for (int mh = wave; mh < M * HR; mh += kWaves) {
    const uint16_t *src = qr + (int64_t)mh * DR;
    float ss = 0.f;
    for (int i = lane; i < DR; i += 64) {
      const float x = bf16_to_f32(src[i]);
      ss += x * x;
    }
    ss = wave_sum(ss);
    if (lane == 0) qscale[mh] = 1.0f / (fmaxf(sqrtf(ss), kEps) * (float)HR);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < NF * 64; idx += blockDim.x) {
    const int l = idx & 63, f = idx >> 6;
    const int h = f / KS, s = f % KS;
    const int r = l & 15, m = r >> 1;
    uint32_t w[4] = {0, 0, 0, 0};
    if (m < M) {
      const uint16_t *src = qr + ((int64_t)m * HR + h) * DR + 32 * s + 8 * (l >> 4);
      const float sc = qscale[m * HR + h];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = bf16_to_f32(src[e]) * sc;
        const uint16_t hi = f32_to_bf16(x);
        const uint16_t val = (r & 1) ? f32_to_bf16(x - bf16_to_f32(hi)) : hi;
        w[e >> 1] |= (uint32_t)val << (16 * (e & 1));
      }
    }
    u32x4 o;
    o.x = w[0]; o.y = w[1]; o.z = w[2]; o.w = w[3];
    afrag[idx] = o;
  }
  __syncthreads();

  const int col = lane & 15, grp = lane >> 4;
  const int diag_src = ((col >> 2) << 4) + col;    // lane holding Gram[col][col]
  const int64_t n_tiles = (n_pool + 15) >> 4;

#if MSA_SCAN_CHUNKED
  // each wave streams one contiguous run of tiles
  const int64_t n_waves = (int64_t)gridDim.x * kWaves, wid = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t t_begin = n_tiles * wid / n_waves, t_end = n_tiles * (wid + 1) / n_waves;
  for (int64_t tile = t_begin; tile < t_end; ++tile) {
#else
  for (int64_t tile = (int64_t)blockIdx.x * kWaves + wave; tile < n_tiles;
       tile += (int64_t)gridDim.x * kWaves) {
#endif
    const int64_t row = tile * 16 + col;
    const int64_t rowc = row < n_pool ? row : n_pool - 1;
    const uint16_t *rp = kr + rowc * ROW + 8 * grp;
    u32x4 cur[GF];
#pragma unroll
    for (int f = 0; f < GF; ++f) cur[f] = SCAN_LD(rp + 32 * f);

    float sc0 = 0.f, sc1 = 0.f;
#if MSA_SCAN_PIPE
#pragma unroll 1
#else
#pragma unroll
#endif
    for (int gi = 0; gi < NG; ++gi) {
      u32x4 nxt[GF];
      if (gi + 1 < NG) {
#pragma unroll
        for (int f = 0; f < GF; ++f) nxt[f] = SCAN_LD(rp + 32 * ((gi + 1) * GF + f));
      }
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const int h = gi * HG + hh;
        f32x4 g = {0.f, 0.f, 0.f, 0.f};
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 bv = __builtin_bit_cast(bf16x8, cur[hh * KS + s]);
          const bf16x8 av = __builtin_bit_cast(bf16x8, afrag[(h * KS + s) * 64 + lane]);
          g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv, bv, g, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, d, 0, 0, 0);
        }
        const int di = col & 3;
        const float mine = di == 0 ? g[0] : di == 1 ? g[1] : di == 2 ? g[2] : g[3];
        const float n2 = __shfl(mine, diag_src, 64);
        const float inv = rsqrtf(fmaxf(n2, kEps2));
        sc0 += (d[0] + d[1]) * inv;      // token 2*grp     (head + remainder rows)
        sc1 += (d[2] + d[3]) * inv;      // token 2*grp + 1
      }
      if (gi + 1 < NG) {
#pragma unroll
        for (int f = 0; f < GF; ++f) cur[f] = nxt[f];
      }
    }
    // gather the 8 token scores of column `col` into lanes 0..15
    float ts[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ts[2 * q] = __shfl(sc0, col + 16 * q, 64);
      ts[2 * q + 1] = __shfl(sc1, col + 16 * q, 64);
    }
    if (grp == 0 && row < n_pool) {
      for (int b = 0; b < B; ++b) {
        float m = -INFINITY;
        for (int t = 0; t < Tq; ++t) {
          const int slot = b * Tq + t;
          float v = ts[0];
#pragma unroll
          for (int q = 1; q < 8; ++q) v = slot == q ? ts[q] : v;
          m = fmaxf(m, v);
        }
        row_score[(int64_t)b * n_pool + row] = m;
      }
    }
  }
}

// --------------------------------------------------------------------------
// 1c. bf16 MFMA scan for many query tokens (more than 8)
// --------------------------------------------------------------------------
// The query side is laid out in M-tiles of 16 rows (one bf16-rounded unit
// query token per row).  With one token per query (Tq == 1) a tile holds 16
// queries.  Otherwise every query gets ceil(Tq/16) tiles of its own and the
// rows past its last token repeat that token, which leaves the max over
// tokens unchanged.  wide_frag[mt][f][lane] is fragment f = h*KS + s of tile
// mt in the lane layout of the narrow scan.
__global__ __launch_bounds__(256) void prep_wide_kernel(const float *__restrict__ qhat, u32x4 *__restrict__ frag,
                                                        int B, int Tq, int Hr, int dr, int n_mt) {
  const int KS = dr / 32, NF = Hr * KS;
  const int mtq = (Tq + 15) / 16;
  const int64_t n = (int64_t)n_mt * NF * 64;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(idx & 63);
    const int f = (int)((idx >> 6) % NF);
    const int mt = (int)((idx >> 6) / NF);
    const int h = f / KS, s = f % KS, r = l & 15;
    int m = -1;                               // query token of this row, or none
    if (Tq == 1) {
      const int b = mt * 16 + r;
      if (b < B) m = b;
    } else {
      const int b = mt / mtq;
      const int t = min((mt % mtq) * 16 + r, Tq - 1);
      m = b * Tq + t;
    }
    uint32_t w[4] = {0, 0, 0, 0};
    if (m >= 0) {
      const float *src = qhat + ((int64_t)m * Hr + h) * dr + 32 * s + 8 * (l >> 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e >> 1] |= (uint32_t)f32_to_bf16(src[e]) << (16 * (e & 1));
    }
    u32x4 o;
    o.x = w[0]; o.y = w[1]; o.z = w[2]; o.w = w[3];
    frag[idx] = o;
  }
}

// One workgroup per CU, one wave per SIMD.  Each wave owns one 16-row bank
// tile at a time with every head's fragments in registers, and loads the
// next tile's while it computes: per head, 4 MFMAs give the tile's Gram
// matrix (norms on its diagonal), then every query M-tile takes 4 MFMAs per
// head against A-fragments read from LDS, scaled by the head's inverse norm.
// Query tiles are staged into LDS MG at a time; when they do not all fit the
// workgroup restages them per group of 4 bank tiles (barriers are uniform:
// every wave walks the same number of groups).
template <int HR, int KS>
struct WideCfg {
  static constexpr int NF = HR * KS;
  static constexpr int MG = (128 / NF) < 16 ? (128 / NF) : 16;   // 128 KiB of query fragments
};

template <int HR, int KS>
__global__ __launch_bounds__(256, 1) void scan_wide_kernel(const uint16_t *__restrict__ kr,
                                                           const u32x4 *__restrict__ frag,
                                                           float *__restrict__ row_score, int64_t n_pool, int B,
                                                           int Tq, int n_mt) {
  constexpr int NF = WideCfg<HR, KS>::NF;
  constexpr int MG = WideCfg<HR, KS>::MG;
  constexpr int ROW = NF * 32;
  __shared__ u32x4 afrag[MG * NF * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int diag_src = ((col >> 2) << 4) + col;
  const int64_t n_tiles = (n_pool + 15) >> 4;
  const int64_t n_groups = (n_tiles + kWaves - 1) / kWaves;
  const int n_chunks = (n_mt + MG - 1) / MG;
  const int mtq = (Tq + 15) / 16;

  auto stage = [&](int c) {
    const int mt0 = c * MG, nm = min(MG, n_mt - mt0);
    const u32x4 *src = frag + (int64_t)mt0 * NF * 64;
    for (int i = threadIdx.x; i < nm * NF * 64; i += blockDim.x) afrag[i] = src[i];
  };
  if (n_chunks == 1) stage(0);
  __syncthreads();

  auto load_tile = [&](int64_t grp_idx, u32x4 *dst) {
    const int64_t tile = grp_idx * kWaves + wave;
    int64_t row = tile * 16 + col;
    row = row < n_pool ? row : n_pool - 1;
    const uint16_t *rp = kr + row * ROW + 8 * grp;
#pragma unroll
    for (int f = 0; f < NF; ++f) dst[f] = ld16(rp + 32 * f);
  };

  u32x4 cur[NF], nxt[NF];
  int64_t gi = blockIdx.x;
  if (gi < n_groups) load_tile(gi, cur);
  for (; gi < n_groups; gi += gridDim.x) {
    const int64_t gnext = gi + gridDim.x;
    if (gnext < n_groups) load_tile(gnext, nxt);
    const int64_t tile = gi * kWaves + wave;
    const int64_t row = tile * 16 + col;

    float inv[HR];
#pragma unroll
    for (int h = 0; h < HR; ++h) {
      f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, cur[h * KS + s]);
        g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv, bv, g, 0, 0, 0);
      }
      const int di = col & 3;
      const float mine = di == 0 ? g[0] : di == 1 ? g[1] : di == 2 ? g[2] : g[3];
      inv[h] = rsqrtf(fmaxf(__shfl(mine, diag_src, 64), kEps2));
    }

    float qmax = -INFINITY;      // running max over the tiles of one query (Tq > 1)
    for (int c = 0; c < n_chunks; ++c) {
      if (n_chunks > 1) {
        __syncthreads();
        stage(c);
        __syncthreads();
      }
      const int nm = min(MG, n_mt - c * MG);
      // four query tiles at a time: four independent MFMA accumulation chains
      for (int mi0 = 0; mi0 < nm; mi0 += kWideChains) {
        f32x4 acc[kWideChains];
#pragma unroll
        for (int u = 0; u < kWideChains; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < HR; ++h) {
          f32x4 d[kWideChains];
#pragma unroll
          for (int u = 0; u < kWideChains; ++u) d[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const bf16x8 bv = __builtin_bit_cast(bf16x8, cur[h * KS + s]);
#pragma unroll
            for (int u = 0; u < kWideChains; ++u) {
              // slots past the staged tiles hold stale fragments; their results are discarded
              const int mi = min(mi0 + u, MG - 1);
              const bf16x8 av = __builtin_bit_cast(bf16x8, afrag[(mi * NF + h * KS + s) * 64 + lane]);
              d[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, d[u], 0, 0, 0);
            }
          }
#pragma unroll
          for (int u = 0; u < kWideChains; ++u) acc[u] += d[u] * inv[h];
        }
#pragma unroll
        for (int u = 0; u < kWideChains; ++u) {
          if (mi0 + u >= nm) break;
          const int mt = c * MG + mi0 + u;
          if (Tq == 1) {
            // rows 4*grp + i of this tile are queries mt*16 + 4*grp + i
            if (row < n_pool) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int b = mt * 16 + 4 * grp + i;
                if (b < B) row_score[(int64_t)b * n_pool + row] = acc[u][i];
              }
            }
          } else {
            float m = fmaxf(fmaxf(acc[u][0], acc[u][1]), fmaxf(acc[u][2], acc[u][3]));
            m = fmaxf(m, __shfl_xor(m, 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            qmax = fmaxf(qmax, m);
            if (mt % mtq == mtq - 1) {
              if (grp == 0 && row < n_pool) row_score[(int64_t)(mt / mtq) * n_pool + row] = qmax;
              qmax = -INFINITY;
            }
          }
        }
      }
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) cur[f] = nxt[f];
  }
}

// --------------------------------------------------------------------------
// 1d. VALU scan (fp32): one wave per row
// --------------------------------------------------------------------------
template <typename T, int EPL>
__global__ __launch_bounds__(256) void scan_valu_kernel(const T *__restrict__ kr, const float *__restrict__ qhat,
                                                        float *__restrict__ row_score, int64_t n_pool, int B,
                                                        int Tq, int lanes_per_head) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rowlen = (int64_t)EPL * 64;
  for (int64_t row = (int64_t)blockIdx.x * kWaves + wave; row < n_pool; row += (int64_t)gridDim.x * kWaves) {
    const T *rp = kr + row * rowlen + lane * EPL;
    float x[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = Elt<T>::get(rp, e);
    float n2 = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) n2 += x[e] * x[e];
    for (int o = 1; o < lanes_per_head; o <<= 1) n2 += __shfl_xor(n2, o, 64);
    const float inv = rsqrtf(fmaxf(n2, kEps2));
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] *= inv;
    for (int b = 0; b < B; ++b) {
      float best = -INFINITY;
      for (int t = 0; t < Tq; ++t) {
        const float *q = qhat + ((int64_t)(b * Tq + t)) * rowlen + lane * EPL;
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) p += q[e] * x[e];
        best = fmaxf(best, wave_sum(p));
      }
      if (lane == 0) row_score[(int64_t)b * n_pool + row] = best;
    }
  }
}

// --------------------------------------------------------------------------
// 2. per-document max, block top-k, and the exact final top-k
// --------------------------------------------------------------------------
__device__ void bitonic_desc(uint64_t *key, int n) {  // n a power of two; all threads call
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n / 2; i += blockDim.x) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = ((lo & size) == 0);
        const uint64_t a = key[lo], b = key[hi];
        if ((a < b) == desc) { key[lo] = b; key[hi] = a; }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ uint64_t doc_key(float score, int d) {
  return ((uint64_t)score_key(score) << 32) | (uint64_t)(0xffffffffu - (uint32_t)d);
}

// Per 256-document block: per-document max -> doc_scores, and the block's
// top-cpb keys sorted descending -> cand.
__global__ __launch_bounds__(kDocsPerBlock) void doc_block_topk_kernel(
    const float *__restrict__ row_score, const int64_t *__restrict__ pool_off, float *__restrict__ doc_scores,
    uint64_t *__restrict__ cand, int n_docs, int64_t n_pool, int cpb) {
  __shared__ uint64_t key[kDocsPerBlock];
  const int b = blockIdx.y, n_blocks = gridDim.x;
  const int tid = threadIdx.x;
  const int d = blockIdx.x * kDocsPerBlock + tid;
  uint64_t kk = 0;
  if (d < n_docs) {
    int64_t r0 = pool_off[d], r1 = pool_off[d + 1];
    r0 = max((int64_t)0, min(r0, n_pool));
    r1 = max(r0, min(r1, n_pool));
    const float *rs = row_score + (int64_t)b * n_pool;
    float best = -INFINITY;
    int64_t r = r0;
    for (; r + 4 <= r1; r += 4) {      // independent loads in flight
      const float x0 = rs[r], x1 = rs[r + 1], x2 = rs[r + 2], x3 = rs[r + 3];
      best = fmaxf(best, fmaxf(fmaxf(x0, x1), fmaxf(x2, x3)));
    }
    for (; r < r1; ++r) best = fmaxf(best, rs[r]);
    doc_scores[(int64_t)b * n_docs + d] = best;
    kk = doc_key(best, d);
  }
  key[tid] = kk;
  __syncthreads();
  bitonic_desc(key, kDocsPerBlock);
  uint64_t *my = cand + ((int64_t)b * n_blocks + blockIdx.x) * cpb;
  for (int i = tid; i < cpb; i += blockDim.x) my[i] = key[i];
}

// One workgroup per query: the exact top-k of the n_blocks sorted candidate
// lists (and, for device-side assembly, the copy plan).  A separate launch
// rather than a last-block-done tail on the kernel above: the device-scope
// release every block would need writes back its XCD's L2, and hundreds of
// those cost far more than one kernel boundary.
__global__ __launch_bounds__(kDocsPerBlock) void topk_final_kernel(
    const uint64_t *__restrict__ cand, const int64_t *__restrict__ pool_off, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_score, GatherPlan *__restrict__ plan, int32_t *__restrict__ mem_len, int mem_cap,
    int append, int n_blocks, int64_t n_pool, int cpb, int k) {
  __shared__ uint64_t sel[kSortCap];
  __shared__ uint32_t hist[kWaves][256];
  __shared__ int top_blk[kFastTopK];
  __shared__ int s_count, s_need;
  __shared__ uint64_t s_prefix, s_mask;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6;

  const uint64_t *c = cand + (int64_t)b * n_blocks * cpb;
  const int n_cand = n_blocks * cpb;
  bool sorted = false;
  if (k <= cpb && k <= kFastTopK && n_blocks <= kSortCap) {
    // Every list is sorted, so its first key is its block's maximum.  With T
    // the k-th largest block maximum, at least k keys are >= T, so every
    // global top-k key is >= T and sits in one of the k blocks whose maximum
    // is >= T, inside that block's top-k list: only those k lists are read.
    int nb2 = 1;
    while (nb2 < n_blocks) nb2 <<= 1;
    for (int i = tid; i < nb2; i += blockDim.x) sel[i] = i < n_blocks ? c[(int64_t)i * cpb] : 0;
    __syncthreads();
    bitonic_desc(sel, nb2);
    const int nb = min(k, n_blocks);
    const uint64_t thr = n_blocks >= k ? sel[k - 1] : 0;
    if (tid < nb) top_blk[tid] = (int)((0xffffffffu - (uint32_t)(sel[tid] & 0xffffffffu)) / kDocsPerBlock);
    if (tid == 0) s_count = 0;
    __syncthreads();
    for (int i = tid; i < nb * cpb; i += blockDim.x) {
      const uint64_t x = c[(int64_t)top_blk[i / cpb] * cpb + i % cpb];
      if (x >= thr) {
        const int pos = atomicAdd(&s_count, 1);
        if (pos < kSortCap) sel[pos] = x;
      }
    }
    __syncthreads();
    sorted = s_count <= kSortCap;
  }
  if (!sorted) {
    // radix select of the k-th largest key, 8 bits per pass, wave-private histograms
    if (tid == 0) { s_prefix = 0; s_mask = 0; s_need = k; s_count = 0; }
    __syncthreads();
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int i = tid; i < kWaves * 256; i += blockDim.x) (&hist[0][0])[i] = 0;
      __syncthreads();
      const uint64_t prefix = s_prefix, mask = s_mask;
      for (int i = tid; i < n_cand; i += blockDim.x) {
        const uint64_t x = c[i];
        if ((x & mask) == prefix) atomicAdd(&hist[wave][(x >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t sum = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) sum += hist[w][tid];
        hist[0][tid] = sum;
      }
      __syncthreads();
      if (tid == 0) {
        int need = s_need, digit = 255;
        for (; digit > 0; --digit) {
          const int cnt = (int)hist[0][digit];
          if (cnt >= need) break;
          need -= cnt;
        }
        s_need = need;
        s_prefix = prefix | ((uint64_t)digit << shift);
        s_mask = mask | ((uint64_t)255 << shift);
      }
      __syncthreads();
    }
    const uint64_t thr = s_prefix;   // the k-th largest key exactly (keys are unique)
    for (int i = tid; i < n_cand; i += blockDim.x) {
      const uint64_t x = c[i];
      if (x >= thr) {
        const int pos = atomicAdd(&s_count, 1);
        if (pos < kSortCap) sel[pos] = x;
      }
    }
    __syncthreads();
  }
  const int n_sel = min(s_count, kSortCap);
  int n2 = 1;
  while (n2 < n_sel) n2 <<= 1;
  for (int i = n_sel + tid; i < n2; i += blockDim.x) sel[i] = 0;
  __syncthreads();
  bitonic_desc(sel, n2);
  for (int i = tid; i < k; i += blockDim.x) {
    const uint64_t x = sel[i];
    topk_idx[(int64_t)b * k + i] = (int32_t)(0xffffffffu - (uint32_t)(x & 0xffffffffu));
    topk_score[(int64_t)b * k + i] = key_score((uint32_t)(x >> 32));
  }
  if (!plan) return;
  // ---- context assembly plan: documents in rank order while they fit ----
  __shared__ int32_t prow[kMaxTopK], pdst[kMaxTopK];
  __syncthreads();                       // sel[] is reused below
  for (int r = tid; r < k; r += blockDim.x) {   // every rank's offsets loaded in parallel
    const int dd = (int)(0xffffffffu - (uint32_t)(sel[r] & 0xffffffffu));
    int64_t r0 = pool_off[dd], r1 = pool_off[dd + 1];
    r0 = max((int64_t)0, min(r0, n_pool));
    r1 = max(r0, min(r1, n_pool));
    sel[r] = (uint64_t)r0;
    prow[r] = (int32_t)min(r1 - r0, (int64_t)mem_cap + 1);
  }
  __syncthreads();
  if (tid == 0) {                        // prefix over LDS only
    int64_t len = append ? max(0, min(mem_len[b], mem_cap)) : 0;
    bool open = true;
    for (int r = 0; r < k; ++r) {
      open = open && len + prow[r] <= mem_cap;
      pdst[r] = open ? (int32_t)len : -1;
      if (open) len += prow[r];
    }
    mem_len[b] = (int32_t)len;
  }
  __syncthreads();
  for (int r = tid; r < k; r += blockDim.x) {
    GatherPlan p = {0, 0, 0};
    if (pdst[r] >= 0) {
      p.src_row = (int64_t)sel[r];
      p.rows = prow[r];
      p.dst_row = pdst[r];
    }
    plan[(int64_t)b * k + r] = p;
  }
}

// --------------------------------------------------------------------------
// 3. device-side assembly: one workgroup per (rank, query), reading the
//    selected rows over the host link from mapped pinned memory
// --------------------------------------------------------------------------
constexpr int kGatherInflight = 4;

__global__ __launch_bounds__(256) void gather_kernel(const u32x4 *__restrict__ host_kv, u32x4 *__restrict__ mem_kv,
                                                     const GatherPlan *__restrict__ plan, int k, int mem_cap,
                                                     int64_t row_vecs) {
  const int r = blockIdx.x, b = blockIdx.y;
  const GatherPlan p = plan[(int64_t)b * k + r];
  if (p.rows <= 0) return;
  const u32x4 *src = host_kv + p.src_row * row_vecs;
  u32x4 *dst = mem_kv + ((int64_t)b * mem_cap + p.dst_row) * row_vecs;
  const int64_t n = (int64_t)p.rows * row_vecs;
  constexpr int step = 256 * kGatherInflight;
  for (int64_t i0 = threadIdx.x; i0 < n; i0 += step) {
    u32x4 v[kGatherInflight];
#pragma unroll
    for (int q = 0; q < kGatherInflight; ++q)
      if (i0 + q * 256 < n) v[q] = src[i0 + q * 256];
#pragma unroll
    for (int q = 0; q < kGatherInflight; ++q)
      if (i0 + q * 256 < n) dst[i0 + q * 256] = v[q];
  }
}

// --------------------------------------------------------------------------
// dispatch
// --------------------------------------------------------------------------
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool mfma_shape(int32_t hr, int32_t dr) {
  const int ks = dr / 32;
  return (ks == 2 || ks == 4) && (hr == 1 || hr == 2 || hr == 4 || hr == 8 || (hr == 16 && ks == 2));
}
// bf16, at most 8 query tokens: fused-prep scan with hi/lo query rows
bool mfma_path(int32_t dtype, int32_t M, int32_t hr, int32_t dr) {
  return dtype == MSA_BF16 && M <= 8 && mfma_shape(hr, dr);
}
// bf16, more query tokens: query M-tiles streamed through LDS
bool wide_path(int32_t dtype, int32_t M, int32_t hr, int32_t dr) {
  return dtype == MSA_BF16 && M > 8 && mfma_shape(hr, dr);
}
int wide_tiles(int32_t batch, int32_t q_tokens) {
  return q_tokens == 1 ? (batch + 15) / 16 : batch * ((q_tokens + 15) / 16);
}

template <int HR, int KS>
hipError_t launch_scan_wide(const msa_route_args &a, const RouteWs &ws, hipStream_t s) {
  const int64_t n_groups = ((a.n_pool + 15) / 16 + kWaves - 1) / kWaves;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(device_info().n_cu, n_groups));
  hipLaunchKernelGGL((scan_wide_kernel<HR, KS>), dim3(grid), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t *>(a.kr_pooled), ws.wide_frag, ws.row_score, a.n_pool,
                     a.batch, a.q_tokens, wide_tiles(a.batch, a.q_tokens));
  return hipGetLastError();
}

template <int HR, int KS>
hipError_t launch_scan_mfma(const msa_route_args &a, const RouteWs &ws, hipStream_t s) {
  constexpr int HG = HR < MSA_SCAN_HG ? HR : MSA_SCAN_HG;
  const int64_t n_tiles = (a.n_pool + 15) / 16;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, scan_mfma_kernel<HR, KS, HG>, 256, 0) != hipSuccess ||
      occ < 1)
    occ = 1;
  const int64_t want = (int64_t)device_info().n_cu * occ * MSA_SCAN_GRID_MULT;
  const int64_t need = (n_tiles + kWaves - 1) / kWaves;
  const int grid = (int)std::max<int64_t>(1, std::min(want, need));
  hipLaunchKernelGGL((scan_mfma_kernel<HR, KS, HG>), dim3(grid), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t *>(a.kr_pooled), reinterpret_cast<const uint16_t *>(a.qr),
                     ws.row_score, a.n_pool, a.batch, a.q_tokens);
  return hipGetLastError();
}

template <typename T, int EPL>
hipError_t launch_scan_valu_t(const msa_route_args &a, const RouteWs &ws, hipStream_t s) {
  const int64_t need = (a.n_pool + kWaves - 1) / kWaves;
  const int64_t want = (int64_t)device_info().n_cu * 8;
  const int grid = (int)std::max<int64_t>(1, std::min(want, need));
  const int lanes_per_head = 64 / a.n_router_heads;
  hipLaunchKernelGGL((scan_valu_kernel<T, EPL>), dim3(grid), dim3(256), 0, s,
                     reinterpret_cast<const T *>(a.kr_pooled), ws.qhat, ws.row_score, a.n_pool, a.batch,
                     a.q_tokens, lanes_per_head);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_scan_valu(const msa_route_args &a, const RouteWs &ws, hipStream_t s) {
  switch (a.n_router_heads * a.router_dim / 64) {
    case 1: return launch_scan_valu_t<T, 1>(a, ws, s);
    case 2: return launch_scan_valu_t<T, 2>(a, ws, s);
    case 4: return launch_scan_valu_t<T, 4>(a, ws, s);
    case 8: return launch_scan_valu_t<T, 8>(a, ws, s);
    case 16: return launch_scan_valu_t<T, 16>(a, ws, s);
    case 32: return launch_scan_valu_t<T, 32>(a, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool route_shape_supported(int32_t hr, int32_t dr) {
  if (dr != 64 && dr != 128) return false;
  if (hr < 1 || hr > 64 || (hr & (hr - 1)) != 0) return false;
  const int epl = hr * dr / 64;
  return epl <= 32 && (64 % hr) == 0;
}

size_t route_ws_layout(int32_t dtype, int32_t batch, int32_t q_tokens, int32_t hr, int32_t dr, int32_t n_docs,
                       int64_t n_pool, int32_t top_k, void *base, RouteWs *ws) {
  const int32_t M = batch * q_tokens;
  const int32_t n_blocks = (n_docs + kDocsPerBlock - 1) / kDocsPerBlock;
  const int32_t cpb = std::min(top_k, kDocsPerBlock);
  size_t off = 0;
  const size_t o_rs = off;
  off = align256(off + sizeof(float) * (size_t)batch * (size_t)n_pool);
  const size_t o_q = off;
  if (!mfma_path(dtype, M, hr, dr)) off = align256(off + sizeof(float) * (size_t)M * hr * dr);
  const size_t o_w = off;
  if (wide_path(dtype, M, hr, dr))
    off = align256(off + sizeof(u32x4) * 64 * (size_t)hr * (dr / 32) * wide_tiles(batch, q_tokens));
  const size_t o_c = off;
  off = align256(off + sizeof(uint64_t) * (size_t)batch * n_blocks * cpb);
  const size_t o_plan = off;
  off = align256(off + sizeof(GatherPlan) * (size_t)batch * top_k);
  if (ws) {
    char *p = reinterpret_cast<char *>(base);
    ws->row_score = reinterpret_cast<float *>(p + o_rs);
    ws->qhat = reinterpret_cast<float *>(p + o_q);
    ws->wide_frag = reinterpret_cast<u32x4 *>(p + o_w);
    ws->cand = reinterpret_cast<uint64_t *>(p + o_c);
    ws->plan = reinterpret_cast<GatherPlan *>(p + o_plan);
    ws->n_blocks = n_blocks;
    ws->cand_per_block = cpb;
  }
  return off;
}

hipError_t launch_route(const msa_route_args &a, const RouteWs &ws, const void *host_kv_dev, hipStream_t s) {
  const int M = a.batch * a.q_tokens;
  hipEvent_t ev0 = reinterpret_cast<hipEvent_t>(a.prof_event_begin);
  hipEvent_t ev1 = reinterpret_cast<hipEvent_t>(a.prof_event_end);
  hipError_t e = hipSuccess;
  if (mfma_path(a.dtype, M, a.n_router_heads, a.router_dim)) {
    if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
    const int ks = a.router_dim / 32;
    switch (a.n_router_heads * 8 + ks) {
      case 1 * 8 + 2: e = launch_scan_mfma<1, 2>(a, ws, s); break;
      case 1 * 8 + 4: e = launch_scan_mfma<1, 4>(a, ws, s); break;
      case 2 * 8 + 2: e = launch_scan_mfma<2, 2>(a, ws, s); break;
      case 2 * 8 + 4: e = launch_scan_mfma<2, 4>(a, ws, s); break;
      case 4 * 8 + 2: e = launch_scan_mfma<4, 2>(a, ws, s); break;
      case 4 * 8 + 4: e = launch_scan_mfma<4, 4>(a, ws, s); break;
      case 8 * 8 + 2: e = launch_scan_mfma<8, 2>(a, ws, s); break;
      case 8 * 8 + 4: e = launch_scan_mfma<8, 4>(a, ws, s); break;
      case 16 * 8 + 2: e = launch_scan_mfma<16, 2>(a, ws, s); break;
      default: e = hipErrorInvalidValue;
    }
  } else {
    const bool bf16 = a.dtype == MSA_BF16;
    const int n = M * a.n_router_heads;
    const int grid = std::max(1, std::min((n + kWaves - 1) / kWaves, 1024));
    if (bf16)
      hipLaunchKernelGGL(prep_unit_kernel<uint16_t>, dim3(grid), dim3(256), 0, s,
                         reinterpret_cast<const uint16_t *>(a.qr), ws.qhat, M, a.n_router_heads, a.router_dim);
    else
      hipLaunchKernelGGL(prep_unit_kernel<float>, dim3(grid), dim3(256), 0, s,
                         reinterpret_cast<const float *>(a.qr), ws.qhat, M, a.n_router_heads, a.router_dim);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (wide_path(a.dtype, M, a.n_router_heads, a.router_dim)) {
      const int n_mt = wide_tiles(a.batch, a.q_tokens);
      const int64_t n = (int64_t)n_mt * a.n_router_heads * (a.router_dim / 32) * 64;
      hipLaunchKernelGGL(prep_wide_kernel, dim3((int)std::min<int64_t>((n + 255) / 256, 4096)), dim3(256), 0, s,
                         ws.qhat, ws.wide_frag, a.batch, a.q_tokens, a.n_router_heads, a.router_dim, n_mt);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
      switch (a.n_router_heads * 8 + a.router_dim / 32) {
        case 1 * 8 + 2: e = launch_scan_wide<1, 2>(a, ws, s); break;
        case 1 * 8 + 4: e = launch_scan_wide<1, 4>(a, ws, s); break;
        case 2 * 8 + 2: e = launch_scan_wide<2, 2>(a, ws, s); break;
        case 2 * 8 + 4: e = launch_scan_wide<2, 4>(a, ws, s); break;
        case 4 * 8 + 2: e = launch_scan_wide<4, 2>(a, ws, s); break;
        case 4 * 8 + 4: e = launch_scan_wide<4, 4>(a, ws, s); break;
        case 8 * 8 + 2: e = launch_scan_wide<8, 2>(a, ws, s); break;
        case 8 * 8 + 4: e = launch_scan_wide<8, 4>(a, ws, s); break;
        case 16 * 8 + 2: e = launch_scan_wide<16, 2>(a, ws, s); break;
        default: e = hipErrorInvalidValue;
      }
    } else {
      if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
      e = bf16 ? launch_scan_valu<uint16_t>(a, ws, s) : launch_scan_valu<float>(a, ws, s);
    }
  }
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return e;

  const bool device_gather = host_kv_dev != nullptr;
  hipLaunchKernelGGL(doc_block_topk_kernel, dim3(ws.n_blocks, a.batch), dim3(kDocsPerBlock), 0, s,
                     ws.row_score, a.doc_pool_off, a.doc_scores, ws.cand, a.n_docs, a.n_pool, ws.cand_per_block);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_final_kernel, dim3(a.batch), dim3(kDocsPerBlock), 0, s, ws.cand, a.doc_pool_off,
                     a.topk_idx, a.topk_score, device_gather ? ws.plan : nullptr, a.mem_len, a.mem_cap, a.append,
                     ws.n_blocks, a.n_pool, ws.cand_per_block, a.top_k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (device_gather) {
    const size_t elt = a.kv_dtype == MSA_BF16 ? 2 : 4;
    const int64_t row_vecs = (int64_t)(2 * (size_t)a.n_kv_heads * a.head_dim * elt / 16);
    hipLaunchKernelGGL(gather_kernel, dim3(a.top_k, a.batch), dim3(256), 0, s,
                       reinterpret_cast<const u32x4 *>(host_kv_dev), reinterpret_cast<u32x4 *>(a.mem_kv), ws.plan,
                       a.top_k, a.mem_cap, row_vecs);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace msa
