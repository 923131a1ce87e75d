// Stage 2: routing - cosine scores of Qr against the pooled router-key bank,
// mean over router heads, max over query tokens, max per document, top-k.
//
// Method: "EverMind-AI/MSA: Memory Sparse Attention for 100M-Token Contexts"
// (hysenlabs.com), section "How MSA compresses and routes documents"; stage 2
// of "EverMind Releases Memory-Sparse Attention Code for Long-Context AI
// Models" (toolmesh.ai), section "Architectural Design and Inference".
//
// Kernels, in launch order:
//  1. prep      normalise every query-token/head vector, fold in 1/Hr, and lay
//               it out as MFMA A-fragments (bf16 path) or fp32 rows (VALU path).
//  2. scan      stream the bank once from HBM, one 16-row tile per wave step:
//               bf16 path: v_mfma_f32_16x16x32_bf16 computes both the query
//               dot products (A = hi/lo split query, so the normalised query
//               keeps ~16 mantissa bits) and the 16x16 Gram matrix of the tile
//               (A = B = bank fragment) whose diagonal is every row's squared
//               norm per head - no cross-lane reduction on the VALU.
//               fp32 path: per-row wave reduction on the VALU.
//               Writes row_score[b, j] = max over the query's tokens.
//  3. reduce    per-document max of row_score -> doc_scores, and a 256-doc
//               block-local top-k (bitonic sort in LDS) -> candidates.
//  4. select    one workgroup per query: radix select of the k-th largest
//               candidate key (8 passes of 8 bits over 64-bit keys), gather
//               the k winners, bitonic sort them.
// Keys are (order-preserving score bits << 32) | (0xffffffff - doc id), so one
// unsigned comparison orders by score descending, then id ascending.
#include "msa_internal.h"

#include <algorithm>

namespace msa {
namespace {

constexpr int kDocsPerBlock = 256;
constexpr int kWaves = 4;            // waves per workgroup in the scan kernels

// --------------------------------------------------------------------------
// shared helpers
// --------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// --------------------------------------------------------------------------
// 1. query preparation
// --------------------------------------------------------------------------
// fp32 unit queries: qhat[m, h*dr + i] = qr[m,h,i] / max(|qr[m,h]|, eps) / Hr
template <typename T>
__global__ __launch_bounds__(256) void prep_unit_kernel(const T *__restrict__ qr, float *__restrict__ qhat,
                                                        int M, int Hr, int dr) {
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

// A-fragments for the bf16 scan, from fp32 unit queries (at most 8 tokens).
// Fragment f = h*KS + s, lane l holds A[row = l%16][k = 32 s + 8 (l/16) + e],
// e < 8, for the k-th element of head h.  Row 2m is the bf16 rounding of
// query token m, row 2m+1 the bf16 rounding of the remainder; rows of absent
// tokens are zero.
__global__ __launch_bounds__(256) void prep_frag_kernel(const float *__restrict__ qhat, u32x4 *__restrict__ frag,
                                                        int M, int Hr, int dr) {
  const int KS = dr / 32;
  const int n = Hr * KS * 64;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += gridDim.x * blockDim.x) {
    const int l = idx & 63, f = idx >> 6;
    const int h = f / KS, s = f % KS;
    const int r = l & 15, m = r >> 1;
    uint32_t w[4] = {0, 0, 0, 0};
    if (m < M) {
      const float *src = qhat + (int64_t)m * Hr * dr + h * dr + 32 * s + 8 * (l >> 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = src[e];
        const uint16_t hi = f32_to_bf16(x);
        const uint16_t val = (r & 1) ? f32_to_bf16(x - bf16_to_f32(hi)) : hi;
        w[e >> 1] |= (uint32_t)val << (16 * (e & 1));
      }
    }
    u32x4 o;
    o.x = w[0]; o.y = w[1]; o.z = w[2]; o.w = w[3];
    frag[idx] = o;
  }
}

// --------------------------------------------------------------------------
// 2a. bf16 MFMA scan, at most 8 query tokens (hi/lo rows: 2 per token)
// --------------------------------------------------------------------------
// Lane l of a wave owns bank row (tile*16 + l%16) and the 8-element slice
// 8*(l/16).. of every 32-element k-step; one load instruction of the wave
// reads 16 rows x 64 contiguous bytes.  Heads are loaded in groups of HG,
// one group ahead of the MFMAs that consume them.
#ifndef MSA_SCAN_HG
#define MSA_SCAN_HG 2
#endif
#ifndef MSA_SCAN_PIPE      // 1: keep the head-group loop rolled (fewer registers)
#define MSA_SCAN_PIPE 0
#endif

template <int HR, int KS, int HG>
__global__ __launch_bounds__(256) void scan_mfma_kernel(const uint16_t *__restrict__ kr,
                                                        const u32x4 *__restrict__ frag,
                                                        float *__restrict__ row_score, int64_t n_pool,
                                                        int B, int Tq) {
  constexpr int NF = HR * KS;                     // fragments per 16-row tile per lane
  constexpr int ROW = HR * KS * 32;               // elements per bank row
  constexpr int NG = HR / HG;                     // head groups per tile
  constexpr int GF = HG * KS;                     // fragments per head group
  __shared__ u32x4 afrag[NF * 64];
  for (int i = threadIdx.x; i < NF * 64; i += blockDim.x) afrag[i] = frag[i];
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int diag_src = ((col >> 2) << 4) + col;    // lane holding Gram[col][col]
  const int64_t n_tiles = (n_pool + 15) >> 4;

  for (int64_t tile = (int64_t)blockIdx.x * kWaves + wave; tile < n_tiles;
       tile += (int64_t)gridDim.x * kWaves) {
    const int64_t row = tile * 16 + col;
    const int64_t rowc = row < n_pool ? row : n_pool - 1;
    const uint16_t *rp = kr + rowc * ROW + 8 * grp;
    u32x4 cur[GF];
#pragma unroll
    for (int f = 0; f < GF; ++f) cur[f] = ld16_nt(rp + 32 * f);

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
        for (int f = 0; f < GF; ++f) nxt[f] = ld16_nt(rp + 32 * ((gi + 1) * GF + f));
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
        sc0 += (d[0] + d[1]) * inv;      // token 2*grp     (hi + lo rows)
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
// 2b. VALU scan (fp32, or bf16 with many query tokens): one wave per row
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
// 3. per-document max and block-local top-k candidates
// --------------------------------------------------------------------------
__device__ void bitonic_desc(uint64_t *key, int n) {  // n power of two, blockDim >= 1
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

__global__ __launch_bounds__(kDocsPerBlock) void doc_reduce_kernel(const float *__restrict__ row_score,
                                                                   const int64_t *__restrict__ pool_off,
                                                                   float *__restrict__ doc_scores,
                                                                   uint64_t *__restrict__ cand, int n_docs,
                                                                   int64_t n_pool, int cpb) {
  __shared__ uint64_t key[kDocsPerBlock];
  const int b = blockIdx.y;
  const int d = blockIdx.x * kDocsPerBlock + threadIdx.x;
  uint64_t kk = 0;
  if (d < n_docs) {
    int64_t r0 = pool_off[d], r1 = pool_off[d + 1];
    r0 = max((int64_t)0, min(r0, n_pool));
    r1 = max(r0, min(r1, n_pool));
    const float *rs = row_score + (int64_t)b * n_pool;
    float best = -INFINITY;
    for (int64_t r = r0; r < r1; ++r) best = fmaxf(best, rs[r]);
    doc_scores[(int64_t)b * n_docs + d] = best;
    kk = ((uint64_t)score_key(best) << 32) | (uint64_t)(0xffffffffu - (uint32_t)d);
  }
  key[threadIdx.x] = kk;
  __syncthreads();
  bitonic_desc(key, kDocsPerBlock);
  for (int i = threadIdx.x; i < cpb; i += blockDim.x)
    cand[((int64_t)b * gridDim.x + blockIdx.x) * cpb + i] = key[i];
}

// --------------------------------------------------------------------------
// 4. exact top-k of the candidates
// --------------------------------------------------------------------------
constexpr int kSelThreads = 1024;

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(const uint64_t *__restrict__ cand, int n_cand,
                                                                  int k, int32_t *__restrict__ topk_idx,
                                                                  float *__restrict__ topk_score) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t s_prefix, s_mask;
  __shared__ int s_need, s_count;
  __shared__ uint64_t sel[kMaxTopK];
  const int b = blockIdx.x;
  const uint64_t *c = cand + (int64_t)b * n_cand;
  if (threadIdx.x == 0) { s_prefix = 0; s_mask = 0; s_need = k; s_count = 0; }
  __syncthreads();
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix, mask = s_mask;
    for (int i = threadIdx.x; i < n_cand; i += blockDim.x) {
      const uint64_t x = c[i];
      if ((x & mask) == prefix) atomicAdd(&hist[(x >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int need = s_need, digit = 255;
      for (; digit > 0; --digit) {
        const int cnt = (int)hist[digit];
        if (cnt >= need) break;
        need -= cnt;
      }
      s_need = need;
      s_prefix = prefix | ((uint64_t)digit << shift);
      s_mask = mask | ((uint64_t)255 << shift);
    }
    __syncthreads();
  }
  const uint64_t thr = s_prefix;   // exactly the k-th largest key (keys are unique)
  for (int i = threadIdx.x; i < n_cand; i += blockDim.x) {
    const uint64_t x = c[i];
    if (x >= thr) {
      const int pos = atomicAdd(&s_count, 1);
      if (pos < kMaxTopK) sel[pos] = x;
    }
  }
  __syncthreads();
  int n2 = 1;
  while (n2 < k) n2 <<= 1;
  for (int i = threadIdx.x; i < n2; i += blockDim.x)
    if (i >= min(s_count, kMaxTopK)) sel[i] = 0;
  __syncthreads();
  bitonic_desc(sel, n2);
  for (int i = threadIdx.x; i < k; i += blockDim.x) {
    const uint64_t x = sel[i];
    topk_idx[(int64_t)b * k + i] = (int32_t)(0xffffffffu - (uint32_t)(x & 0xffffffffu));
    topk_score[(int64_t)b * k + i] = key_score((uint32_t)(x >> 32));
  }
}

// --------------------------------------------------------------------------
// dispatch
// --------------------------------------------------------------------------
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool mfma_path(int32_t dtype, int32_t M, int32_t hr, int32_t dr) {
  if (dtype != MSA_BF16 || M > 8) return false;
  const int ks = dr / 32;
  return (ks == 2 || ks == 4) && (hr == 1 || hr == 2 || hr == 4 || hr == 8 || (hr == 16 && ks == 2));
}

template <int HR, int KS>
hipError_t launch_scan_mfma(const msa_route_args &a, const RouteWs &ws, hipStream_t s) {
  constexpr int HG = HR < MSA_SCAN_HG ? HR : MSA_SCAN_HG;
  const int64_t n_tiles = (a.n_pool + 15) / 16;
  int occ = 0;
  hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, scan_mfma_kernel<HR, KS, HG>, 256, 0);
  if (occ < 1) occ = 1;
  const int64_t want = (int64_t)device_info().n_cu * occ;
  const int64_t need = (n_tiles + kWaves - 1) / kWaves;
  const int grid = (int)std::max<int64_t>(1, std::min(want, need));
  hipLaunchKernelGGL((scan_mfma_kernel<HR, KS, HG>), dim3(grid), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t *>(a.kr_pooled),
                     reinterpret_cast<const u32x4 *>(ws.qprep), ws.row_score, a.n_pool, a.batch,
                     a.q_tokens);
  return hipGetLastError();
}

template <typename T, int EPL>
hipError_t launch_scan_valu_t(const msa_route_args &a, const RouteWs &ws, hipStream_t s) {
  const int64_t need = (a.n_pool + kWaves - 1) / kWaves;
  const int64_t want = (int64_t)device_info().n_cu * 8;
  const int grid = (int)std::max<int64_t>(1, std::min(want, need));
  const int lanes_per_head = 64 / a.n_router_heads;
  hipLaunchKernelGGL((scan_valu_kernel<T, EPL>), dim3(grid), dim3(256), 0, s,
                     reinterpret_cast<const T *>(a.kr_pooled), reinterpret_cast<const float *>(ws.qprep),
                     ws.row_score, a.n_pool, a.batch, a.q_tokens, lanes_per_head);
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

size_t route_ws_layout(int32_t dtype, int32_t batch, int32_t q_tokens, int32_t hr, int32_t dr,
                       int32_t n_docs, int64_t n_pool, int32_t top_k, void *base, RouteWs *ws) {
  const int32_t M = batch * q_tokens;
  const int32_t n_blocks = (n_docs + kDocsPerBlock - 1) / kDocsPerBlock;
  const int32_t cpb = std::min(top_k, kDocsPerBlock);
  size_t off = 0;
  const size_t o_rs = off;
  off = align256(off + sizeof(float) * (size_t)batch * (size_t)n_pool);
  const size_t o_q = off;
  size_t qbytes = sizeof(float) * (size_t)M * hr * dr;                 // unit queries
  if (mfma_path(dtype, M, hr, dr)) qbytes += (size_t)hr * (dr / 32) * 64 * 16;  // + fragments
  off = align256(off + qbytes);
  const size_t o_c = off;
  off = align256(off + sizeof(uint64_t) * (size_t)batch * n_blocks * cpb);
  if (ws) {
    char *p = reinterpret_cast<char *>(base);
    ws->row_score = reinterpret_cast<float *>(p + o_rs);
    ws->qprep = p + o_q;
    ws->cand = reinterpret_cast<uint64_t *>(p + o_c);
    ws->n_blocks = n_blocks;
    ws->cand_per_block = cpb;
  }
  return off;
}

hipError_t launch_route(const msa_route_args &a, const RouteWs &ws, hipStream_t s) {
  const int M = a.batch * a.q_tokens;
  float *qhat = reinterpret_cast<float *>(ws.qprep);
  const bool bf16 = a.dtype == MSA_BF16;
  {
    const int n = M * a.n_router_heads;
    const int grid = std::max(1, std::min((n + kWaves - 1) / kWaves, 1024));
    if (bf16)
      hipLaunchKernelGGL(prep_unit_kernel<uint16_t>, dim3(grid), dim3(256), 0, s,
                         reinterpret_cast<const uint16_t *>(a.qr), qhat, M, a.n_router_heads, a.router_dim);
    else
      hipLaunchKernelGGL(prep_unit_kernel<float>, dim3(grid), dim3(256), 0, s,
                         reinterpret_cast<const float *>(a.qr), qhat, M, a.n_router_heads, a.router_dim);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipSuccess;
  hipEvent_t ev0 = reinterpret_cast<hipEvent_t>(a.prof_event_begin);
  hipEvent_t ev1 = reinterpret_cast<hipEvent_t>(a.prof_event_end);
  if (mfma_path(a.dtype, M, a.n_router_heads, a.router_dim)) {
    u32x4 *frag = reinterpret_cast<u32x4 *>(
        reinterpret_cast<char *>(ws.qprep) + sizeof(float) * (size_t)M * a.n_router_heads * a.router_dim);
    const int n = a.n_router_heads * (a.router_dim / 32) * 64;
    hipLaunchKernelGGL(prep_frag_kernel, dim3((n + 255) / 256), dim3(256), 0, s, qhat, frag, M,
                       a.n_router_heads, a.router_dim);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    RouteWs w2 = ws;
    w2.qprep = frag;
    const int ks = a.router_dim / 32;
    if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
    switch (a.n_router_heads * 8 + ks) {
      case 1 * 8 + 2: e = launch_scan_mfma<1, 2>(a, w2, s); break;
      case 1 * 8 + 4: e = launch_scan_mfma<1, 4>(a, w2, s); break;
      case 2 * 8 + 2: e = launch_scan_mfma<2, 2>(a, w2, s); break;
      case 2 * 8 + 4: e = launch_scan_mfma<2, 4>(a, w2, s); break;
      case 4 * 8 + 2: e = launch_scan_mfma<4, 2>(a, w2, s); break;
      case 4 * 8 + 4: e = launch_scan_mfma<4, 4>(a, w2, s); break;
      case 8 * 8 + 2: e = launch_scan_mfma<8, 2>(a, w2, s); break;
      case 8 * 8 + 4: e = launch_scan_mfma<8, 4>(a, w2, s); break;
      case 16 * 8 + 2: e = launch_scan_mfma<16, 2>(a, w2, s); break;
      default: e = hipErrorInvalidValue;
    }
  } else {
    if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
    e = bf16 ? launch_scan_valu<uint16_t>(a, ws, s) : launch_scan_valu<float>(a, ws, s);
  }
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return e;

  hipLaunchKernelGGL(doc_reduce_kernel, dim3(ws.n_blocks, a.batch), dim3(kDocsPerBlock), 0, s, ws.row_score,
                     a.doc_pool_off, a.doc_scores, ws.cand, a.n_docs, a.n_pool, ws.cand_per_block);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_select_kernel, dim3(a.batch), dim3(kSelThreads), 0, s, ws.cand,
                     ws.n_blocks * ws.cand_per_block, a.top_k, a.topk_idx, a.topk_score);
  return hipGetLastError();
}

}  // namespace msa
