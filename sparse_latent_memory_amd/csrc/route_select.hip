// Routing, stage 2 of the method: per-document reduction, the exact top-k,
// and the device side of context assembly.
//
// Method: "EverMind-AI/MSA: Memory Sparse Attention for 100M-Token Contexts"
// (hysenlabs.com), section "How MSA compresses and routes documents" (a
// document's score is its best pooled row; the top-k documents are selected
// and their pooled K/V concatenated); stage 2 of "EverMind Releases
// Memory-Sparse Attention Code for Long-Context AI Models" (toolmesh.ai),
// section "Architectural Design and Inference" (the selected documents' K/V
// are loaded from host memory to the GPU).
//
// Kernels, in launch order:
//  0. map      (document path only, before the scan) per 16-row tile of the
//              bank: the document holding its first row and a bit per row
//              that starts a document, so the scan can reduce each tile per
//              document itself.
//  1. reduce   per block of 256 documents: each document's score ->
//              doc_scores, and the block's best document key -> blockmax.
//              Row path: the max over the document's row scores.  Document
//              path: the max of the scan's part for the tile where the
//              document starts and its continuation parts in later tiles.
//  2. final    one workgroup per query selects the exact top-k: T, the k-th
//              largest block-maximum score, bounds the global k-th key from
//              below (the k blocks behind those maxima hold k keys >= T), so
//              only the blocks whose maximum scores >= T can hold winners;
//              their documents' keys >= T are collected and ordered.  A radix
//              select over all documents covers what that path does not
//              (k > 64, more than 4096 blocks, or too many survivors).  With
//              device-side assembly it also writes the copy plan.
//  3. gather   (device-side assembly only) copy the selected documents'
//              pooled K/V rows from mapped pinned host memory into mem_kv.
// Keys are (order-preserving score bits << 32) | (0xffffffff - doc id), so one
// unsigned comparison orders by score descending, then id ascending.
#include "msa_internal.h"

#include <algorithm>

namespace msa {
namespace {

constexpr int kWaves = kDocsPerBlock / 64;   // waves per workgroup
constexpr int kSortCap = kMaxTopK;           // keys the final selection can order in LDS
constexpr int kFastTopK = 64;                // k up to this uses the block-maximum bound
constexpr int kBallotLists = 16;             // block maxima per lane in the ballot threshold (<= 1024 blocks)
constexpr int kNarrow = 128;                 // block maxima at or above the lane bound searched in two lists
constexpr int kSmallDocs = 4096;             // banks up to this many documents: every key in registers

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o, 64));
  return x;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, o, 64));
  return x;
}

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

// Rank of key x (at index i) among key[0..n): the keys greater than x plus
// the equal keys at lower indices, so every index gets a distinct rank.
__device__ __forceinline__ int rank_of(const uint64_t *key, int n, uint64_t x, int i) {
  int r = 0;
#pragma unroll 8
  for (int j = 0; j < n; ++j) {
    const uint64_t y = key[j];
    r += (y > x) | ((y == x) & (j < i));
  }
  return r;
}

__device__ __forceinline__ uint64_t doc_key(float score, int d) {
  return ((uint64_t)score_key(score) << 32) | (uint64_t)(0xffffffffu - (uint32_t)d);
}

// f(key) for every document d = tid, tid + blockDim, ... with eight loads
// in flight per thread: unconditional loads of clamped indices (a load under
// a branch is waited for before the branch joins)
template <typename F>
__device__ __forceinline__ void for_doc_keys(const float *ds, int n_docs, F f) {
  const int nt = blockDim.x;
  for (int d0 = threadIdx.x; d0 < n_docs; d0 += 8 * nt) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ds[min(d0 + u * nt, n_docs - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (d0 + u * nt < n_docs) f(doc_key(v[u], d0 + u * nt));
  }
}

// The k-th largest of the wave's P*64 nonzero values v[] (0 where fewer
// than k), bit by bit: the count of values >= a candidate is a sum of ballot
// popcounts.
template <int P>
__device__ __forceinline__ uint32_t wave_kth_score(const uint32_t *v, int k) {
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    int c = 0;
#pragma unroll
    for (int u = 0; u < P; ++u) c += __popcll(__ballot(v[u] >= cand));
    if (c >= k) t = cand;
  }
  return t;
}

__device__ __forceinline__ int64_t clamp_row(int64_t r, int64_t n_pool) {
  return r < 0 ? 0 : (r > n_pool ? n_pool : r);
}

// Maximum of one key per thread over the workgroup (all threads call; the
// result is valid in every thread).
__device__ __forceinline__ uint64_t block_max_key(uint64_t k, uint64_t *red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t y = __shfl_xor(k, o, 64);
    k = y > k ? y : k;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();                       // red[] free from a previous use
  if ((threadIdx.x & 63) == 0) red[wave] = k;
  __syncthreads();
  uint64_t m = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = red[w] > m ? red[w] : m;
  return m;
}

// --------------------------------------------------------------------------
// 0. document map (document path)
// --------------------------------------------------------------------------
// Thread d owns the tiles whose first row lies in document d (with valid
// offsets every tile has exactly one such document): it records d and the
// rows of the tile where a document starts, including the bank's end (row
// n_pool), which keeps the rows past it out of every document.
__global__ __launch_bounds__(256) void doc_map_kernel(const int64_t *__restrict__ pool_off,
                                                      int32_t *__restrict__ tile_doc,
                                                      uint32_t *__restrict__ tile_bits, int n_docs,
                                                      int64_t n_pool) {
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= n_docs) return;
  const int64_t r0 = clamp_row(pool_off[d], n_pool);
  const int64_t r1 = max(r0, clamp_row(pool_off[d + 1], n_pool));
  const int64_t n_tiles = (n_pool + 15) >> 4;
  for (int64_t t = (r0 + 15) >> 4; t * 16 < r1 && t < n_tiles; ++t) {
    const int64_t base = t * 16;
    uint32_t bits = r0 == base ? 1u : 0u;
    for (int i = 1; i <= 16 && d + i <= n_docs; ++i) {   // a tile holds at most 16 starts
      const int64_t s = d + i < n_docs ? clamp_row(pool_off[d + i], n_pool) : n_pool;
      if (s >= base + 16) break;
      if (s > base) bits |= 1u << (s - base);
    }
    tile_doc[t] = d;
    tile_bits[t] = bits;
  }
}

// --------------------------------------------------------------------------
// 1. per-document scores and block maxima
// --------------------------------------------------------------------------
// Row path: per 256-document block and query, the max over the document's
// row scores (row_score holds n_parts partial token maxima per query and
// row; the document max runs over all of them).
__global__ __launch_bounds__(kDocsPerBlock) void doc_rows_kernel(
    const float *__restrict__ row_score, const int64_t *__restrict__ pool_off, float *__restrict__ doc_scores,
    uint64_t *__restrict__ blockmax, int n_docs, int64_t n_pool, int n_parts) {
  __shared__ uint64_t red[kWaves];
  const int b = blockIdx.y, n_blocks = gridDim.x;
  const int d = blockIdx.x * kDocsPerBlock + threadIdx.x;
  uint64_t kk = 0;
  if (d < n_docs) {
    const int64_t r0 = clamp_row(pool_off[d], n_pool);
    const int64_t r1 = max(r0, clamp_row(pool_off[d + 1], n_pool));
    float best = -INFINITY;
    for (int part = 0; part < n_parts; ++part) {
      const float *rs = row_score + ((int64_t)b * n_parts + part) * n_pool;
      int64_t r = r0;
      for (; r + 4 <= r1; r += 4) {    // independent loads in flight
        const float x0 = rs[r], x1 = rs[r + 1], x2 = rs[r + 2], x3 = rs[r + 3];
        best = fmaxf(best, fmaxf(fmaxf(x0, x1), fmaxf(x2, x3)));
      }
      for (; r < r1; ++r) best = fmaxf(best, rs[r]);
    }
    doc_scores[(int64_t)b * n_docs + d] = best;
    kk = doc_key(best, d);
  }
  const uint64_t m = block_max_key(kk, red);
  if (threadIdx.x == 0) blockmax[(int64_t)b * n_blocks + blockIdx.x] = m;
}

// Document path: per 256-document block and QC queries (the query stride
// is a multiple of QC), a document's score is the max of the scan's part
// for the tile where it starts and the continuation parts of the later
// tiles it covers.
template <int QC>
__global__ __launch_bounds__(kDocsPerBlock) void doc_parts_kernel(
    const float *__restrict__ doc_part, const float *__restrict__ tile_cont, const int64_t *__restrict__ pool_off,
    float *__restrict__ doc_scores, uint64_t *__restrict__ blockmax, int n_docs, int64_t n_pool, int B,
    int qstride) {
  const int n_blocks = gridDim.x;
  const int q0 = blockIdx.y * QC;
  const int d = blockIdx.x * kDocsPerBlock + threadIdx.x;
  const bool valid = d < n_docs;
  float sc[QC];
#pragma unroll
  for (int i = 0; i < QC; ++i) sc[i] = -INFINITY;
  if (valid) {
    const f32x4 *p = reinterpret_cast<const f32x4 *>(doc_part + (int64_t)d * qstride + q0);
#pragma unroll
    for (int v = 0; v < QC / 4; ++v) {
      const f32x4 x = p[v];
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[4 * v + e] = x[e];
    }
    const int64_t r0 = clamp_row(pool_off[d], n_pool);
    const int64_t r1 = max(r0, clamp_row(pool_off[d + 1], n_pool));
    if (r1 > r0) {
      for (int64_t t = (r0 >> 4) + 1; t <= ((r1 - 1) >> 4); ++t) {   // tiles the document continues into
        const f32x4 *c = reinterpret_cast<const f32x4 *>(tile_cont + t * qstride + q0);
#pragma unroll
        for (int v = 0; v < QC / 4; ++v) {
          const f32x4 x = c[v];
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[4 * v + e] = fmaxf(sc[4 * v + e], x[e]);
        }
      }
    }
  }
  // block maxima of all QC queries behind one barrier: per wave the best
  // score (shuffles) and the lowest document holding it (ballot), then the
  // max of the four waves' keys
  __shared__ uint64_t wmax[kWaves][QC];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d0 = blockIdx.x * kDocsPerBlock + wave * 64;  // document of lane 0
#pragma unroll
  for (int i = 0; i < QC; ++i) {
    const int b = q0 + i;
    if (b >= B) break;                   // (uniform)
    if (valid) doc_scores[(int64_t)b * n_docs + d] = sc[i];
    const float v = valid ? sc[i] : -INFINITY;
    float m = v;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    // keys order scores by their key bits, so compare those (-0 == +0 there)
    const uint64_t hit = __ballot(valid && score_key(v) == score_key(m));
    if (lane == 0) wmax[wave][i] = hit ? doc_key(m, d0 + __ffsll((unsigned long long)hit) - 1) : 0ull;
  }
  __syncthreads();
  if (threadIdx.x < QC && q0 + (int)threadIdx.x < B) {
    uint64_t best = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) best = wmax[w][threadIdx.x] > best ? wmax[w][threadIdx.x] : best;
    blockmax[(int64_t)(q0 + threadIdx.x) * n_blocks + blockIdx.x] = best;
  }
}

// --------------------------------------------------------------------------
// Context assembly plan of one query: its documents in rank order while they
// fit in the memory after len0 rows; the first one that does not fit closes
// the plan for every later rank.  doc(r) is rank r's document, or a negative
// value, which ends the list.  Writes plan_b[r] for every rank (rows 0 when
// not copied) and the new length.  Every thread of the block calls it; k <= 64
// runs in wave 0 alone (a prefix over lanes), larger k serially over LDS
// (r0s, prow, pdst: k entries each).
// --------------------------------------------------------------------------
template <typename DocOf>
__device__ __forceinline__ void assembly_plan(DocOf doc, int k, const int64_t *__restrict__ pool_off, int n_docs,
                                              int64_t n_pool, int mem_cap, int64_t len0, GatherPlan *plan_b,
                                              int32_t *mem_len_b, uint64_t *r0s, int32_t *prow, int32_t *pdst) {
  const int tid = threadIdx.x;
  // rank r's first row and row count; a missing document counts as too large
  auto rows_of = [&](int r, int64_t *r0) -> int64_t {
    const int d = doc(r);
    if (d < 0) { *r0 = 0; return (int64_t)mem_cap + 1; }
    const int dd = min(d, n_docs - 1);
    *r0 = clamp_row(pool_off[dd], n_pool);
    const int64_t r1 = max(*r0, clamp_row(pool_off[dd + 1], n_pool));
    return min(r1 - *r0, (int64_t)mem_cap + 1);
  };
  if (k <= 64) {
    if ((tid >> 6) != 0) return;
    const int r = tid;
    int64_t r0 = 0, pr = 0;
    if (r < k) pr = rows_of(r, &r0);
    int64_t inc = pr;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up((long)inc, o, 64);
      if (r >= o) inc += y;
    }
    const bool open = r < k && len0 + inc <= mem_cap;
    GatherPlan p = {0, 0, 0};
    if (open) {
      p.src_row = r0;
      p.rows = (int32_t)pr;
      p.dst_row = (int32_t)(len0 + inc - pr);
    }
    if (r < k) plan_b[r] = p;
    const uint64_t end = __ballot(open);                   // open ranks are a prefix
    const int n_open = __popcll(end);
    const int64_t len = n_open ? len0 + __shfl(inc, n_open - 1, 64) : len0;
    if (r == 0) *mem_len_b = (int32_t)len;
    return;
  }
  for (int r = tid; r < k; r += blockDim.x) {              // every rank's offsets loaded in parallel
    int64_t r0 = 0;
    prow[r] = (int32_t)rows_of(r, &r0);
    r0s[r] = (uint64_t)r0;
  }
  __syncthreads();
  if (tid == 0) {                                          // prefix over LDS only
    int64_t len = len0;
    bool open = true;
    for (int r = 0; r < k; ++r) {
      open = open && len + prow[r] <= mem_cap;
      pdst[r] = open ? (int32_t)len : -1;
      if (open) len += prow[r];
    }
    *mem_len_b = (int32_t)len;
  }
  __syncthreads();
  for (int r = tid; r < k; r += blockDim.x) {
    GatherPlan p = {0, 0, 0};
    if (pdst[r] >= 0) {
      p.src_row = (int64_t)r0s[r];
      p.rows = prow[r];
      p.dst_row = pdst[r];
    }
    plan_b[r] = p;
  }
}

// --------------------------------------------------------------------------
// 2. exact top-k per query
// --------------------------------------------------------------------------
// A separate launch rather than a last-block-done tail on the kernel above:
// the device-scope release every block would need writes back its XCD's L2,
// and hundreds of those cost far more than one kernel boundary.
__global__ __launch_bounds__(kDocsPerBlock) void topk_final_kernel(
    const uint64_t *__restrict__ blockmax, const float *__restrict__ doc_scores,
    const int64_t *__restrict__ pool_off, int32_t *__restrict__ topk_idx, float *__restrict__ topk_score,
    GatherPlan *__restrict__ plan, int32_t *__restrict__ mem_len, int mem_cap, int append, int n_blocks,
    int n_docs, int64_t n_pool, int k) {
  __shared__ uint64_t sel[kSortCap];
  __shared__ uint32_t hist[kWaves][256];
  __shared__ int top_blk[kFastTopK];
  __shared__ uint32_t nar_key[kNarrow];
  __shared__ int nar_blk[kNarrow];
  __shared__ uint64_t ranked[kFastTopK];
  __shared__ uint64_t s_thr;
  __shared__ int s_nb;
  __shared__ int s_count, s_need;
  __shared__ uint64_t s_prefix, s_mask;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6;
  const uint64_t *bm = blockmax + (int64_t)b * n_blocks;
  const float *ds = doc_scores + (int64_t)b * n_docs;
  const int len_in = plan && append ? mem_len[b] : 0;   // read early; written at the end

  bool sorted = false;
  if (k <= kFastTopK && n_docs <= kSmallDocs) {
    // A small bank (the block bound is weak when there are fewer blocks than
    // k): every document key stays in registers, thread t holding documents
    // t, t + 256, ...  Each wave finds, bit by bit from ballot popcounts, the
    // k-th largest score among its own documents; that wave holds k
    // documents scoring at least that much, so the largest of the four wave
    // values, L, bounds the k-th largest score overall from below, and the
    // documents scoring >= L - k from the best wave and at most k (plus
    // ties) from each other one - hold every winner.  One barrier shares the
    // four values; the survivors are ranked below.
    __shared__ uint32_t s_wl[kWaves];
    constexpr int PER = kSmallDocs / kDocsPerBlock;
    const int n_per = (n_docs + kDocsPerBlock - 1) / kDocsPerBlock;   // keys a thread holds, at most PER
    uint64_t x[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int d = tid + u * kDocsPerBlock;
      const float v = ds[min(d, n_docs - 1)];              // unconditional: a guarded load is waited for at once
      x[u] = d < n_docs ? doc_key(v, d) : 0ull;
    }
    if (tid == 0) s_count = 0;
    // score halves of the keys, 0 for slots past the last document (a
    // candidate is never 0, so those never count); the search over 8 or 16
    // slots is chosen once, with no branch inside it
    uint32_t sk[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) sk[u] = (uint32_t)(x[u] >> 32);
    const uint32_t wl = n_per <= PER / 2 ? wave_kth_score<PER / 2>(sk, k) : wave_kth_score<PER>(sk, k);
    if ((tid & 63) == 0) s_wl[wave] = wl;
    __syncthreads();
    uint32_t L = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) L = max(L, s_wl[w]);
    const uint64_t thr = (uint64_t)L << 32;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if (tid + u * kDocsPerBlock < n_docs && x[u] >= thr) {
        const int pos = atomicAdd(&s_count, 1);
        if (pos < kSortCap) sel[pos] = x[u];
      }
    }
    __syncthreads();
    sorted = true;                                         // at most n_docs <= kSortCap survivors
  } else if (k <= kFastTopK && n_blocks <= kSortCap) {
    if (n_blocks <= 64 * kBallotLists) {
      // Wave 0 finds the score half T of the bound: the k-th largest block
      // maximum (score bits only).  The blocks whose maximum scores >= T -
      // k of them, more only where scores tie - hold every winner, all with
      // keys >= T << 32.  Each lane holds up to kBallotLists maxima.
      //  1. L, the k-th largest of the lane maxima, bounds T from below (k
      //     lanes hold a maximum >= L), so only the maxima >= L matter;
      //  2. those are compacted into LDS (if at most kNarrow of them) and T
      //     is found bit by bit over them: the count of maxima >= a
      //     candidate is a sum of ballot popcounts, and the bits above the
      //     highest one where L and the largest maximum differ are already
      //     fixed, since T lies between the two.
      if (wave == 0) {
        const int lane = tid & 63;
        const uint64_t below = (1ull << lane) - 1ull;
        const int n_lists = (n_blocks + 63) / 64;
        uint32_t sk[kBallotLists];
        uint32_t lm = 0;
#pragma unroll
        for (int m = 0; m < kBallotLists; ++m) {
          const int i = lane + 64 * m;
          const uint32_t x = (uint32_t)(bm[min(i, n_blocks - 1)] >> 32);   // unconditional, as below
          sk[m] = i < n_blocks ? x : 0u;
          lm = max(lm, sk[m]);
        }
        // (wave-uniform values are made scalar, so the bit loops below run on
        // scalar registers and branches)
        const uint32_t mx = __builtin_amdgcn_readfirstlane(wave_max_u32(lm));
        // 1. L over one list, from the highest bit where the lane maxima differ
        uint32_t L = 0;
        {
          const uint32_t mn = __builtin_amdgcn_readfirstlane(wave_min_u32(lm));
          const int hb = mx == mn ? -1 : 31 - __builtin_clz(mx ^ mn);
          L = hb < 0 ? mx : (hb == 31 ? 0u : (mx >> (hb + 1)) << (hb + 1));
          for (int bit = hb; bit >= 0; --bit) {
            const uint32_t cand = L | (1u << bit);
            if (__popcll(__ballot(lm >= cand)) >= k) L = cand;
          }
        }
        // 2. compaction of the maxima >= L (keys and block numbers)
        int n_s = 0;
#pragma unroll
        for (int m = 0; m < kBallotLists; ++m) {
          if (m < n_lists) {                               // uniform
            const int i = lane + 64 * m;
            const bool take = i < n_blocks && sk[m] >= L;
            const uint64_t mask = __ballot(take);
            const int pos = n_s + __popcll(mask & below);
            if (take && pos < kNarrow) { nar_key[pos] = sk[m]; nar_blk[pos] = i; }
            n_s += __popcll(mask);
          }
        }
        // LDS operations of one wave complete in order; keep the compiler's too
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        uint32_t T = 0;
        int base = 0;
        if (n_s <= kNarrow) {
          uint32_t nk[kNarrow / 64];
          int nbk[kNarrow / 64];
#pragma unroll
          for (int m = 0; m < kNarrow / 64; ++m) {
            const int i = lane + 64 * m;
            nk[m] = i < n_s ? nar_key[i] : 0u;
            nbk[m] = i < n_s ? nar_blk[i] : 0;
          }
          const int hb = L == mx ? -1 : 31 - __builtin_clz(L ^ mx);
          T = hb < 0 ? L : (hb == 31 ? 0u : (L >> (hb + 1)) << (hb + 1));
          for (int bit = hb; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int m = 0; m < kNarrow / 64; ++m) cnt += __popcll(__ballot(nk[m] >= cand));
            if (cnt >= k) T = cand;
          }
#pragma unroll
          for (int m = 0; m < kNarrow / 64; ++m) {
            const bool take = lane + 64 * m < n_s && nk[m] >= T;
            const uint64_t mask = __ballot(take);
            const int pos = base + __popcll(mask & below);
            if (take && pos < kFastTopK) top_blk[pos] = nbk[m];
            base += __popcll(mask);
          }
        } else {
          // many maxima tie near the bound: the same search over every list
          for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int m = 0; m < kBallotLists; ++m)
              if (m < n_lists) cnt += __popcll(__ballot(sk[m] >= cand));
            if (cnt >= k) T = cand;
          }
#pragma unroll
          for (int m = 0; m < kBallotLists; ++m) {
            if (m < n_lists) {
              const int i = lane + 64 * m;
              const bool take = i < n_blocks && sk[m] >= T;
              const uint64_t mask = __ballot(take);
              const int pos = base + __popcll(mask & below);
              if (take && pos < kFastTopK) top_blk[pos] = i;
              base += __popcll(mask);
            }
          }
        }
        if (lane == 0) {
          s_nb = base;
          s_thr = (uint64_t)T << 32;
          s_count = 0;
        }
      }
    } else {
      int nb2 = 1;
      while (nb2 < n_blocks) nb2 <<= 1;
      for (int i = tid; i < nb2; i += blockDim.x) sel[i] = i < n_blocks ? bm[i] : 0;
      __syncthreads();
      bitonic_desc(sel, nb2);
      const int nb = min(k, n_blocks);
      if (tid < nb) top_blk[tid] = (int)((0xffffffffu - (uint32_t)(sel[tid] & 0xffffffffu)) / kDocsPerBlock);
      if (tid == 0) {
        s_nb = nb;
        s_thr = n_blocks >= k ? sel[k - 1] : 0;
        s_count = 0;
      }
    }
    __syncthreads();
    const int nb = s_nb;
    const uint64_t thr = s_thr;
    if (nb <= kFastTopK) {
      // the documents of the selected blocks whose keys reach the bound:
      // thread t takes position t of every block, sixteen blocks' loads in
      // flight before any is used (blockDim == kDocsPerBlock)
      for (int j0 = 0; j0 < nb; j0 += 16) {
        float v[16];
        int dd[16];
        // unconditional loads of clamped indices: a load under a branch is
        // waited for before the branch joins, which would serialize them
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int blk = j0 + u < nb ? min(max(top_blk[j0 + u], 0), n_blocks - 1) : 0;
          dd[u] = j0 + u < nb ? blk * kDocsPerBlock + tid : n_docs;
          v[u] = ds[min(dd[u], n_docs - 1)];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (dd[u] < n_docs) {
            const uint64_t x = doc_key(v[u], dd[u]);
            if (x >= thr) {
              const int pos = atomicAdd(&s_count, 1);
              if (pos < kSortCap) sel[pos] = x;
            }
          }
        }
      }
      __syncthreads();
      sorted = s_count <= kSortCap;
    }
  }
  if (!sorted) {
    // radix select of the k-th largest document key, 8 bits per pass,
    // wave-private histograms
    if (tid == 0) { s_prefix = 0; s_mask = 0; s_need = k; s_count = 0; }
    __syncthreads();
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int i = tid; i < kWaves * 256; i += blockDim.x) (&hist[0][0])[i] = 0;
      __syncthreads();
      const uint64_t prefix = s_prefix, mask = s_mask;
      for_doc_keys(ds, n_docs, [&](uint64_t x) {
        if ((x & mask) == prefix) atomicAdd(&hist[wave][(x >> shift) & 255u], 1u);
      });
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
    for_doc_keys(ds, n_docs, [&](uint64_t x) {
      if (x >= thr) {
        const int pos = atomicAdd(&s_count, 1);
        if (pos < kSortCap) sel[pos] = x;
      }
    });
    __syncthreads();
  }
  // Order the survivors.  At most one per thread: rank counting (a key's
  // rank is the number of keys before it, greater or equal at a lower index,
  // found by one broadcast pass over LDS behind a single barrier, where a
  // bitonic sort of 256 keys takes 36 barrier-separated stages); more: sort.
  const int n_sel = min(s_count, kSortCap);
  uint64_t *top = sel;                   // the k winners in order
  if (k <= kFastTopK && n_sel <= (int)blockDim.x && n_sel >= k) {
    if (tid < n_sel) {
      const uint64_t x = sel[tid];
      const int r = rank_of(sel, n_sel, x, tid);
      if (r < k) ranked[r] = x;
    }
    top = ranked;
  } else {
    int n2 = 1;
    while (n2 < n_sel) n2 <<= 1;
    for (int i = n_sel + tid; i < n2; i += blockDim.x) sel[i] = 0;
    __syncthreads();
    bitonic_desc(sel, n2);
  }
  __syncthreads();
  for (int i = tid; i < k; i += blockDim.x) {
    const uint64_t x = top[i];
    topk_idx[(int64_t)b * k + i] = (int32_t)(0xffffffffu - (uint32_t)(x & 0xffffffffu));
    topk_score[(int64_t)b * k + i] = key_score((uint32_t)(x >> 32));
  }
  if (!plan) return;
  __shared__ int32_t prow[kMaxTopK], pdst[kMaxTopK];
  __syncthreads();                       // top[] is reused by the plan
  const int64_t len0 = append ? max(0, min(len_in, mem_cap)) : 0;
  assembly_plan([&](int r) { return (int)(0xffffffffu - (uint32_t)(top[r] & 0xffffffffu)); }, k, pool_off, n_docs,
                n_pool, mem_cap, len0, plan + (int64_t)b * k, mem_len + b, top, prow, pdst);
}

// Context assembly from given top-k ids (msa_assemble): the plan alone.
__global__ __launch_bounds__(kDocsPerBlock) void assemble_plan_kernel(
    const int32_t *__restrict__ topk_idx, const int64_t *__restrict__ pool_off, GatherPlan *__restrict__ plan,
    int32_t *__restrict__ mem_len, int mem_cap, int append, int n_docs, int64_t n_pool, int k) {
  __shared__ uint64_t r0s[kMaxTopK];
  __shared__ int32_t prow[kMaxTopK], pdst[kMaxTopK];
  const int b = blockIdx.x;
  const int64_t len0 = append ? max(0, min(mem_len[b], mem_cap)) : 0;
  const int32_t *ids = topk_idx + (int64_t)b * k;
  assembly_plan([&](int r) { const int d = ids[r]; return d >= 0 && d < n_docs ? d : -1; }, k, pool_off, n_docs,
                n_pool, mem_cap, len0, plan + (int64_t)b * k, mem_len + b, r0s, prow, pdst);
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

}  // namespace

hipError_t launch_assemble(const msa_assemble_args &a, GatherPlan *plan, const void *host_kv_dev, hipStream_t s) {
  hipLaunchKernelGGL(assemble_plan_kernel, dim3(a.batch), dim3(kDocsPerBlock), 0, s, a.topk_idx, a.doc_pool_off, plan,
                     a.mem_len, a.mem_cap, a.append, a.n_docs, a.n_pool, a.top_k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t elt = a.kv_dtype == MSA_BF16 ? 2 : 4;
  const int64_t row_vecs = (int64_t)(2 * (size_t)a.n_kv_heads * a.head_dim * elt / 16);
  hipLaunchKernelGGL(gather_kernel, dim3(a.top_k, a.batch), dim3(256), 0, s,
                     reinterpret_cast<const u32x4 *>(host_kv_dev), reinterpret_cast<u32x4 *>(a.mem_kv), plan,
                     a.top_k, a.mem_cap, row_vecs);
  return hipGetLastError();
}

hipError_t launch_doc_map(const int64_t *pool_off, int32_t n_docs, int64_t n_pool, int32_t *tile_doc,
                          uint32_t *tile_bits, hipStream_t s) {
  hipLaunchKernelGGL(doc_map_kernel, dim3((n_docs + 255) / 256), dim3(256), 0, s, pool_off, tile_doc, tile_bits,
                     n_docs, n_pool);
  return hipGetLastError();
}

hipError_t launch_select(const msa_route_args &a, const RouteWs &ws, const void *host_kv_dev, hipStream_t s) {
  const bool device_gather = host_kv_dev != nullptr;
  if (ws.qstride > 0) {
    // query chunk: 16 on the wide scan's stride (a multiple of 16), else the stride (4 or 8)
    const int qc = ws.qstride % 16 == 0 ? 16 : ws.qstride;
    const dim3 grid(ws.n_blocks, (a.batch + qc - 1) / qc);
    if (qc == 16)
      hipLaunchKernelGGL(doc_parts_kernel<16>, grid, dim3(kDocsPerBlock), 0, s, ws.doc_part, ws.tile_cont,
                         a.doc_pool_off, a.doc_scores, ws.blockmax, a.n_docs, a.n_pool, a.batch, ws.qstride);
    else if (qc == 8)
      hipLaunchKernelGGL(doc_parts_kernel<8>, grid, dim3(kDocsPerBlock), 0, s, ws.doc_part, ws.tile_cont,
                         a.doc_pool_off, a.doc_scores, ws.blockmax, a.n_docs, a.n_pool, a.batch, ws.qstride);
    else
      hipLaunchKernelGGL(doc_parts_kernel<4>, grid, dim3(kDocsPerBlock), 0, s, ws.doc_part, ws.tile_cont,
                         a.doc_pool_off, a.doc_scores, ws.blockmax, a.n_docs, a.n_pool, a.batch, ws.qstride);
  } else
    hipLaunchKernelGGL(doc_rows_kernel, dim3(ws.n_blocks, a.batch), dim3(kDocsPerBlock), 0, s, ws.row_score,
                       a.doc_pool_off, a.doc_scores, ws.blockmax, a.n_docs, a.n_pool, ws.n_parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_final_kernel, dim3(a.batch), dim3(kDocsPerBlock), 0, s, ws.blockmax, a.doc_scores,
                     a.doc_pool_off, a.topk_idx, a.topk_score, device_gather ? ws.plan : nullptr, a.mem_len,
                     a.mem_cap, a.append, ws.n_blocks, a.n_docs, a.n_pool, a.top_k);
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
