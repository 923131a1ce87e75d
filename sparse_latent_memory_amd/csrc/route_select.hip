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
//  1. block    per 256-document block: per-document max -> doc_scores, block
//              top-k by a bitonic sort in LDS -> candidates.
//  2. final    one workgroup per query selects the exact top-k: the k-th
//              largest block maximum T bounds the global k-th key from below
//              and only the k blocks whose maximum is >= T can hold winners,
//              so at most k*k keys are ranked; a radix select over
//              wave-private histograms covers what that path does not
//              (k > 64, more than 4096 blocks).  With device-side assembly it
//              also writes the copy plan.
// The final survivors (at most one per thread) are ordered by rank counting
// rather than sorting: a key's rank is the number of keys before it
// (greater, or equal and at a lower index), found by one pass over the set
// in LDS (every lane of a wave reads the same word, a broadcast) behind a
// single barrier, where a bitonic sort of 256 keys takes 36 barrier-separated
// stages (measured 2 us faster).  The 256-document blocks and the block
// maxima stay sorted: there the rank pass measured slower than the sort.
//  3. gather   (device-side assembly only) copy the selected documents'
//              pooled K/V rows from mapped pinned host memory into mem_kv.
// Keys are (order-preserving score bits << 32) | (0xffffffff - doc id), so one
// unsigned comparison orders by score descending, then id ascending.
#include "msa_internal.h"

#include <algorithm>

namespace msa {
namespace {

constexpr int kWaves = kDocsPerBlock / 64;   // waves per workgroup
constexpr int kSortCap = kMaxTopK;           // keys the final selection can sort in LDS
constexpr int kFastTopK = 64;                // k up to this uses the block-maximum bound (<= k*k survivors)
constexpr int kBallotLists = 16;             // block maxima per lane in the ballot threshold (<= 1024 blocks)

// --------------------------------------------------------------------------
// per-document max, block top-k, and the exact final top-k
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

// Per 256-document block: per-document max -> doc_scores, and the block's
// top-cpb keys sorted descending -> cand.  row_score holds n_parts partial
// token maxima per query and row; the document max runs over all of them.
__global__ __launch_bounds__(kDocsPerBlock) void doc_block_topk_kernel(
    const float *__restrict__ row_score, const int64_t *__restrict__ pool_off, float *__restrict__ doc_scores,
    uint64_t *__restrict__ cand, int n_docs, int64_t n_pool, int cpb, int n_parts) {
  __shared__ uint64_t key[kDocsPerBlock];
  const int b = blockIdx.y, n_blocks = gridDim.x;
  const int tid = threadIdx.x;
  const int d = blockIdx.x * kDocsPerBlock + tid;
  uint64_t kk = 0;
  if (d < n_docs) {
    int64_t r0 = pool_off[d], r1 = pool_off[d + 1];
    r0 = max((int64_t)0, min(r0, n_pool));
    r1 = max(r0, min(r1, n_pool));
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
  __shared__ uint64_t ranked[kFastTopK];
  __shared__ uint64_t s_thr;
  __shared__ int s_nb;
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
    if (n_blocks <= 64 * kBallotLists) {
      // Wave 0 finds the score half T of that bound bit by bit: each lane
      // holds up to kBallotLists block maxima, and the count of maxima
      // scoring >= a candidate is a sum of ballot popcounts (no barrier, no
      // sort).  The lists whose maximum scores >= T - k of them, more only
      // where scores tie - hold every winner, all with keys >= T << 32.
      if (wave == 0) {
        const int lane = tid & 63;
        uint32_t sk[kBallotLists];
#pragma unroll
        for (int m = 0; m < kBallotLists; ++m) {
          const int i = lane + 64 * m;
          sk[m] = i < n_blocks ? (uint32_t)(c[(int64_t)i * cpb] >> 32) : 0u;
        }
        uint32_t T = 0;
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t cand = T | (1u << bit);
          int cnt = 0;
#pragma unroll
          for (int m = 0; m < kBallotLists; ++m) cnt += __popcll(__ballot(sk[m] >= cand));
          if (cnt >= k) T = cand;
        }
        const uint64_t below = (1ull << lane) - 1ull;
        int base = 0;
#pragma unroll
        for (int m = 0; m < kBallotLists; ++m) {
          const int i = lane + 64 * m;
          const bool take = i < n_blocks && sk[m] >= T;
          const uint64_t mask = __ballot(take);
          const int pos = base + __popcll(mask & below);
          if (take && pos < kFastTopK) top_blk[pos] = i;
          base += __popcll(mask);
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
      for (int i = tid; i < nb2; i += blockDim.x) sel[i] = i < n_blocks ? c[(int64_t)i * cpb] : 0;
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
  uint64_t *top = sel;                   // the k winners in order
  if (k <= kFastTopK && n_sel <= (int)blockDim.x && n_sel >= k) {
    // one survivor per thread (at least k of them: every top-k key survives)
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
  // ---- context assembly plan: documents in rank order while they fit ----
  __shared__ int32_t prow[kMaxTopK], pdst[kMaxTopK];
  __syncthreads();                       // top[] is reused below
  for (int r = tid; r < k; r += blockDim.x) {   // every rank's offsets loaded in parallel
    const int dd = (int)(0xffffffffu - (uint32_t)(top[r] & 0xffffffffu));
    int64_t r0 = pool_off[dd], r1 = pool_off[dd + 1];
    r0 = max((int64_t)0, min(r0, n_pool));
    r1 = max(r0, min(r1, n_pool));
    top[r] = (uint64_t)r0;
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
      p.src_row = (int64_t)top[r];
      p.rows = prow[r];
      p.dst_row = pdst[r];
    }
    plan[(int64_t)b * k + r] = p;
  }
}

// --------------------------------------------------------------------------
// device-side assembly: one workgroup per (rank, query), reading the
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

hipError_t launch_select(const msa_route_args &a, const RouteWs &ws, const void *host_kv_dev, hipStream_t s) {
  const bool device_gather = host_kv_dev != nullptr;
  hipLaunchKernelGGL(doc_block_topk_kernel, dim3(ws.n_blocks, a.batch), dim3(kDocsPerBlock), 0, s, ws.row_score,
                     a.doc_pool_off, a.doc_scores, ws.cand, a.n_docs, a.n_pool, ws.cand_per_block, ws.n_parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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
