// Stage 1: chunk-mean pooling with document-wise RoPE on K.
//
// Method: "EverMind-AI/MSA: Memory Sparse Attention for 100M-Token Contexts"
// (hysenlabs.com), section "How MSA compresses and routes documents", and
// "EverMind Releases Memory-Sparse Attention Code for Long-Context AI Models"
// (toolmesh.ai), section "Architectural Design and Inference" (stage 1, the
// cached pooled triples; positions restart at zero per document).
//
// Kernel design (HBM-bound: reads 2*Hkv*D + Hr*dr elements per token, writes
// 1/P of that):
// - a workgroup walks pooled rows grid-stride; each lane owns one slot for
//   the whole launch: a 16-byte vector of K rotate-half pairs (the VW
//   elements at j0.. and their partners at j0+D/2..), of V or of Kr, and one
//   of SPL lanes sharing that vector's tokens (token u goes to lane u % SPL),
//   so one row is read by every lane at once, coalesced, each token once;
// - RoPE of K: the lane's tokens sit at p0 + part, p0 + part + SPL, ...; the
//   phasor e^{i p w_j} starts exact for each row (angle reduced in fp64) and
//   advances by e^{i SPL w_j} per token (relative drift ~1e-7 per step, far
//   below a bf16 step for any chunk length); the rotated vectors are summed
//   directly;
// - the SPL partial sums of a vector meet by lane shuffles (adjacent lanes).
#include "msa_internal.h"

namespace msa {
namespace {

#ifndef MSA_POOL_KSPLIT      // lanes sharing one K vector
#define MSA_POOL_KSPLIT 2
#endif
#ifndef MSA_POOL_VSPLIT      // lanes sharing one V or Kr vector
#define MSA_POOL_VSPLIT 1
#endif
#ifndef MSA_POOL_UNROLL
#define MSA_POOL_UNROLL 8
#endif
constexpr int kUnroll = MSA_POOL_UNROLL;   // tokens in flight per lane (x2 loads for K)

template <typename T, int KSPL, int VSPL>
__global__ __launch_bounds__(512) void pool_kernel(
    const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ kr,
    const int64_t *__restrict__ tok_off, const int64_t *__restrict__ pool_off,
    T *__restrict__ kv_out, T *__restrict__ kr_out, int n_docs, int64_t n_tokens, int64_t n_pool,
    int P, int Hkv, int D, int Hr, int dr, double log2_theta, int kr_tiled, int64_t kr_row_base) {
  constexpr int VW = Elt<T>::kPerVec;
  __shared__ double omega[64];
  const int half = D / 2;
  for (int j = threadIdx.x; j < half; j += blockDim.x) omega[j] = exp2(-(2.0 * j / D) * log2_theta);
  __syncthreads();

  const int n_kp = Hkv * half / VW;
  const int n_v = Hkv * D / VW;
  const int n_r = Hr * dr / VW;
  const int n_slots = n_kp * KSPL + (n_v + n_r) * VSPL;
  const int64_t krow = (int64_t)Hkv * D;
  const int64_t rrow = (int64_t)Hr * dr;

  for (int slot = threadIdx.x; slot < n_slots; slot += blockDim.x) {
    const bool is_k = slot < n_kp * KSPL;
    const int task = is_k ? slot / KSPL : (slot - n_kp * KSPL) / VSPL;
    const int part = is_k ? slot % KSPL : (slot - n_kp * KSPL) % VSPL;
    int e = 0, h = 0, j0 = 0;
    const T *src = nullptr;
    int64_t stride = krow;
    bool is_v = false;
    float wc[VW], ws[VW];                        // e^{i SPL w_j}
    if (is_k) {
      e = task * VW;
      h = e / half;
      j0 = e % half;
      src = k + (int64_t)h * D + j0;
#pragma unroll
      for (int i = 0; i < VW; ++i) rope_phasor((double)KSPL, omega[j0 + i], &wc[i], &ws[i]);
    } else {
      is_v = task < n_v;
      e = (is_v ? task : task - n_v) * VW;
      stride = is_v ? krow : rrow;
      src = (is_v ? v : kr) + e;
    }

    int doc = 0;
    for (int64_t row = blockIdx.x; row < n_pool; row += gridDim.x) {
      // document of this row: rows only grow, so search upward from the last
      // one (always within [0, n_docs - 1], whatever the offsets hold)
      if (doc + 1 < n_docs && pool_off[doc + 1] <= row) {
        int lo = doc + 1, hi = n_docs - 1;       // last document whose first row is <= row
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (pool_off[mid] <= row) lo = mid; else hi = mid - 1;
        }
        doc = lo;
      }
      const int64_t c = row - pool_off[doc];
      int64_t t0 = tok_off[doc] + c * P;
      int64_t t1 = min(t0 + (int64_t)P, tok_off[doc + 1]);
      t0 = max((int64_t)0, min(t0, n_tokens));
      t1 = max(t0, min(t1, n_tokens));
      const int n = (int)(t1 - t0);
      const float inv_n = n > 0 ? 1.0f / (float)n : 0.0f;
      const T *base = src + t0 * stride;

      if (is_k) {
        const T *bhi = base + half;
        const double p0 = (double)c * (double)P;
        float alo[VW], ahi[VW], zc[VW], zs[VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) alo[i] = ahi[i] = 0.f;
        int u = part;
#pragma unroll
        for (int i = 0; i < VW; ++i) rope_phasor(p0 + (double)u, omega[j0 + i], &zc[i], &zs[i]);
        auto rotate_add = [&](const u32x4 &vl, const u32x4 &vh) {
          float xl[VW], xh[VW];
          Elt<T>::unpack(vl, xl);
          Elt<T>::unpack(vh, xh);
#pragma unroll
          for (int i = 0; i < VW; ++i) {
            alo[i] += xl[i] * zc[i] - xh[i] * zs[i];
            ahi[i] += xh[i] * zc[i] + xl[i] * zs[i];
            const float c2 = zc[i] * wc[i] - zs[i] * ws[i];
            zs[i] = zs[i] * wc[i] + zc[i] * ws[i];
            zc[i] = c2;
          }
          u += KSPL;
        };
        for (; u + (kUnroll - 1) * KSPL < n;) {
          u32x4 vl[kUnroll], vh[kUnroll];
#pragma unroll
          for (int q = 0; q < kUnroll; ++q) {
            vl[q] = ld16_nt(base + (int64_t)(u + q * KSPL) * krow);
            vh[q] = ld16_nt(bhi + (int64_t)(u + q * KSPL) * krow);
          }
#pragma unroll
          for (int q = 0; q < kUnroll; ++q) rotate_add(vl[q], vh[q]);
        }
        while (u < n) rotate_add(ld16_nt(base + (int64_t)u * krow), ld16_nt(bhi + (int64_t)u * krow));
#pragma unroll
        for (int o = 1; o < KSPL; o <<= 1)
#pragma unroll
          for (int i = 0; i < VW; ++i) {
            alo[i] += __shfl_xor(alo[i], o, 64);
            ahi[i] += __shfl_xor(ahi[i], o, 64);
          }
        if (part == 0) {
#pragma unroll
          for (int i = 0; i < VW; ++i) { alo[i] *= inv_n; ahi[i] *= inv_n; }
          T *out = kv_out + row * 2 * krow + (int64_t)h * D + j0;
          st16(out, Elt<T>::pack(alo));
          st16(out + half, Elt<T>::pack(ahi));
        }
      } else {
        // plain chunk mean of a V vector or a Kr vector
        float acc[VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[i] = 0.f;
        int u = part;
        for (; u + (kUnroll - 1) * VSPL < n; u += kUnroll * VSPL) {
          u32x4 vv[kUnroll];
#pragma unroll
          for (int q = 0; q < kUnroll; ++q) vv[q] = ld16_nt(base + (int64_t)(u + q * VSPL) * stride);
#pragma unroll
          for (int q = 0; q < kUnroll; ++q) {
            float x[VW];
            Elt<T>::unpack(vv[q], x);
#pragma unroll
            for (int i = 0; i < VW; ++i) acc[i] += x[i];
          }
        }
        for (; u < n; u += VSPL) {
          float x[VW];
          Elt<T>::unpack(ld16_nt(base + (int64_t)u * stride), x);
#pragma unroll
          for (int i = 0; i < VW; ++i) acc[i] += x[i];
        }
#pragma unroll
        for (int o = 1; o < VSPL; o <<= 1)
#pragma unroll
          for (int i = 0; i < VW; ++i) acc[i] += __shfl_xor(acc[i], o, 64);
        if (part == 0) {
#pragma unroll
          for (int i = 0; i < VW; ++i) acc[i] *= inv_n;
          // Kr goes to bank row R; in the tiled bank a 16-row tile stores its
          // rows' VW-element pieces piece-major
          const int64_t R = kr_row_base + row;
          T *out = is_v       ? kv_out + row * 2 * krow + krow + e
                   : kr_tiled ? kr_out + (R >> 4) * 16 * rrow + (16 * (e / VW) + (R & 15)) * VW
                              : kr_out + R * rrow + e;
          st16(out, Elt<T>::pack(acc));
        }
      }
    }
  }
}

template <typename T>
hipError_t launch_pool_t(const msa_pool_args &a, hipStream_t s) {
  constexpr int VW = Elt<T>::kPerVec;
  constexpr int KSPL = MSA_POOL_KSPLIT, VSPL = MSA_POOL_VSPLIT;
  const int half = a.head_dim / 2;
  const int n_slots = a.n_kv_heads * half / VW * KSPL +
                      (a.n_kv_heads * a.head_dim / VW + a.n_router_heads * a.router_dim / VW) * VSPL;
  int block = ((n_slots + 63) / 64) * 64;
  if (block > 512) block = 512;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, pool_kernel<T, KSPL, VSPL>, block, 0) != hipSuccess ||
      occ < 1)
    occ = 1;
  const int64_t want = (int64_t)device_info().n_cu * occ;
  const int grid = (int)(a.n_pool < want ? a.n_pool : want);
  hipLaunchKernelGGL((pool_kernel<T, KSPL, VSPL>), dim3(grid), dim3(block), 0, s,
                     reinterpret_cast<const T *>(a.k), reinterpret_cast<const T *>(a.v),
                     reinterpret_cast<const T *>(a.kr), a.doc_tok_off, a.doc_pool_off,
                     reinterpret_cast<T *>(a.kv_pooled), reinterpret_cast<T *>(a.kr_pooled), a.n_docs,
                     a.n_tokens, a.n_pool, a.pool_size, a.n_kv_heads, a.head_dim, a.n_router_heads,
                     a.router_dim, log2(a.rope_theta), a.kr_layout == MSA_KR_TILED ? 1 : 0, a.kr_row_base);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const msa_pool_args &a, hipStream_t s) {
  if (a.n_pool == 0) return hipSuccess;
  return a.dtype == MSA_BF16 ? launch_pool_t<uint16_t>(a, s) : launch_pool_t<float>(a, s);
}

}  // namespace msa
