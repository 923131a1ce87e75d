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
// - one workgroup per pooled row, grid-stride over rows so a fixed grid fills
//   the chip and amortises the per-workgroup RoPE table;
// - lane tasks are 16-byte vectors: a K task holds VW rotate-half pairs (the
//   VW elements at j0.. and their partners at j0+D/2..), V and Kr tasks hold
//   VW consecutive elements; every token row is read once, coalesced;
// - RoPE: the chunk's positions are p0 + u (p0 = c*P).  Splitting u into
//   64-token sub-blocks, sum_u R(p0+u) x_u = sum_blk R(p0+64 blk) *
//   sum_t R(t) x_{64 blk + t}; R(t) for t < 64 comes from an LDS table, and
//   R(p0 + 64 blk) is evaluated once per sub-block with the angle reduced in
//   fp64, so large in-document positions keep full fp32 accuracy.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kSub = 64;     // positions covered by the LDS phasor table
constexpr int kUnroll = 4;   // tokens in flight per lane (x2 loads for K tasks)

template <typename T>
__global__ __launch_bounds__(512) void pool_kernel(
    const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ kr,
    const int64_t *__restrict__ tok_off, const int64_t *__restrict__ pool_off,
    T *__restrict__ kv_out, T *__restrict__ kr_out, int n_docs, int64_t n_tokens, int64_t n_pool,
    int P, int Hkv, int D, int Hr, int dr, double log2_theta) {
  constexpr int VW = Elt<T>::kPerVec;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int half = D / 2;
  double *omega = reinterpret_cast<double *>(smem_raw);                 // [half]
  float *tab_c = reinterpret_cast<float *>(smem_raw + 8 * half);        // [kSub][half]
  float *tab_s = tab_c + kSub * half;

  for (int j = threadIdx.x; j < half; j += blockDim.x) omega[j] = exp2(-(2.0 * j / D) * log2_theta);
  __syncthreads();
  for (int i = threadIdx.x; i < kSub * half; i += blockDim.x) {
    float c, s;
    rope_phasor((double)(i / half), omega[i % half], &c, &s);
    tab_c[i] = c;
    tab_s[i] = s;
  }
  __syncthreads();

  const int n_kp = Hkv * half / VW;
  const int n_v = Hkv * D / VW;
  const int n_r = Hr * dr / VW;
  const int n_tasks = n_kp + n_v + n_r;
  const int64_t krow = (int64_t)Hkv * D;
  const int64_t rrow = (int64_t)Hr * dr;

  for (int64_t row = blockIdx.x; row < n_pool; row += gridDim.x) {
    int lo = 0, hi = n_docs - 1;  // last document whose first pooled row is <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pool_off[mid] <= row) lo = mid; else hi = mid - 1;
    }
    const int64_t c = row - pool_off[lo];
    int64_t t0 = tok_off[lo] + c * P;
    int64_t t1 = min(t0 + (int64_t)P, tok_off[lo + 1]);
    t0 = max((int64_t)0, min(t0, n_tokens));
    t1 = max(t0, min(t1, n_tokens));
    const int n = (int)(t1 - t0);
    const float inv_n = n > 0 ? 1.0f / (float)n : 0.0f;
    const double p0 = (double)c * (double)P;

    for (int task = threadIdx.x; task < n_tasks; task += blockDim.x) {
      if (task < n_kp) {
        const int e = task * VW;
        const int h = e / half, j0 = e % half;
        const T *blo = k + t0 * krow + (int64_t)h * D + j0;
        const T *bhi = blo + half;
        float tlo[VW], thi[VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) tlo[i] = thi[i] = 0.f;
        for (int u0 = 0; u0 < n; u0 += kSub) {
          const int ue = min(n, u0 + kSub);
          float slo[VW], shi[VW];
#pragma unroll
          for (int i = 0; i < VW; ++i) slo[i] = shi[i] = 0.f;
          int u = u0;
          for (; u + kUnroll <= ue; u += kUnroll) {
            u32x4 vl[kUnroll], vh[kUnroll];
#pragma unroll
            for (int q = 0; q < kUnroll; ++q) {
              vl[q] = ld16_nt(blo + (int64_t)(u + q) * krow);
              vh[q] = ld16_nt(bhi + (int64_t)(u + q) * krow);
            }
#pragma unroll
            for (int q = 0; q < kUnroll; ++q) {
              float xl[VW], xh[VW];
              Elt<T>::unpack(vl[q], xl);
              Elt<T>::unpack(vh[q], xh);
              const float *cc = tab_c + (u + q - u0) * half + j0;
              const float *ss = tab_s + (u + q - u0) * half + j0;
#pragma unroll
              for (int i = 0; i < VW; ++i) {
                slo[i] += xl[i] * cc[i] - xh[i] * ss[i];
                shi[i] += xh[i] * cc[i] + xl[i] * ss[i];
              }
            }
          }
          for (; u < ue; ++u) {
            float xl[VW], xh[VW];
            Elt<T>::unpack(ld16_nt(blo + (int64_t)u * krow), xl);
            Elt<T>::unpack(ld16_nt(bhi + (int64_t)u * krow), xh);
            const float *cc = tab_c + (u - u0) * half + j0;
            const float *ss = tab_s + (u - u0) * half + j0;
#pragma unroll
            for (int i = 0; i < VW; ++i) {
              slo[i] += xl[i] * cc[i] - xh[i] * ss[i];
              shi[i] += xh[i] * cc[i] + xl[i] * ss[i];
            }
          }
#pragma unroll
          for (int i = 0; i < VW; ++i) {
            float cb, sb;
            rope_phasor(p0 + (double)u0, omega[j0 + i], &cb, &sb);
            tlo[i] += slo[i] * cb - shi[i] * sb;
            thi[i] += shi[i] * cb + slo[i] * sb;
          }
        }
#pragma unroll
        for (int i = 0; i < VW; ++i) { tlo[i] *= inv_n; thi[i] *= inv_n; }
        T *out = kv_out + row * 2 * krow + (int64_t)h * D + j0;
        st16(out, Elt<T>::pack(tlo));
        st16(out + half, Elt<T>::pack(thi));
      } else {
        // plain chunk mean of a V vector or a Kr vector
        const bool is_v = task < n_kp + n_v;
        const int e = (is_v ? task - n_kp : task - n_kp - n_v) * VW;
        const int64_t stride = is_v ? krow : rrow;
        const T *base = (is_v ? v : kr) + t0 * stride + e;
        float acc[VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[i] = 0.f;
        int u = 0;
        for (; u + kUnroll <= n; u += kUnroll) {
          u32x4 vv[kUnroll];
#pragma unroll
          for (int q = 0; q < kUnroll; ++q) vv[q] = ld16_nt(base + (int64_t)(u + q) * stride);
#pragma unroll
          for (int q = 0; q < kUnroll; ++q) {
            float x[VW];
            Elt<T>::unpack(vv[q], x);
#pragma unroll
            for (int i = 0; i < VW; ++i) acc[i] += x[i];
          }
        }
        for (; u < n; ++u) {
          float x[VW];
          Elt<T>::unpack(ld16_nt(base + (int64_t)u * stride), x);
#pragma unroll
          for (int i = 0; i < VW; ++i) acc[i] += x[i];
        }
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[i] *= inv_n;
        T *out = is_v ? kv_out + row * 2 * krow + krow + e : kr_out + row * rrow + e;
        st16(out, Elt<T>::pack(acc));
      }
    }
  }
}

template <typename T>
hipError_t launch_pool_t(const msa_pool_args &a, hipStream_t s) {
  constexpr int VW = Elt<T>::kPerVec;
  const int half = a.head_dim / 2;
  const int n_tasks = a.n_kv_heads * half / VW + a.n_kv_heads * a.head_dim / VW +
                      a.n_router_heads * a.router_dim / VW;
  int block = ((n_tasks + 63) / 64) * 64;
  if (block > 512) block = 512;
  const int64_t want = (int64_t)device_info().n_cu * 8;
  const int grid = (int)(a.n_pool < want ? a.n_pool : want);
  const size_t smem = 8 * (size_t)half + 2 * sizeof(float) * kSub * (size_t)half;
  hipLaunchKernelGGL(pool_kernel<T>, dim3(grid), dim3(block), smem, s,
                     reinterpret_cast<const T *>(a.k), reinterpret_cast<const T *>(a.v),
                     reinterpret_cast<const T *>(a.kr), a.doc_tok_off, a.doc_pool_off,
                     reinterpret_cast<T *>(a.kv_pooled), reinterpret_cast<T *>(a.kr_pooled), a.n_docs,
                     a.n_tokens, a.n_pool, a.pool_size, a.n_kv_heads, a.head_dim, a.n_router_heads,
                     a.router_dim, log2(a.rope_theta));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const msa_pool_args &a, hipStream_t s) {
  if (a.n_pool == 0) return hipSuccess;
  return a.dtype == MSA_BF16 ? launch_pool_t<uint16_t>(a, s) : launch_pool_t<float>(a, s);
}

}  // namespace msa
