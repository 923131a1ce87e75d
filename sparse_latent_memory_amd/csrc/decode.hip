// Stage 3: one sparse decode-attention step over [pooled memory ; local K/V].
//
// Method: "EverMind-AI/MSA: Memory Sparse Attention for 100M-Token Contexts"
// (hysenlabs.com), section "How MSA compresses and routes documents" (the
// pooled K/V of the chosen documents come first and the query's own K/V
// after them; global RoPE moves the query start by k, keeping the order
// background -> query -> generation) and stage 3 of "EverMind Releases Memory-Sparse Attention Code
// for Long-Context AI Models" (toolmesh.ai), "Architectural Design and
// Inference".
//
// Split-KV design: grid (split, kv head, query).  Each workgroup owns a
// contiguous key range of one (query, KV head) and all Hq/Hkv query heads of
// that group (they share every staged K/V tile).  Per 64-key tile:
//   stage   K and V global loads are issued first (16 bytes per lane,
//           coalesced); the RoPE phasors of the local keys are computed while
//           they are in flight; local keys are rotated at o + i, memory keys
//           used as stored; both land in LDS in the storage type;
//   scores  wave w <-> query head, lane <-> key: dot(q', K[key]) from LDS;
//   softmax online, wave-wide max/sum, exp2 with log2(e) folded into q';
//   PV      wave w <-> query head, lane <-> D/64 output dims.
// Partials (m, l, unnormalised acc) go to the workspace; a merge kernel
// combines the splits with their log-sum-exp weights.
#include "msa_internal.h"

#include <algorithm>

namespace msa {
namespace {

constexpr int kTile = 64;
constexpr int kReseed = 16;    // tiles between exact RoPE phasor evaluations
constexpr int kMaxGroup = 8;   // query heads per KV head handled per workgroup
constexpr int kMaxSplit = 1024;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
// fp32 at D = 128 stages 66 KiB of K/V per workgroup in LDS: two fit on a CU
template <typename T, int D>
__global__ __launch_bounds__(256, (sizeof(T) == 4 && D == 128) ? 2 : 3) void decode_split_kernel(
    const T *__restrict__ q, const T *__restrict__ mem_kv, const int32_t *__restrict__ mem_len,
    const T *__restrict__ local_k, const T *__restrict__ local_v, const int32_t *__restrict__ local_len,
    const int32_t *__restrict__ pos_offset, float *__restrict__ part_acc, float *__restrict__ part_ml,
    int Hq, int Hkv, int mem_cap, int local_cap, int split_len, int n_split, float scale_log2,
    double log2_theta) {
  constexpr int VW = Elt<T>::kPerVec;     // elements per 16-byte vector
  constexpr int HALF = D / 2;
  constexpr int KSTR = D + VW;            // padded LDS row of K (conflict-free row reads)
  constexpr int DPL = D / 64;             // output dims per lane
  constexpr int KCH = HALF / VW;          // 16-byte pair-chunks per key
  constexpr int KTPT = kTile * KCH / 256; // K tasks per thread
  constexpr int KSTEP = 256 / KCH;        // key stride between a thread's K tasks
  constexpr int VCH = D / VW;             // 16-byte chunks per V row
  constexpr int VTPT = kTile * VCH / 256;
  constexpr int VSTEP = 256 / VCH;
  __shared__ __align__(16) T ks[kTile * KSTR];
  __shared__ __align__(16) T vs[kTile * D];
  __shared__ __align__(16) float qs[kMaxGroup * D];
  __shared__ float ps[kMaxGroup * kTile];
  __shared__ double omega[HALF];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int M = max(0, min(mem_len[b], mem_cap));
  const int Tl = max(0, min(local_len[b], local_cap));
  const int o = pos_offset[b];
  const int total = M + Tl;
  const int k0 = split * split_len;
  const int k1 = min(total, k0 + split_len);

  // output slots of this (query, split) for the G heads of the group
  auto slot = [&](int hh) { return ((int64_t)b * Hq + g * G + hh) * n_split + split; };

  if (k0 >= k1) {
    // an empty split: weight 0 in the merge, and finite zeros where the
    // merge reads its accumulator (0 times stale workspace contents could
    // be NaN)
    for (int hh = threadIdx.x; hh < G; hh += blockDim.x) {
      part_ml[2 * slot(hh)] = -INFINITY;
      part_ml[2 * slot(hh) + 1] = 0.f;
    }
    for (int i = threadIdx.x; i < G * D; i += blockDim.x) part_acc[slot(i / D) * D + i % D] = 0.f;
    return;
  }

  for (int j = threadIdx.x; j < HALF; j += blockDim.x) omega[j] = exp2(-(2.0 * j / D) * log2_theta);
  __syncthreads();
  // q' = RoPE(q, o + Tl - 1), with the softmax scale and log2(e) folded in
  for (int t = threadIdx.x; t < G * HALF; t += blockDim.x) {
    const int hh = t / HALF, j = t % HALF;
    const T *src = q + ((int64_t)b * Hq + g * G + hh) * D;
    const float x1 = Elt<T>::get(src, j), x2 = Elt<T>::get(src, j + HALF);
    float c, s;
    rope_phasor((double)o + (double)Tl - 1.0, omega[j], &c, &s);
    qs[hh * D + j] = (x1 * c - x2 * s) * scale_log2;
    qs[hh * D + j + HALF] = (x2 * c + x1 * s) * scale_log2;
  }

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  float acc[2][DPL];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[r][i] = 0.f;

  const int64_t mem_row = 2LL * Hkv * D;      // elements per pooled memory row
  const int64_t loc_row = (int64_t)Hkv * D;   // elements per local token

  // Thread t always owns the VW rotate-half pairs cj.. of the keys
  // kk0 + j*KSTEP of every tile, so the RoPE phasor of each (key, pair)
  // advances by e^{i 64 omega} from one tile to the next: it is evaluated
  // exactly (fp64 angle reduction) once every kReseed tiles and carried by
  // complex multiplication in between.
  const int cj = (threadIdx.x % KCH) * VW, kk0 = threadIdx.x / KCH;
  const int vj = (threadIdx.x % VCH) * VW, vk0 = threadIdx.x / VCH;
  float zc[KTPT][VW], zs[KTPT][VW], wc[VW], ws[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) rope_phasor((double)kTile, omega[cj + e], &wc[e], &ws[e]);

  for (int kt = k0, tile = 0; kt < k1; kt += kTile, ++tile) {
    const int nk = min(kTile, k1 - kt);
    // ---- issue this tile's global loads ----
    u32x4 kl[KTPT], kh[KTPT], vv[VTPT];
#pragma unroll
    for (int j = 0; j < KTPT; ++j) {
      const int kk = kk0 + j * KSTEP, key = kt + kk;
      if (kk < nk) {
        const T *src = key < M ? mem_kv + ((int64_t)b * mem_cap + key) * mem_row + (int64_t)g * D
                               : local_k + ((int64_t)b * local_cap + (key - M)) * loc_row + (int64_t)g * D;
        kl[j] = ld16(src + cj);
        kh[j] = ld16(src + cj + HALF);
      }
    }
#pragma unroll
    for (int j = 0; j < VTPT; ++j) {
      const int kk = vk0 + j * VSTEP, key = kt + kk;
      if (kk < nk) {
        const T *src = key < M ? mem_kv + ((int64_t)b * mem_cap + key) * mem_row + loc_row + (int64_t)g * D
                               : local_v + ((int64_t)b * local_cap + (key - M)) * loc_row + (int64_t)g * D;
        vv[j] = ld16(src + vj);
      }
    }
    // ---- phasors while the loads are in flight ----
    if (tile % kReseed == 0) {
#pragma unroll
      for (int j = 0; j < KTPT; ++j)
#pragma unroll
        for (int e = 0; e < VW; ++e)
          rope_phasor((double)o - M + kt + kk0 + j * KSTEP, omega[cj + e], &zc[j][e], &zs[j][e]);
    } else {
#pragma unroll
      for (int j = 0; j < KTPT; ++j)
#pragma unroll
        for (int e = 0; e < VW; ++e) {
          const float c = zc[j][e] * wc[e] - zs[j][e] * ws[e];
          zs[j][e] = zs[j][e] * wc[e] + zc[j][e] * ws[e];
          zc[j][e] = c;
        }
    }
    __syncthreads();  // previous tile fully consumed (and qs written on the first pass)
    // ---- K (rotated when local) and V into LDS ----
#pragma unroll
    for (int j = 0; j < KTPT; ++j) {
      const int kk = kk0 + j * KSTEP, key = kt + kk;
      u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (kk < nk) {
        lo = kl[j];
        hi = kh[j];
        if (key >= M) {
          float xl[VW], xh[VW], rl[VW], rh[VW];
          Elt<T>::unpack(lo, xl);
          Elt<T>::unpack(hi, xh);
#pragma unroll
          for (int e = 0; e < VW; ++e) {
            rl[e] = xl[e] * zc[j][e] - xh[e] * zs[j][e];
            rh[e] = xh[e] * zc[j][e] + xl[e] * zs[j][e];
          }
          lo = Elt<T>::pack(rl);
          hi = Elt<T>::pack(rh);
        }
      }
      st16(ks + kk * KSTR + cj, lo);
      st16(ks + kk * KSTR + cj + HALF, hi);
    }
#pragma unroll
    for (int j = 0; j < VTPT; ++j) {
      const int kk = vk0 + j * VSTEP;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (kk < nk) x = vv[j];
      st16(vs + kk * D + vj, x);
    }
    __syncthreads();

    // ---- scores, online softmax, PV: wave <-> query head ----
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int hh = wave + 4 * r;
      if (hh >= G) break;
      float logit = -INFINITY;
      if (lane < nk) {
        const T *kr = ks + lane * KSTR;
        const float *qr = qs + hh * D;
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < D; i += VW) {
          float x[VW];
          Elt<T>::unpack(*reinterpret_cast<const u32x4 *>(kr + i), x);
#pragma unroll
          for (int e = 0; e < VW; e += 2) {
            a0 += qr[i + e] * x[e];
            a1 += qr[i + e + 1] * x[e + 1];
          }
        }
        logit = a0 + a1;
      }
      const float m_tile = wave_max(logit);
      const float m_new = fmaxf(m_run[r], m_tile);
      const float p = lane < nk ? exp2f(logit - m_new) : 0.f;
      const float corr = exp2f(m_run[r] - m_new);   // 0 on the first tile (m_run = -inf)
      l_run[r] = l_run[r] * corr + wave_sum(p);
      m_run[r] = m_new;
      ps[hh * kTile + lane] = p;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[r][i] *= corr;
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      const float *pr = ps + hh * kTile;
      for (int kk = 0; kk < nk; ++kk) {
        const float w = pr[kk];
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[r][i] += w * Elt<T>::get(vs + kk * D, lane * DPL + i);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int hh = wave + 4 * r;
    if (hh >= G) break;
    const int64_t sl = slot(hh);
    float *dst = part_acc + sl * D + lane * DPL;
#pragma unroll
    for (int i = 0; i < DPL; ++i) dst[i] = acc[r][i];
    if (lane == 0) {
      part_ml[2 * sl] = m_run[r];
      part_ml[2 * sl + 1] = l_run[r];
    }
  }
}

// Combine the splits of one (query, head).  Wave 0 forms the weights
// 2^(m_s - max m) in LDS and their l-weighted sum; then every thread owns a
// float4 of the output and a stride of splits, with all its loads issued
// before the adds.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float *__restrict__ part_acc,
                                                          const float *__restrict__ part_ml, T *__restrict__ out,
                                                          float *__restrict__ lse, int n_split) {
  constexpr int NV = D / 4;               // float4 per output row
  constexpr int NGRP = 256 / NV;          // split groups
  __shared__ float w[kMaxSplit];
  __shared__ float s_m, s_l;
  __shared__ float4 part[NGRP][NV];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const float *ml = part_ml + bh * n_split * 2;
  if (tid < 64) {
    float m = -INFINITY;
    for (int s = tid; s < n_split; s += 64) m = fmaxf(m, ml[2 * s]);
    m = wave_max(m);
    float l = 0.f;
    for (int s = tid; s < n_split; s += 64) {
      const float ms = ml[2 * s];
      const float ws = (ms == -INFINITY) ? 0.f : exp2f(ms - m);
      w[s] = ws;
      l += ws * ml[2 * s + 1];
    }
    l = wave_sum(l);
    if (tid == 0) { s_m = m; s_l = l; }
  }
  __syncthreads();
  const int v = tid % NV, grp = tid / NV;
  const float4 *pa = reinterpret_cast<const float4 *>(part_acc + bh * n_split * D) + v;
  float4 a = {0.f, 0.f, 0.f, 0.f};
  int s = grp;
  for (; s + 3 * NGRP < n_split; s += 4 * NGRP) {
    float4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = pa[(int64_t)(s + u * NGRP) * NV];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float ws = w[s + u * NGRP];
      a.x += ws * x[u].x; a.y += ws * x[u].y; a.z += ws * x[u].z; a.w += ws * x[u].w;
    }
  }
  for (; s < n_split; s += NGRP) {
    const float ws = w[s];
    const float4 x = pa[(int64_t)s * NV];
    a.x += ws * x.x; a.y += ws * x.y; a.z += ws * x.z; a.w += ws * x.w;
  }
  part[grp][v] = a;
  __syncthreads();
  const float L = s_l;
  if (tid < NV) {
    float4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g2 = 0; g2 < NGRP; ++g2) {
      r.x += part[g2][tid].x; r.y += part[g2][tid].y; r.z += part[g2][tid].z; r.w += part[g2][tid].w;
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    Elt<T>::put(out, bh * D + 4 * tid + 0, r.x * inv);
    Elt<T>::put(out, bh * D + 4 * tid + 1, r.y * inv);
    Elt<T>::put(out, bh * D + 4 * tid + 2, r.z * inv);
    Elt<T>::put(out, bh * D + 4 * tid + 3, r.w * inv);
  }
  if (lse && tid == 0) lse[bh] = L > 0.f ? (s_m + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// Keys per split: enough splits that batch * Hkv * n_split workgroups fill the
// chip, in whole 64-key tiles.
int choose_split_len(int32_t batch, int32_t mem_cap, int32_t local_cap) {
  const int64_t total = (int64_t)mem_cap + local_cap;
  int64_t len = (total * batch + 255) / 256;
  len = ((len + kTile - 1) / kTile) * kTile;
  if (len < kTile) len = kTile;
  return (int)len;
}

template <typename T, int D>
hipError_t launch_t(const msa_decode_args &a, float *part_acc, float *part_ml, int32_t n_split, hipStream_t s) {
  const int split_len = choose_split_len(a.batch, a.mem_cap, a.local_cap);
  const float scale = a.softmax_scale > 0.f ? a.softmax_scale : 1.0f / sqrtf((float)a.head_dim);
  hipError_t e = hipSuccess;
  if (n_split > kMaxSplit) return hipErrorInvalidValue;
  hipExtLaunchKernelGGL((decode_split_kernel<T, D>), dim3(n_split, a.n_kv_heads, a.batch), dim3(256), 0, s,
                        prof_event(a.prof_event_begin), prof_event(a.prof_event_end), 0,
                        reinterpret_cast<const T *>(a.q), reinterpret_cast<const T *>(a.mem_kv), a.mem_len,
                        reinterpret_cast<const T *>(a.local_k), reinterpret_cast<const T *>(a.local_v),
                        a.local_len, a.pos_offset, part_acc, part_ml, a.n_q_heads, a.n_kv_heads, a.mem_cap,
                        a.local_cap, split_len, n_split, scale * kLog2e, log2(a.rope_theta));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(a.batch * a.n_q_heads), dim3(256), 0, s, part_acc,
                     part_ml, reinterpret_cast<T *>(a.out), a.lse, n_split);
  return hipGetLastError();
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t decode_ws_layout(int32_t batch, int32_t hq, int32_t d, int32_t mem_cap, int32_t local_cap, void *base,
                        float **part_acc, float **part_ml, int32_t *n_split) {
  const int split_len = choose_split_len(batch, mem_cap, local_cap);
  const int64_t total = (int64_t)mem_cap + local_cap;
  const int32_t ns = (int32_t)std::max<int64_t>(1, (total + split_len - 1) / split_len);
  const size_t slots = (size_t)batch * hq * ns;
  const size_t o_acc = 0;
  const size_t o_ml = align256(sizeof(float) * slots * d);
  const size_t end = align256(o_ml + sizeof(float) * 2 * slots);
  if (base) {
    *part_acc = reinterpret_cast<float *>(reinterpret_cast<char *>(base) + o_acc);
    *part_ml = reinterpret_cast<float *>(reinterpret_cast<char *>(base) + o_ml);
  }
  if (n_split) *n_split = ns;
  return end;
}

hipError_t launch_decode(const msa_decode_args &a, float *part_acc, float *part_ml, int32_t n_split,
                         hipStream_t s) {
  if (a.dtype != MSA_F32) return hipErrorInvalidValue;   // bf16 runs the block-attention kernel
  return a.head_dim == 128 ? launch_t<float, 128>(a, part_acc, part_ml, n_split, s)
                           : launch_t<float, 64>(a, part_acc, part_ml, n_split, s);
}

}  // namespace msa
