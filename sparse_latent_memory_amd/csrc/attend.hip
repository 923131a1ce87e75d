// Stage 3 for a block of query tokens: attention of Tq query tokens (the last
// Tq tokens of each local context) over [pooled memory ; causal local K/V],
// with global RoPE.  Tq = 1 is the decode step.
//
// Method: "EverMind-AI/MSA: Memory Sparse Attention for 100M-Token Contexts"
// (hysenlabs.com), section "How MSA compresses and routes documents" (the
// pooled K/V of the chosen documents come first and the query's own K/V
// after them; global RoPE moves the query start by k, keeping the order
// background -> query -> generation); stage 3 of "EverMind Releases
// Memory-Sparse Attention Code for Long-Context AI Models" (toolmesh.ai),
// "Architectural Design and Inference".  The block form (token t of the
// block is local token T - Tq + t and sees local tokens up to itself) is
// this library's reading.
//
// Work item = one wave: (query b, KV head g, 16-row query tile, key split).
// Rows of a tile are (token, head) pairs of one KV group, row = t*G + hh.
// Per 16-key group:
//   K   loaded straight from HBM in the MFMA A-operand layout (lane l: key
//       l%16, dims 32s + 8(l/16) .. +8); local keys rotated in registers -
//       the rotate-half partner of dim j < D/2 is in the same lane (block
//       s + D/64), so RoPE needs no data exchange.  The phasor of (key, j)
//       is one exact evaluation per 64-key block and pair (one per lane),
//       times a table entry e^{i c w_j} for the key's offset c < 16;
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with the rotated, scaled query
//       split into bf16 head + remainder (two MFMAs per k-block);
//       lane l then holds S[row l%16][keys 4(l/16) .. +4], which is exactly
//       the A-operand layout of v_mfma_f32_16x16x16bf16_1k, so P feeds the
//       PV product without any exchange;
//   online softmax per row (exp2, log2(e) folded into q);
//   V   loaded as 4 keys x D/16 dims per lane, written transposed into a
//       per-wave LDS tile and read back as B-operands of the PV MFMAs.
// The next group's K/V loads are issued before the current group is
// computed.  Partials (m, l, acc) per (slot, row) go to the workspace; a
// merge kernel combines the splits.  No barrier follows the one-time table
// setup.
#include "msa_internal.h"

#include <algorithm>
#include <type_traits>

namespace msa {
namespace {

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int kAWaves = 4;          // independent work items per workgroup
constexpr int kAMaxSplit = 4096;
#ifndef MSA_ATT_SPLIT_MAX   // longest key split, a multiple of 64
#define MSA_ATT_SPLIT_MAX 512
#endif
// Work items run KV head fastest, so the Hkv waves of one key range read
// whole K/V rows together, and each query walks its splits from a different
// start.  With split-fastest order and no rotation, capacities whose row
// strides are multiples of large powers of two (4096 local tokens, 12288
// memory rows) made concurrent waves collide in the memory system: 613 us
// against 313 us for the same 64 x 4696 keys.
#ifndef MSA_ATT_ORDER       // work item order: 0 split fastest, 1 KV head fastest
#define MSA_ATT_ORDER 1
#endif
#ifndef MSA_ATT_PREROT      // 1: rotate local keys once when several query tiles read them
#define MSA_ATT_PREROT 1
#endif
#ifndef MSA_ATT_WAVES_PER_CU   // work items (waves) per CU the key splits aim for
#define MSA_ATT_WAVES_PER_CU 16
#endif
#ifndef MSA_ATT_BLOCK       // 1: prefill (>= 4 query tiles per KV head) shares key groups across a workgroup
#define MSA_ATT_BLOCK 1
#endif
#ifndef MSA_ATT_MERGE_WAVE  // 1: merge with one wave per output row when there are at most 64 splits
#define MSA_ATT_MERGE_WAVE 1
#endif
#ifndef MSA_ATT_ROTATE      // 1: rotate each query's split order by its index
#define MSA_ATT_ROTATE 1
#endif
#ifndef MSA_ATT_BLOCK_QLO   // 1: the block kernel keeps the query's bf16 remainder term (two MFMAs per k-block)
#define MSA_ATT_BLOCK_QLO 1
#endif
#ifndef MSA_ATT_BLOCK_NWMAX // largest number of query tiles (waves) per block-kernel workgroup: 4, 8 or 16
#define MSA_ATT_BLOCK_NWMAX 16
#endif
#ifndef MSA_ATT_BLOCK_WAVES // waves per CU (4 SIMDs) the block kernel's register budget aims for
#define MSA_ATT_BLOCK_WAVES 8
#endif
constexpr float kALog2e = 1.4426950408889634f;
constexpr float kALazy = 8.f;   // block kernel: raise the running max only past this margin (log2 units)

template <int D>
struct AttnCfg {
  static constexpr int KS = D / 32;   // 32-wide k-blocks of Q K^T
  static constexpr int HS = KS / 2;   // k-blocks of the first rotate-half
  static constexpr int NT = D / 16;   // 16-wide output column tiles
  static constexpr int DB = D / 16;   // dims per lane in V staging
  static constexpr int VTS = 16 + 4;  // LDS row (16 keys + pad) of the transposed V group, in bf16
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float amax4(const f32x4 &v) { return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])); }

// bf16 number e (0..7) of a 16-byte vector
__device__ __forceinline__ uint32_t bf16_at(const u32x4 &v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}
__device__ __forceinline__ uint32_t bf16_at(const u32x2 &v, int e) {
  const uint32_t w = e < 2 ? v.x : v.y;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// PREROT: the local keys come already rotated to their positions (o + i)
// and the query rotated and scaled (rot_q, fp32), from rope_prepass_kernel;
// the kernel then rotates nothing.
template <int D, bool PREROT>
__global__ __launch_bounds__(kAWaves * 64, 2) void attend_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ mem_kv, const int32_t *__restrict__ mem_len,
    const uint16_t *__restrict__ local_k, const uint16_t *__restrict__ local_v,
    const int32_t *__restrict__ local_len, const int32_t *__restrict__ pos_offset, float *__restrict__ part_acc,
    float *__restrict__ part_ml, int B, int Tq, int Hq, int Hkv, int mem_cap, int local_cap, int n_mt, int n_split,
    int split_len, int rps, float scale_log2, double log2_theta, const float *__restrict__ rot_q) {
  using C = AttnCfg<D>;
  constexpr int KS = C::KS, HS = C::HS, NT = C::NT, DB = C::DB, VTS = C::VTS, HALF = D / 2;
  using VVec = typename std::conditional<DB == 8, u32x4, u32x2>::type;
  __shared__ double omega[HALF];
  __shared__ float2 step16[HALF];                          // e^{i 16 omega_j}
  // rows padded so that the 16 key columns (F) and the 4 lane groups (zb)
  // of one read fall in different LDS banks
  constexpr int FS = HALF + 1;                             // F row stride
  constexpr int ZS = HALF + HALF / 16;                     // zb row stride, entry j at j + j/16
  __shared__ float2 ftab[16 * FS];                         // e^{i c omega_j}, c < 16
  __shared__ float2 zb_all[kAWaves][4 * ZS];               // per wave: block phasors
  __shared__ __align__(16) uint16_t vt_all[kAWaves][D * VTS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  int g, split_i, mt, b;
  bool live;
  if (n_mt > 1) {
    // Several query tiles per KV head read the same keys: workgroup w serves
    // KV head w % Hkv only.  Workgroups go round-robin over the 8 XCDs, so an
    // XCD's L2 holds the keys of one head (Hkv = 8), or of a few, instead of
    // all of them.  Its waves take consecutive (query, tile, split) items of
    // that head.
    g = (int)(blockIdx.x % Hkv);
    int64_t r = (int64_t)(blockIdx.x / Hkv) * kAWaves + wave;
    live = r < (int64_t)B * n_mt * n_split;
    if (!live) r = 0;                                      // decoded but never written
    split_i = (int)(r % n_split);
    r /= n_split;
    mt = (int)(r % n_mt);
    b = (int)(r / n_mt);
  } else {
    int64_t item = (int64_t)blockIdx.x * kAWaves + wave;
    live = item < (int64_t)B * Hkv * n_mt * n_split;
    if (!live) item = 0;                                   // decoded but never written
#if MSA_ATT_ORDER == 1
    // KV head fastest: the Hkv waves of one key range read whole K/V rows together
    g = (int)(item % Hkv);
    item /= Hkv;
    split_i = (int)(item % n_split);
    item /= n_split;
    mt = (int)(item % n_mt);
    b = (int)(item / n_mt);
#else
    split_i = (int)(item % n_split);
    item /= n_split;
    mt = (int)(item % n_mt);
    item /= n_mt;
    g = (int)(item % Hkv);
    b = (int)(item / Hkv);
#endif
  }
#if MSA_ATT_ROTATE
  const int split = (int)((split_i + 5LL * b) % n_split);  // queries walk their key ranges out of step
#else
  const int split = split_i;
#endif
  const int G = Hq / Hkv;
  uint16_t *vt = vt_all[wave];
  float2 *zb = zb_all[wave];

  const int M = max(0, min(mem_len[b], mem_cap));
  const int T = max(0, min(local_len[b], local_cap));
  const int o = pos_offset[b];
  const int n_rows = Tq * G;
  const int col = lane & 15, grp = lane >> 4;
  // this lane's query row in the S layout and in the Q fragments
  const int R = mt * 16 + col;
  const bool row_ok = R < n_rows;
  const int t_row = row_ok ? R / G : 0;
  const int i_row = T - Tq + t_row;                        // local index of the row's token
  const int i_first = T - Tq + (mt * 16) / G;              // ... of the tile's first token
  // keys the tile can see: the memory, then local tokens up to its last token
  const int t_last = min(Tq - 1, (mt * 16 + 15) / G);
  const int key_end = M + max(0, min(T, T - Tq + t_last + 1));
  const int k_begin = split * split_len;
  const int k_end = min(key_end, k_begin + split_len);
  const int64_t slot = (((int64_t)b * Hkv + g) * n_mt + mt) * n_split + split;
  const bool active = live && k_begin < k_end;

  // RoPE tables, only in workgroups with work (every thread reaches both
  // barriers): w_j, e^{i c w_j} for c < 16 by products of e^{i w_j}, and
  // e^{i 16 w_j}
  if (__syncthreads_or(active)) {
    if (threadIdx.x < HALF) {
      const int j = threadIdx.x;
      const double w = exp2(-(2.0 * j / D) * log2_theta);
      omega[j] = w;
      float c1, s1;
      rope_phasor(1.0, w, &c1, &s1);
      float2 z = make_float2(1.f, 0.f);
      for (int c = 0; c < 16; ++c) {
        ftab[c * FS + j] = z;
        z = make_float2(z.x * c1 - z.y * s1, z.y * c1 + z.x * s1);
      }
      step16[j] = z;
    }
    __syncthreads();
  }
  if (!live) return;                                       // no barrier follows

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (active) {
    // ---- rotated, scaled query as B-operand fragments (hi + lo bf16) ----
    u32x4 qhi[KS], qlo[KS];
    {
      float x[KS][8];
      const int64_t qrow = ((int64_t)b * Tq + t_row) * Hq + g * G + (row_ok ? R % G : 0);
      if (PREROT) {
        const float4 *src = reinterpret_cast<const float4 *>(rot_q + qrow * D + 8 * grp);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const float4 u = row_ok ? src[8 * s] : float4{0.f, 0.f, 0.f, 0.f};
          const float4 w = row_ok ? src[8 * s + 1] : float4{0.f, 0.f, 0.f, 0.f};
          x[s][0] = u.x; x[s][1] = u.y; x[s][2] = u.z; x[s][3] = u.w;
          x[s][4] = w.x; x[s][5] = w.y; x[s][6] = w.z; x[s][7] = w.w;
        }
      } else {
        const uint16_t *src = q + qrow * D + 8 * grp;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4 v = row_ok ? ld16(src + 32 * s) : u32x4{0u, 0u, 0u, 0u};
          float f[8];
          Elt<uint16_t>::unpack(v, f);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[s][e] = f[e];
        }
#pragma unroll
        for (int s = 0; s < HS; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float c, sn;
            rope_phasor((double)o + (double)i_row, omega[32 * s + 8 * grp + e], &c, &sn);
            const float x1 = x[s][e], x2 = x[s + HS][e];
            x[s][e] = (x1 * c - x2 * sn) * scale_log2;
            x[s + HS][e] = (x2 * c + x1 * sn) * scale_log2;
          }
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        float hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          hi[e] = bf16_to_f32(f32_to_bf16(x[s][e]));
          lo[e] = x[s][e] - hi[e];
        }
        qhi[s] = Elt<uint16_t>::pack(hi);
        qlo[s] = Elt<uint16_t>::pack(lo);
      }
    }

    // Key k lives in memory row k (k < M) or local row k - M; its K and V
    // are selected branch-free: element offset base + k * stride in the
    // array of its kind (one 32 x 32 -> 64-bit multiply-add per key).
    const uint32_t mrow = 2u * Hkv * D, lrow = (uint32_t)Hkv * D;
    const int64_t mem_base = (int64_t)b * mem_cap * mrow + (int64_t)g * D;
    const int64_t loc_base = ((int64_t)b * local_cap - M) * lrow + (int64_t)g * D;   // + k * lrow for k >= M
    auto key_ptrs = [&](int k, const uint16_t *&kp, const uint16_t *&vp) {
      const bool mem = k < M;
      const int64_t off = (mem ? mem_base : loc_base) + (int64_t)((uint64_t)(uint32_t)k * (mem ? mrow : lrow));
      kp = (mem ? mem_kv : local_k) + off;
      vp = (mem ? mem_kv + lrow : local_v) + off;
    };
    // loads of the 16-key group at kb (keys past k_end read key k_end - 1;
    // their scores are masked)
    const int kq = lane & 3, db = lane >> 2;                // V staging: keys 4kq.., dims db*DB..
    auto load = [&](int kb, u32x4 *kf, VVec *vv) {
      const bool inside = kb + 15 < k_end;                  // (uniform) no clamping needed
      const uint16_t *kp, *vp;
      key_ptrs(inside ? kb + col : min(kb + col, k_end - 1), kp, vp);
      kp += 8 * grp;
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[s] = ld16(kp + 32 * s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kv = kb + 4 * kq + i;
        key_ptrs(inside ? kv : min(kv, k_end - 1), kp, vp);
        vv[i] = *reinterpret_cast<const VVec *>(vp + db * DB);
      }
    };

    // RoPE of local keys.  Lane l holds key kb + col and the pairs
    // j = 32 s + 8 grp + e (s < HS); its phasor e^{i (o + key - M) w_j} is
    // zb[gi][j] * F[col][j], where zb[gi][j] = e^{i (o + kb0 - M + 16 gi) w_j}
    // is evaluated exactly once per 64-key block (one pair per lane) and
    // F[col][j] = e^{i col w_j} is a per-workgroup table.
    auto block_phasors = [&](int kb0) {
      if (lane < HALF) {
        float c, sn;
        rope_phasor((double)o + (double)(kb0 - M), omega[lane], &c, &sn);
        float2 z = make_float2(c, sn);
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          zb[gi * ZS + lane + (lane >> 4)] = z;
          const float2 w = step16[lane];
          z = make_float2(z.x * w.x - z.y * w.y, z.y * w.x + z.x * w.y);
        }
      }
    };
    auto rotate = [&](int gi, int kb, u32x4 *kf) {
      if (kb + col < M) return;                             // memory keys are used as stored
#pragma unroll
      for (int s = 0; s < HS; ++s) {
        float a[8], c2[8], r1[8], r2[8];
        Elt<uint16_t>::unpack(kf[s], a);
        Elt<uint16_t>::unpack(kf[s + HS], c2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 32 * s + 8 * grp + e;
          const float2 zz = zb[gi * ZS + j + (j >> 4)], ff = ftab[col * FS + j];
          const float zc = zz.x * ff.x - zz.y * ff.y, zs = zz.y * ff.x + zz.x * ff.y;
          r1[e] = a[e] * zc - c2[e] * zs;
          r2[e] = c2[e] * zc + a[e] * zs;
        }
        kf[s] = Elt<uint16_t>::pack(r1);
        kf[s + HS] = Elt<uint16_t>::pack(r2);
      }
    };
    // one 16-key group: rotation, S^T = K Q^T, online softmax, V transposed
    // through LDS, O += P V
    auto group = [&](int gi, int kb, u32x4 *kf, const VVec *vv) {
      if (!PREROT && kb + 15 >= M) rotate(gi, kb, kf);
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kv8 = __builtin_bit_cast(bf16x8, kf[s]);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv8, __builtin_bit_cast(bf16x8, qhi[s]), sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv8, __builtin_bit_cast(bf16x8, qlo[s]), sc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < DB; ++e) {
        u32x2 w;
        w.x = bf16_at(vv[0], e) | (bf16_at(vv[1], e) << 16);
        w.y = bf16_at(vv[2], e) | (bf16_at(vv[3], e) << 16);
        *reinterpret_cast<u32x2 *>(vt + (db * DB + e) * VTS + 4 * kq) = w;
      }
      // mask: row must exist, key in range, local keys up to the row's token;
      // not needed when every key of the group is in range and visible to
      // the tile's first token (rows that do not exist are never stored)
      if (!(kb + 15 < k_end && kb + 15 - M <= i_first)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb + 4 * grp + r;
          const bool ok = row_ok && key < k_end && (key < M || key - M <= i_row);
          sc[r] = ok ? sc[r] : -INFINITY;
        }
      }
      float mt_ = amax4(sc);
      mt_ = fmaxf(mt_, __shfl_xor(mt_, 16, 64));
      mt_ = fmaxf(mt_, __shfl_xor(mt_, 32, 64));
      const float m_new = fmaxf(m_run, mt_);
      const bool none = m_new == -INFINITY;
      const float corr = none ? 1.f : exp2f(m_run - m_new);
      float psum = 0.f;
      s16x4 pa;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = none ? 0.f : exp2f(sc[r] - m_new);
        psum += pr;
        pa[r] = (short)f32_to_bf16(pr);
      }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      l_run = l_run * corr + psum;
      // rows 4 grp + r of the accumulators take the factor of their row,
      // which is exactly 1 unless the row's running max rose
      if (__any(m_new > m_run)) {
        float cr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * grp + r, 64);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[nt][r] *= cr[r];
      }
      m_run = m_new;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const u32x2 vb = *reinterpret_cast<const u32x2 *>(vt + (16 * nt + col) * VTS + 4 * grp);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_bit_cast(s16x4, vb), acc[nt], 0, 0, 0);
      }
    };

    u32x4 kfa[KS], kfb[KS];
    VVec vva[4], vvb[4];
    load(k_begin, kfa, vva);
    for (int ks0 = k_begin; ks0 < k_end; ks0 += 64) {
      if (!PREROT && ks0 + 63 >= M) block_phasors(ks0);
      // four groups, buffers alternating; the last one loads the next block's first
      load(ks0 + 16, kfb, vvb);
      group(0, ks0, kfa, vva);
      load(ks0 + 32, kfa, vva);
      group(1, ks0 + 16, kfb, vvb);
      load(ks0 + 48, kfb, vvb);
      group(2, ks0 + 32, kfa, vva);
      load(ks0 + 64, kfa, vva);
      group(3, ks0 + 48, kfb, vvb);
    }
  }

  // ---- partials: (m, l) from the S layout, acc from the O layout ----
  if (grp == 0 && col < rps && row_ok) {
    part_ml[2 * (slot * rps + col)] = m_run;
    part_ml[2 * (slot * rps + col) + 1] = l_run;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * grp + r;
    if (row < rps && mt * 16 + row < n_rows) {
      float *dst = part_acc + (slot * rps + row) * D + col;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) dst[16 * nt] = acc[nt][r];
    }
  }
}

// Block form for launches with at least four 16-row query tiles per KV head
// (prefill): a workgroup of NW waves takes NW consecutive tiles of one
// (query, KV head, key split), one tile per wave, and shares every 64-key
// group, which the workgroup stages once in LDS - K row-major in padded rows
// (a wave's A-operand reads of 16 rows hit 64 distinct banks), V transposed
// per 32-key half with its keys in the order of the score layout, so that a
// lane's V^T operand is one 16-byte read - double buffered, one barrier per
// group.  A group is taken in two 32-key halves: S^T = K Q^T for two
// quarters, the online softmax over the half's 8 scores per lane (column
// maxima over four lanes by lane swaps) and O^T += V^T P^T on
// v_mfma_f32_16x16x32_bf16 with the two quarters as one 32-key step: P^T is
// the softmax's output as it stands, and O^T keeps each query in one lane
// column, so the rescale needs no exchange.  The running max is raised only
// when a half's max exceeds it by more than kALazy (log2 units): the weights
// then stay below 2^kALazy, and the result is the same function of the
// scores (the merge and the normaliser use the max that was kept).  Local
// keys and the query come rotated (rope_prepass_kernel), so nothing is
// rotated here.
// Scores, masking and the partials are those of attend_kernel, with the
// tile's own causal key range: quarters past it are skipped, and a wave
// whose tile lies past the last one loads and synchronises but stores
// nothing.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, MSA_ATT_BLOCK_WAVES / 4 > 0 ? MSA_ATT_BLOCK_WAVES / 4 : 1) void attend_block_kernel(
    const uint16_t *__restrict__ mem_kv, const int32_t *__restrict__ mem_len, const uint16_t *__restrict__ local_k,
    const uint16_t *__restrict__ local_v, const int32_t *__restrict__ local_len, float *__restrict__ part_acc,
    float *__restrict__ part_ml, int B, int Tq, int Hq, int Hkv, int mem_cap, int local_cap, int n_mt, int n_split,
    int split_len, int rps, const float *__restrict__ rot_q) {
  using C = AttnCfg<D>;
  constexpr int KS = C::KS, NT = C::NT;
  constexpr int KG = 64;                                   // keys per group: four 16-key quarters, two halves
  constexpr int KRS = D + 8;                               // K row stride in LDS (bf16)
  constexpr int VRS = 32 + 8;                              // V^T row (one dim, a half's 32 keys + pad), bf16
  constexpr int NTH = NW * 64;
  constexpr int KPN = KG * (D / 8), VPN = (KG / 4) * (D / 2);   // 16-byte K pieces, (4 keys x 2 dims) V pieces
  constexpr int KPT = (KPN + NTH - 1) / NTH, VPT = (VPN + NTH - 1) / NTH;   // per thread per group
  static_assert(KPN % NTH == 0 || KPN < NTH, "K pieces: whole rounds, or one partial round");
  static_assert(VPN % NTH == 0 || VPN < NTH, "V pieces: whole rounds, or one partial round");
  __shared__ __align__(16) uint16_t ks[2][KG * KRS];
  // per half: [dim][slot], key 32 h + 16 jj + 4 q + r of the group in slot
  // 8 q + 4 jj + r - the k-slot that lane group q gives it in P^T
  __shared__ __align__(16) uint16_t vt[2][2][D * VRS];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // work item of the workgroup: (query, NW-tile group, split) of KV head g
  const int n_tg = (n_mt + NW - 1) / NW;
  const int g = (int)(blockIdx.x % Hkv);
  int64_t r = (int64_t)(blockIdx.x / Hkv);
  if (r >= (int64_t)B * n_tg * n_split) return;           // the whole workgroup: no barrier is left waiting
  const int split_i = (int)(r % n_split);
  r /= n_split;
  const int tgi = (int)(r % n_tg);
  const int b = (int)(r / n_tg);
#if MSA_ATT_ROTATE
  const int split = (int)((split_i + 5LL * b) % n_split);
#else
  const int split = split_i;
#endif
  const int G = Hq / Hkv;
  const int M = max(0, min(mem_len[b], mem_cap));
  const int T = max(0, min(local_len[b], local_cap));
  const int n_rows = Tq * G;
  const int col = lane & 15, grp = lane >> 4;
  // keys a tile sees: the memory, then local tokens up to its last token
  auto key_end_of = [&](int tile) {
    const int t_last = min(Tq - 1, (tile * 16 + 15) / G);
    return M + max(0, min(T, T - Tq + t_last + 1));
  };
  const int k_begin = split * split_len;
  const int k_end_g = min(key_end_of(min(NW * tgi + NW - 1, n_mt - 1)), k_begin + split_len);   // the workgroup's
  const int mt = NW * tgi + wave;                          // this wave's tile
  const bool tile_ok = mt < n_mt;
  const int R = mt * 16 + col;
  const bool row_ok = tile_ok && R < n_rows;
  const int i_row = T - Tq + (row_ok ? R / G : 0);         // the row's token, as a local index
  const int i_first = T - Tq + (mt * 16) / G;              // the tile's first token
  const int k_end = tile_ok ? min(key_end_of(mt), k_begin + split_len) : k_begin;
  // keys below k_full are seen by every row of the tile: memory, and local
  // keys up to the tile's first token
  const int k_full = min(k_end, M + max(0, i_first + 1));

  // Cooperative loads of the 64-key group at kb (keys past the workgroup's
  // range read its last key; every wave masks them).  K piece p of this
  // thread: key (tid + p NTH) / (D/8), 16-byte chunk (tid + p NTH) % (D/8);
  // V piece p: keys 4 qd .. +3 and dims 2 dp, 2 dp + 1 of
  // (qd, dp) = ((tid + p NTH) / (D/2), (tid + p NTH) % (D/2)).
  const uint32_t mrow = 2u * Hkv * D, lrow = (uint32_t)Hkv * D;
  const uint16_t *mem_b = mem_kv + (int64_t)b * mem_cap * mrow + (int64_t)g * D;
  const uint16_t *lk_b = local_k + (int64_t)b * local_cap * lrow + (int64_t)g * D;
  const uint16_t *lv_b = local_v + (int64_t)b * local_cap * lrow + (int64_t)g * D;
  auto key_k = [&](int k) -> const uint16_t * {
    return k < M ? mem_b + (int64_t)k * mrow : lk_b + (int64_t)(k - M) * lrow;
  };
  auto key_v = [&](int k) -> const uint16_t * {
    return k < M ? mem_b + (int64_t)k * mrow + lrow : lv_b + (int64_t)(k - M) * lrow;
  };
  u32x4 kreg[KPT];
  uint32_t vreg[VPT][4];
  auto gload = [&](int kb) {
    const bool in_mem = kb + KG <= M, in_loc = kb >= M;   // (uniform)
    if (kb + KG <= k_end_g && (in_mem || in_loc)) {
      // the whole group in one array and in range: one base (scalar), one
      // row stride, 32-bit byte offsets per lane
      const uint32_t stride = in_mem ? mrow : lrow;
      const char *kbase = reinterpret_cast<const char *>(in_mem ? mem_b + (int64_t)kb * mrow
                                                                : lk_b + (int64_t)(kb - M) * lrow);
      const char *vbase = reinterpret_cast<const char *>(in_mem ? mem_b + (int64_t)kb * mrow + lrow
                                                                : lv_b + (int64_t)(kb - M) * lrow);
#pragma unroll
      for (int p = 0; p < KPT; ++p) {
        const int i = tid + p * NTH;
        if (KPN >= NTH || i < KPN)
          kreg[p] = ld16(kbase + 2u * ((uint32_t)(i / (D / 8)) * stride + 8u * (uint32_t)(i % (D / 8))));
      }
#pragma unroll
      for (int p = 0; p < VPT; ++p) {
        const int i = tid + p * NTH, qd = i / (D / 2), dp = i % (D / 2);
        if (VPN >= NTH || i < VPN) {
          const uint32_t off = 2u * ((uint32_t)(4 * qd) * stride + 2u * (uint32_t)dp);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            vreg[p][e] = *reinterpret_cast<const uint32_t *>(vbase + (size_t)(2u * e * stride) + off);
        }
      }
      return;
    }
    // a group across the boundary or past the range (keys past it read the last one)
#pragma unroll
    for (int p = 0; p < KPT; ++p) {
      const int i = tid + p * NTH;
      if (KPN >= NTH || i < KPN) kreg[p] = ld16(key_k(min(kb + i / (D / 8), k_end_g - 1)) + 8 * (i % (D / 8)));
    }
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
      const int i = tid + p * NTH, qd = i / (D / 2), dp = i % (D / 2);
      if (VPN >= NTH || i < VPN) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vreg[p][e] = *reinterpret_cast<const uint32_t *>(key_v(min(kb + 4 * qd + e, k_end_g - 1)) + 2 * dp);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KPT; ++p) {
      const int i = tid + p * NTH;
      if (KPN >= NTH || i < KPN) st16(&ks[buf][(i / (D / 8)) * KRS + 8 * (i % (D / 8))], kreg[p]);
    }
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
      const int i = tid + p * NTH, qd = i / (D / 2), dp = i % (D / 2);
      if (VPN < NTH && i >= VPN) continue;
      // keys 4 qd .. 4 qd + 3: half qd / 8, slots from 8 (qd % 4) + 4 ((qd / 4) % 2)
      const int hv = qd >> 3, sb = 8 * (qd & 3) + 4 * ((qd >> 2) & 1);
      u32x2 lo, hi;                                        // dims 2dp and 2dp+1 of the four keys
      lo.x = (vreg[p][0] & 0xffffu) | (vreg[p][1] << 16);
      lo.y = (vreg[p][2] & 0xffffu) | (vreg[p][3] << 16);
      hi.x = (vreg[p][0] >> 16) | (vreg[p][1] & 0xffff0000u);
      hi.y = (vreg[p][2] >> 16) | (vreg[p][3] & 0xffff0000u);
      *reinterpret_cast<u32x2 *>(&vt[buf][hv][(2 * dp) * VRS + sb]) = lo;
      *reinterpret_cast<u32x2 *>(&vt[buf][hv][(2 * dp + 1) * VRS + sb]) = hi;
    }
  };

  float m_run = -INFINITY, l_run = 0.f;                    // l_run: this lane's part of the sum
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 qhi[KS], qlo[KS];
  int buf = 0;

  // S^T for quarter j of the staged group
  auto s_quarter = [&](int j, f32x4 &sc) {
    sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kv8 = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4 *>(&ks[buf][(16 * j + col) * KRS + 32 * s + 8 * grp]));
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv8, __builtin_bit_cast(bf16x8, qhi[s]), sc, 0, 0, 0);
      if (MSA_ATT_BLOCK_QLO)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv8, __builtin_bit_cast(bf16x8, qlo[s]), sc, 0, 0, 0);
    }
  };
  // online softmax of a half's 8 scores per lane: raises the running max if
  // due (the factor for the accumulators in corr; raise: some lane must
  // apply it) and returns P^T for the half
  auto softmax = [&](const f32x4 &s0, const f32x4 &s1, float &corr, bool &raise) -> u32x4 {
    const float mx = col_max4(fmaxf(amax4(s0), amax4(s1)));
    raise = mx > m_run + kALazy;                           // (true for the first finite score)
    corr = raise ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;   // (0 while nothing was seen)
    m_run = raise ? mx : m_run;
    l_run *= corr;
    // scores -inf (masked) weigh 0, also while no score was finite
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float pr[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = __builtin_amdgcn_exp2f((i < 4 ? s0[i] : s1[i - 4]) - m_use);
      psum += pr[i];
    }
    l_run += psum;
    return u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]), pack_bf16x2(pr[4], pr[5]),
                 pack_bf16x2(pr[6], pr[7])};
  };
  // the accumulators hold O^T: this lane's column is its query, so the
  // factor is the lane's own (exactly 1 where the max was kept)
  auto rescale = [&](float corr, bool raise) {
    if (__any(raise)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[nt][rr] *= corr;
    }
  };
  // O^T += V^T P^T for half h: k-slot 8 grp + i is key 4 grp + i of quarter
  // 2h (i < 4) or of quarter 2h + 1 (i >= 4), for V^T and P^T alike (a
  // quarter past the tile's keys has weights 0 and finite staged values)
  auto pv = [&](int h, const u32x4 &pp) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const bf16x8 vv = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4 *>(&vt[buf][h][(16 * nt + col) * VRS + 8 * grp]));
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, __builtin_bit_cast(bf16x8, pp), acc[nt], 0, 0, 0);
    }
  };
  // mask: keys out of the tile's range, local keys after the row's token
  auto mask = [&](int kj, f32x4 &sc) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int key = kj + 4 * grp + rr;
      const bool ok = row_ok && key < k_end && (key < M || key - M <= i_row);
      sc[rr] = ok ? sc[rr] : -INFINITY;
    }
  };

  if (k_begin < k_end_g) {                                 // (uniform over the workgroup)
    gload(k_begin);
    // the query rows (rotated and scaled by the pre-pass, fp32) as B-operand
    // fragments (hi + lo bf16); the loads overlap the first group's
    {
      const float4 *src = reinterpret_cast<const float4 *>(
          rot_q + (((int64_t)b * Tq + (row_ok ? R / G : 0)) * Hq + g * G + (row_ok ? R % G : 0)) * D + 8 * grp);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const float4 x0 = src[8 * s], x1 = src[8 * s + 1];
        const float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        float hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = row_ok ? f[e] : 0.f;
          hi[e] = bf16_to_f32(f32_to_bf16(x));
          lo[e] = x - hi[e];
        }
        qhi[s] = Elt<uint16_t>::pack(hi);
        qlo[s] = Elt<uint16_t>::pack(lo);
      }
    }
    lstore(0);
    __syncthreads();                                       // the first group in place
    for (int kb = k_begin; kb < k_end_g; kb += KG) {
      const bool more = kb + KG < k_end_g;                 // (uniform)
      if (more) gload(kb + KG);
      // quarters of this group the tile sees (keys kb + 16 j .. below k_end)
      const int nq = min(4, max(0, (k_end - kb + 15) >> 4));   // (uniform over the wave)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (2 * h >= nq) continue;                        // (uniform) no key of this half is seen
        f32x4 sc[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int j = 2 * h + jj;
          if (j < nq) {
            s_quarter(j, sc[jj]);
            if (!(kb + 16 * j + 15 < k_full)) mask(kb + 16 * j, sc[jj]);
          } else {
            sc[jj] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
          }
        }
        float corr;
        bool raise;
        const u32x4 pp = softmax(sc[0], sc[1], corr, raise);
        rescale(corr, raise);
        pv(h, pp);
      }
      if (more) lstore(buf ^ 1);
      __syncthreads();                                     // next group in place; this one free
      buf ^= 1;
    }
  }

  // ---- partials: lane (col, grp) holds query row col of the tile: its
  // (m, l) and dims 16 nt + 4 grp .. + 3 of its accumulator ----
  if (!tile_ok) return;
  const float l = col_sum4(l_run);
  const int64_t slot = (((int64_t)b * Hkv + g) * n_mt + mt) * n_split + split;
  if (col < rps && row_ok) {
    if (grp == 0) *reinterpret_cast<float2 *>(part_ml + 2 * (slot * rps + col)) = float2{m_run, l};
    float *dst = part_acc + (slot * rps + col) * D + 4 * grp;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<float4 *>(dst + 16 * nt) = float4{acc[nt][0], acc[nt][1], acc[nt][2], acc[nt][3]};
  }
}

// The pre-pass of launches in which several query tiles per KV head read
// every key (prefill): the local keys rotated once to their positions o + i
// (i < local_len), and the query block rotated to its tokens' positions
// o + T - Tq + t and scaled (scale * log2 e, as the kernels use it) into
// fp32, so the attention kernels rotate nothing.  Thread per (row, 8 pairs):
// key rows first, then query rows; each phasor is evaluated exactly (angle
// reduced in fp64), the frequencies come from a per-workgroup table.
template <int D>
__global__ __launch_bounds__(256) void rope_prepass_kernel(const uint16_t *__restrict__ local_k,
                                                           const uint16_t *__restrict__ q,
                                                           const int32_t *__restrict__ local_len,
                                                           const int32_t *__restrict__ pos_offset,
                                                           uint16_t *__restrict__ rot_k, float *__restrict__ rot_q,
                                                           int B, int Tq, int Hq, int Hkv, int local_cap,
                                                           float scale_log2, double log2_theta) {
  constexpr int HALF = D / 2, NC = HALF / 8;              // 8-pair chunks per head
  __shared__ double omega[HALF];
  if (threadIdx.x < HALF) omega[threadIdx.x] = exp2(-(2.0 * threadIdx.x / D) * log2_theta);
  __syncthreads();
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_k = (int64_t)B * local_cap * Hkv * NC;
  const int64_t n_q = (int64_t)B * Tq * Hq * NC;
  if (id >= n_k + n_q) return;
  const bool key = id < n_k;
  const int64_t idx = key ? id : id - n_k;
  const int c = (int)(idx % NC);
  const int64_t row = idx / NC;                            // key: (b * local_cap + i) * Hkv + g; query: (b * Tq + t) * Hq + h
  const int64_t bt = row / (key ? Hkv : Hq);
  const int b = (int)(bt / (key ? local_cap : Tq)), it = (int)(bt % (key ? local_cap : Tq));
  const int T = max(0, min(local_len[b], local_cap));
  if (key && it >= T) return;                              // never read
  const double pos = (double)pos_offset[b] + (double)(key ? it : T - Tq + it);
  const uint16_t *src = (key ? local_k : q) + row * D + 8 * c;
  float a[8], z[8], r1[8], r2[8];
  Elt<uint16_t>::unpack(ld16(src), a);
  Elt<uint16_t>::unpack(ld16(src + HALF), z);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float cs, sn;
    rope_phasor(pos, omega[8 * c + e], &cs, &sn);
    r1[e] = a[e] * cs - z[e] * sn;
    r2[e] = z[e] * cs + a[e] * sn;
  }
  if (key) {
    uint16_t *dst = rot_k + row * D + 8 * c;
    st16(dst, Elt<uint16_t>::pack(r1));
    st16(dst + HALF, Elt<uint16_t>::pack(r2));
  } else {
    float4 *dst = reinterpret_cast<float4 *>(rot_q + row * D + 8 * c);
    dst[0] = make_float4(r1[0] * scale_log2, r1[1] * scale_log2, r1[2] * scale_log2, r1[3] * scale_log2);
    dst[1] = make_float4(r1[4] * scale_log2, r1[5] * scale_log2, r1[6] * scale_log2, r1[7] * scale_log2);
    dst += HALF / 4;
    dst[0] = make_float4(r2[0] * scale_log2, r2[1] * scale_log2, r2[2] * scale_log2, r2[3] * scale_log2);
    dst[1] = make_float4(r2[4] * scale_log2, r2[5] * scale_log2, r2[6] * scale_log2, r2[7] * scale_log2);
  }
}

// Combine the splits of one output row (b, t, h).  Wave 0 forms the
// weights 2^(m_s - max m) in LDS and their l-weighted sum; then every thread
// owns a float4 of the row and a stride of splits, with its loads issued
// before the adds.
template <int D>
__global__ __launch_bounds__(256) void attend_merge_kernel(const float *__restrict__ part_acc,
                                                          const float *__restrict__ part_ml, uint16_t *__restrict__ out,
                                                          float *__restrict__ lse, int Tq, int Hq, int Hkv, int n_mt,
                                                          int n_split, int rps) {
  constexpr int NV = D / 4;               // float4 per output row
  constexpr int NGRP = 256 / NV;          // split groups
  __shared__ float w[kAMaxSplit];
  __shared__ float s_m, s_l;
  __shared__ float4 part[NGRP][NV];
  const int64_t bth = blockIdx.x;                          // (b * Tq + t) * Hq + h
  const int h = (int)(bth % Hq);
  const int t = (int)((bth / Hq) % Tq);
  const int b = (int)(bth / ((int64_t)Hq * Tq));
  const int G = Hq / Hkv, g = h / G;
  const int R = t * G + (h % G);
  const int mt = R / 16, row = R % 16;
  const int64_t base = ((((int64_t)b * Hkv + g) * n_mt + mt) * n_split) * rps + row;   // split s: base + s * rps
  const int tid = threadIdx.x;
  if (tid < 64) {
    float m = -INFINITY;
    for (int s = tid; s < n_split; s += 64) m = fmaxf(m, part_ml[2 * (base + (int64_t)s * rps)]);
    m = wave_max(m);
    float l = 0.f;
    for (int s = tid; s < n_split; s += 64) {
      const int64_t i = base + (int64_t)s * rps;
      const float ms = part_ml[2 * i];
      const float ws = ms == -INFINITY ? 0.f : exp2f(ms - m);
      w[s] = ws;
      l += ws * part_ml[2 * i + 1];
    }
    l = wave_sum(l);
    if (tid == 0) { s_m = m; s_l = l; }
  }
  __syncthreads();
  const int v = tid % NV, gq = tid / NV;
  float4 a = {0.f, 0.f, 0.f, 0.f};
  int s = gq;
  for (; s + 3 * NGRP < n_split; s += 4 * NGRP) {
    float4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      x[u] = reinterpret_cast<const float4 *>(part_acc + (base + (int64_t)(s + u * NGRP) * rps) * D)[v];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float ws = w[s + u * NGRP];
      a.x += ws * x[u].x; a.y += ws * x[u].y; a.z += ws * x[u].z; a.w += ws * x[u].w;
    }
  }
  for (; s < n_split; s += NGRP) {
    const float ws = w[s];
    const float4 x = reinterpret_cast<const float4 *>(part_acc + (base + (int64_t)s * rps) * D)[v];
    a.x += ws * x.x; a.y += ws * x.y; a.z += ws * x.z; a.w += ws * x.w;
  }
  part[gq][v] = a;
  __syncthreads();
  if (tid < NV) {
    float4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q2 = 0; q2 < NGRP; ++q2) {
      r.x += part[q2][tid].x; r.y += part[q2][tid].y; r.z += part[q2][tid].z; r.w += part[q2][tid].w;
    }
    const float L = s_l;
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    uint16_t *o = out + bth * D + 4 * tid;
    *reinterpret_cast<uint2 *>(o) = make_uint2(pack_bf16x2(r.x * inv, r.y * inv), pack_bf16x2(r.z * inv, r.w * inv));
  }
  if (lse && tid == 0) lse[bth] = s_l > 0.f ? (s_m + log2f(s_l)) * 0.69314718055994531f : -INFINITY;
}

// The same combination with one wave per output row and kAWaves rows per
// workgroup, for at most 64 splits: lane s holds split s's weight, and the
// lanes (v, gq) = (lane % NV, lane / NV) own float4 v of the row over splits
// gq, gq + 64/NV, ...; a butterfly over gq completes the sum.
template <int D>
__global__ __launch_bounds__(kAWaves * 64) void attend_merge_wave_kernel(
    const float *__restrict__ part_acc, const float *__restrict__ part_ml, uint16_t *__restrict__ out,
    float *__restrict__ lse, int64_t n_out, int Tq, int Hq, int Hkv, int n_mt, int n_split, int rps) {
  constexpr int NV = D / 4, SG = 64 / NV;
  const int lane = threadIdx.x & 63;
  const int64_t bth = (int64_t)blockIdx.x * kAWaves + (threadIdx.x >> 6);  // (b * Tq + t) * Hq + h
  if (bth >= n_out) return;                                // no barrier in this kernel
  const int h = (int)(bth % Hq);
  const int t = (int)((bth / Hq) % Tq);
  const int b = (int)(bth / ((int64_t)Hq * Tq));
  const int G = Hq / Hkv, g = h / G;
  const int R = t * G + (h % G);
  const int mt = R / 16, row = R % 16;
  const int64_t base = ((((int64_t)b * Hkv + g) * n_mt + mt) * n_split) * rps + row;   // split s: base + s * rps
  float ms = -INFINITY, ls = 0.f;
  if (lane < n_split) {
    const float2 ml = *reinterpret_cast<const float2 *>(part_ml + 2 * (base + (int64_t)lane * rps));
    ms = ml.x;
    ls = ml.y;
  }
  const float m = wave_max(ms);
  const float ws = ms == -INFINITY ? 0.f : exp2f(ms - m);
  const float l = wave_sum(ws * ls);
  const int v = lane % NV, gq = lane / NV;
  float4 a = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_split; s0 += 4 * SG) {
    float4 x[4];
    float w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sp = s0 + u * SG + gq;
      w[u] = __shfl(ws, sp & 63, 64);
      x[u] = sp < n_split ? reinterpret_cast<const float4 *>(part_acc + (base + (int64_t)sp * rps) * D)[v]
                          : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a.x += w[u] * x[u].x; a.y += w[u] * x[u].y; a.z += w[u] * x[u].z; a.w += w[u] * x[u].w;
    }
  }
#pragma unroll
  for (int o = NV; o < 64; o <<= 1) {
    a.x += __shfl_xor(a.x, o, 64); a.y += __shfl_xor(a.y, o, 64);
    a.z += __shfl_xor(a.z, o, 64); a.w += __shfl_xor(a.w, o, 64);
  }
  if (gq == 0) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    *reinterpret_cast<uint2 *>(out + bth * D + 4 * v) =
        make_uint2(pack_bf16x2(a.x * inv, a.y * inv), pack_bf16x2(a.z * inv, a.w * inv));
  }
  if (lse && lane == 0) lse[bth] = l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

// Waves (query tiles) per workgroup of the block kernel: as many as there
// are tiles per KV head, up to 16.
static int block_waves(int n_mt) {
  return n_mt >= 16 && MSA_ATT_BLOCK_NWMAX >= 16 ? 16 : n_mt >= 8 && MSA_ATT_BLOCK_NWMAX >= 8 ? 8 : 4;
}

// Keys per split: enough work items (waves) to give every CU about 16, in
// whole 64-key blocks, between 64 and 512 keys.  Sized from the capacities,
// which the host knows; splits past a tile's visible keys exit at once.  The
// block kernel (prefill) counts its workgroups of NW tiles instead and cuts
// the keys into whole 16-key quarters, so that the workgroups fill the CUs.
void attend_plan(int32_t batch, int32_t q_tokens, int32_t hq, int32_t hkv, int32_t mem_cap, int32_t local_cap,
                 AttendPlan *p) {
  const int G = hq / hkv;
  p->n_mt = (q_tokens * G + 15) / 16;
  p->rps = std::min(16, q_tokens * G);
  const int64_t total = std::max<int64_t>(1, (int64_t)mem_cap + local_cap);
  const int64_t want = (int64_t)device_info().n_cu * MSA_ATT_WAVES_PER_CU;
  if (MSA_ATT_PREROT && MSA_ATT_BLOCK && p->n_mt >= 4) {
    const int nw = block_waves(p->n_mt);
    const int64_t wgs = (int64_t)batch * hkv * ((p->n_mt + nw - 1) / nw);   // workgroups per split
    // as many waves as the CUs hold at the kernel's register budget
    const int64_t want_b = (int64_t)device_info().n_cu * std::max(nw, MSA_ATT_BLOCK_WAVES);
    const int64_t ns0 = std::max<int64_t>(1, std::min<int64_t>(kAMaxSplit, want_b / (wgs * nw)));
    int64_t len = ((total + ns0 - 1) / ns0 + 15) / 16 * 16;
    len = std::max<int64_t>(64, std::min<int64_t>(MSA_ATT_SPLIT_MAX, len));
    p->split_len = (int)len;
    p->n_split = (int)std::min<int64_t>(kAMaxSplit, (total + len - 1) / len);
    return;
  }
  const int64_t tiles = (int64_t)batch * hkv * p->n_mt;
  int64_t len = (total * tiles + want - 1) / want;
  len = std::max<int64_t>(64, std::min<int64_t>(MSA_ATT_SPLIT_MAX, ((len + 63) / 64) * 64));
  int64_t ns = (total + len - 1) / len;
  if (ns > kAMaxSplit) {
    ns = kAMaxSplit;
    len = ((total + ns - 1) / ns + 63) / 64 * 64;
    ns = (total + len - 1) / len;
  }
  p->split_len = (int)len;
  p->n_split = (int)ns;
}

size_t attend_ws_layout(int32_t batch, int32_t q_tokens, int32_t hq, int32_t hkv, int32_t d, int32_t mem_cap,
                        int32_t local_cap, void *base, AttendWs *ws) {
  AttendPlan p;
  attend_plan(batch, q_tokens, hq, hkv, mem_cap, local_cap, &p);
  const size_t rows = (size_t)batch * hkv * p.n_mt * p.n_split * p.rps;
  const size_t o_ml = (sizeof(float) * rows * d + 255) & ~(size_t)255;
  const size_t o_rk = (o_ml + sizeof(float) * 2 * rows + 255) & ~(size_t)255;
  // several query tiles per KV head read every local key: rotate the keys
  // (bf16) and the query block (fp32) once
  const bool prerot = p.n_mt > 1;
  const size_t o_rq = (o_rk + sizeof(uint16_t) * (size_t)batch * local_cap * hkv * d + 255) & ~(size_t)255;
  const size_t end = prerot ? (o_rq + sizeof(float) * (size_t)batch * q_tokens * hq * d + 255) & ~(size_t)255 : o_rk;
  if (base) {
    ws->part_acc = reinterpret_cast<float *>(base);
    ws->part_ml = reinterpret_cast<float *>(reinterpret_cast<char *>(base) + o_ml);
    ws->rot_k = prerot ? reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(base) + o_rk) : nullptr;
    ws->rot_q = prerot ? reinterpret_cast<float *>(reinterpret_cast<char *>(base) + o_rq) : nullptr;
  }
  return end;
}

template <int D, int NW>
static hipError_t launch_block(const msa_attend_args &a, const AttendPlan &p, const AttendWs &ws, const uint16_t *lk,
                               hipStream_t s) {
  const int64_t n_wg = (int64_t)a.n_kv_heads * a.batch * ((p.n_mt + NW - 1) / NW) * p.n_split;
  if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
  hipExtLaunchKernelGGL((attend_block_kernel<D, NW>), dim3((unsigned)n_wg), dim3(NW * 64), 0, s,
                        prof_event(a.prof_event_begin), prof_event(a.prof_event_end), 0,
                        reinterpret_cast<const uint16_t *>(a.mem_kv), a.mem_len, lk,
                        reinterpret_cast<const uint16_t *>(a.local_v), a.local_len, ws.part_acc, ws.part_ml, a.batch,
                        a.q_tokens, a.n_q_heads, a.n_kv_heads, a.mem_cap, a.local_cap, p.n_mt, p.n_split,
                        p.split_len, p.rps, ws.rot_q);
  return hipGetLastError();
}

template <int D, bool PREROT>
static hipError_t launch_attend_t(const msa_attend_args &a, const AttendWs &ws, hipStream_t s) {
  AttendPlan p;
  attend_plan(a.batch, a.q_tokens, a.n_q_heads, a.n_kv_heads, a.mem_cap, a.local_cap, &p);
  const float scale = a.softmax_scale > 0.f ? a.softmax_scale : 1.0f / sqrtf((float)D);
  // one KV head per workgroup when several tiles share its keys (see the kernel)
  const int64_t per_head = (int64_t)a.batch * p.n_mt * p.n_split;
  const int64_t grid = p.n_mt > 1 ? (int64_t)a.n_kv_heads * ((per_head + kAWaves - 1) / kAWaves)
                                  : (per_head * a.n_kv_heads + kAWaves - 1) / kAWaves;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  const uint16_t *lk = reinterpret_cast<const uint16_t *>(a.local_k);
  if (PREROT) {
    const int64_t n = ((int64_t)a.batch * a.local_cap * a.n_kv_heads + (int64_t)a.batch * a.q_tokens * a.n_q_heads) *
                      (D / 16);
    hipLaunchKernelGGL((rope_prepass_kernel<D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, lk,
                       reinterpret_cast<const uint16_t *>(a.q), a.local_len, a.pos_offset, ws.rot_k, ws.rot_q,
                       a.batch, a.q_tokens, a.n_q_heads, a.n_kv_heads, lk ? a.local_cap : 0, scale * kALog2e,
                       log2(a.rope_theta));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (lk) lk = ws.rot_k;
  }
  if (PREROT && MSA_ATT_BLOCK && p.n_mt >= 4) {
    // as many query tiles per workgroup as there are, up to 16
    const int nw = block_waves(p.n_mt);
    e = nw == 16 ? launch_block<D, 16>(a, p, ws, lk, s)
        : nw == 8 ? launch_block<D, 8>(a, p, ws, lk, s)
                  : launch_block<D, 4>(a, p, ws, lk, s);
    if (e != hipSuccess) return e;
  } else {
    hipExtLaunchKernelGGL((attend_kernel<D, PREROT>), dim3((unsigned)grid), dim3(kAWaves * 64), 0, s,
                          prof_event(a.prof_event_begin), prof_event(a.prof_event_end), 0,
                          reinterpret_cast<const uint16_t *>(a.q), reinterpret_cast<const uint16_t *>(a.mem_kv),
                          a.mem_len, lk, reinterpret_cast<const uint16_t *>(a.local_v), a.local_len, a.pos_offset,
                          ws.part_acc, ws.part_ml, a.batch, a.q_tokens, a.n_q_heads, a.n_kv_heads, a.mem_cap,
                          a.local_cap, p.n_mt, p.n_split, p.split_len, p.rps, scale * kALog2e, log2(a.rope_theta),
                          ws.rot_q);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t rows = (int64_t)a.batch * a.q_tokens * a.n_q_heads;
  if (MSA_ATT_MERGE_WAVE && p.n_split <= 64)
    hipLaunchKernelGGL((attend_merge_wave_kernel<D>), dim3((unsigned)((rows + kAWaves - 1) / kAWaves)),
                       dim3(kAWaves * 64), 0, s, ws.part_acc, ws.part_ml, reinterpret_cast<uint16_t *>(a.out), a.lse,
                       rows, a.q_tokens, a.n_q_heads, a.n_kv_heads, p.n_mt, p.n_split, p.rps);
  else
    hipLaunchKernelGGL((attend_merge_kernel<D>), dim3((unsigned)rows), dim3(256), 0, s, ws.part_acc, ws.part_ml,
                       reinterpret_cast<uint16_t *>(a.out), a.lse, a.q_tokens, a.n_q_heads, a.n_kv_heads, p.n_mt,
                       p.n_split, p.rps);
  return hipGetLastError();
}

hipError_t launch_attend(const msa_attend_args &a, const AttendWs &ws, hipStream_t s) {
  const bool pre = ws.rot_k != nullptr && MSA_ATT_PREROT;
  if (a.head_dim == 128)
    return pre ? launch_attend_t<128, true>(a, ws, s) : launch_attend_t<128, false>(a, ws, s);
  return pre ? launch_attend_t<64, true>(a, ws, s) : launch_attend_t<64, false>(a, ws, s);
}

}  // namespace msa
