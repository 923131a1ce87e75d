// Routing, stage 2 of the method: the bank scan for at most 8 bf16 query
// tokens (decode-time routing, one or a few queries).
//
// Method: "EverMind-AI/MSA: Memory Sparse Attention for 100M-Token Contexts"
// (hysenlabs.com), section "How MSA compresses and routes documents": the
// score of a pooled row is the cosine of the routing query and the pooled
// router key, averaged over router heads and maximised over query tokens.
//
// The bank is streamed once from HBM, one 16-row tile per wave step.  Every
// workgroup first builds the normalised query as MFMA A-fragments in LDS:
// each token is split into a bf16 head and a bf16 remainder row, so the
// query keeps ~16 mantissa bits.  v_mfma_f32_16x16x32_bf16 then computes the
// query dot products and the 16x16 Gram matrix of the tile (A = B = bank
// fragment), whose diagonal is every row's squared norm per head, so no
// cross-lane reduction runs on the VALU.  Output: row_score[b, j] = max over
// query b's tokens.
#include "msa_internal.h"

#include <algorithm>

namespace msa {
namespace {

constexpr int kWaves = 4;   // waves per workgroup

// --------------------------------------------------------------------------
// bf16 MFMA scan with the query preparation fused in
// --------------------------------------------------------------------------
// A-fragment f = h*KS + s, lane l holds A[row = l%16][k = 32 s + 8 (l/16) + e]
// (e < 8) of head h.  Row 2m is the bf16 rounding of unit query token m, row
// 2m+1 the bf16 rounding of its remainder; rows of absent tokens are zero.
// Lane l owns bank row (tile*16 + l%16) and the same k slice.  In the
// row-major bank one load instruction of the wave reads 16 rows x 64
// contiguous bytes; in the tiled bank (16-byte pieces of a 16-row tile
// stored piece-major) fragment f of the tile is the contiguous 1 KiB at
// 1024 f, lane l's 16 bytes at 16 l, and the loads are non-temporal: a
// streaming read of that order runs ~10% faster than of the row order.
// Heads are loaded in groups of HG, one group ahead of the MFMAs that
// consume them.
#ifndef MSA_SCAN_HG
#define MSA_SCAN_HG 1
#endif
#ifndef MSA_SCAN_PIPE      // 1: keep the head-group loop rolled (fewer registers)
#define MSA_SCAN_PIPE 0
#endif
#ifndef MSA_SCAN_NT        // 1: non-temporal bank loads (the bank is read once per call)
#define MSA_SCAN_NT 0
#endif
#ifndef MSA_SCAN_BUF       // tiles whose row scores a wave keeps in LDS before storing them in one
#define MSA_SCAN_BUF 16       //   burst (0: store after every tile)
#endif
#ifndef MSA_SCAN_GRID_MULT // workgroups launched per resident workgroup slot
#define MSA_SCAN_GRID_MULT 1
#endif
#ifndef MSA_SCAN_TILED_NT  // 1: non-temporal loads from the tiled bank
#define MSA_SCAN_TILED_NT 1
#endif
#if MSA_SCAN_NT
#define SCAN_LD ld16_nt
#else
#define SCAN_LD ld16
#endif

template <bool TILED>
__device__ __forceinline__ u32x4 scan_ld(const uint16_t *p) {
  if constexpr (TILED && MSA_SCAN_TILED_NT) return ld16_nt(p);
  else return SCAN_LD(p);
}

// DOCS (one token per query, the document path): instead of B scores per
// bank row the epilogue writes, per tile, the max over each run of rows that
// belongs to one document (a segmented max over the tile's 16 rows, runs
// marked by the document map): doc_part[d] for the document starting in the
// tile, tile_cont[tile] for rows continuing an earlier document.
template <int HR, int KS, int HG, bool TILED, bool DOCS>
__global__ __launch_bounds__(256) void scan_mfma_kernel(
    const uint16_t *__restrict__ kr, const uint16_t *__restrict__ qr, float *__restrict__ row_score,
    const int32_t *__restrict__ tile_doc, const uint32_t *__restrict__ tile_bits, float *__restrict__ doc_part,
    float *__restrict__ tile_cont, int qs, int n_docs, int64_t n_pool, int B, int Tq) {
  constexpr int NF = HR * KS;                     // fragments per 16-row tile per lane
  constexpr int DR = KS * 32;                     // router head dim
  constexpr int ROW = HR * DR;                    // elements per bank row
  constexpr int NG = HR / HG;                     // head groups per tile
  constexpr int GF = HG * KS;                     // fragments per head group
  __shared__ u32x4 afrag[NF * 64];
  __shared__ float qscale[8 * HR];
#if MSA_SCAN_BUF
  __shared__ float rbuf_all[kWaves * MSA_SCAN_BUF * 8 * 16];
#endif
  const int M = B * Tq;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  // 1 / (|q| Hr) per (token, head): four threads per (token, head), each
  // summing a quarter of the head's squares, with all of a thread's loads
  // in flight at once (at most 8 tokens x 8 heads: one pass)
  static_assert(DR % 32 == 0, "router head dim a multiple of 32");
  for (int base = 0; base < M * HR; base += 64) {
    const int mh = base + (threadIdx.x >> 2), part = threadIdx.x & 3;
    float ss = 0.f;
    if (mh < M * HR) {
      const uint16_t *src = qr + (int64_t)mh * DR + part * (DR / 4);
      u32x4 v[DR / 32];
#pragma unroll
      for (int i = 0; i < DR / 32; ++i) v[i] = ld16(src + 8 * i);
#pragma unroll
      for (int i = 0; i < DR / 32; ++i) {
        float x[8];
        Elt<uint16_t>::unpack(v[i], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
      }
    }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    if (part == 0 && mh < M * HR) qscale[mh] = 1.0f / (fmaxf(sqrtf(ss), kEps) * (float)HR);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < NF * 64; idx += blockDim.x) {
    const int l = idx & 63, f = idx >> 6;
    const int h = f / KS, s = f % KS;
    const int r = l & 15, m = r >> 1;
    uint32_t w[4] = {0, 0, 0, 0};
    if (m < M) {
      float x[8];
      Elt<uint16_t>::unpack(ld16(qr + ((int64_t)m * HR + h) * DR + 32 * s + 8 * (l >> 4)), x);
      const float sc = qscale[m * HR + h];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = x[e] * sc;
        const uint16_t hi = f32_to_bf16(y);
        const uint16_t val = (r & 1) ? f32_to_bf16(y - bf16_to_f32(hi)) : hi;
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

  const int64_t t_step = (int64_t)gridDim.x * kWaves;
#if MSA_SCAN_BUF
  // Row scores wait in LDS and go out in bursts of MSA_SCAN_BUF tiles: a store
  // after every tile (64 bytes per query) measured 1-6% slower (B = 1-8);
  // issuing the burst behind the next tile's first loads measured slower
  // still, as did storing in the order a wave produces the scores.
  float *rbuf = rbuf_all + wave * (MSA_SCAN_BUF * 8 * 16);   // [slot][query][row in tile]
  int n_buf = 0;
#endif
  for (int64_t tile = (int64_t)blockIdx.x * kWaves + wave; tile < n_tiles; tile += t_step) {
    const int64_t row = tile * 16 + col;
    // fragment f of this lane at rp + FS * f (the tiled bank holds whole
    // tiles; the row-major one is clamped to its last row)
    constexpr int FS = TILED ? 512 : 32;
    const uint16_t *rp;
    if constexpr (TILED) {
      rp = kr + tile * (16 * ROW) + 8 * lane;
    } else {
      const int64_t rowc = row < n_pool ? row : n_pool - 1;
      rp = kr + rowc * ROW + 8 * grp;
    }
    u32x4 cur[GF];
#pragma unroll
    for (int f = 0; f < GF; ++f) cur[f] = scan_ld<TILED>(rp + FS * f);
    uint32_t bits = 0;                     // the tile's document map, used at its end
    int32_t tdoc = 0;
    if constexpr (DOCS) {
      bits = tile_bits[tile];
      tdoc = tile_doc[tile];
    }

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
        for (int f = 0; f < GF; ++f) nxt[f] = scan_ld<TILED>(rp + FS * ((gi + 1) * GF + f));
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
    if constexpr (DOCS) {
      // query b's score of row col is ts[b]; runs: doubling steps within the
      // 16 lanes of a group, each taken only while no document starts between
      const bool run_start = col == 0 || ((bits >> col) & 1u);
      const bool starts_doc = (bits >> col) & 1u;
      int d = tdoc + __popc(bits & ((2u << col) - 2u));   // clamped: bad offsets give wrong numbers only
      d = d < 0 ? 0 : (d >= n_docs ? n_docs - 1 : d);
#pragma unroll
      for (int sh = 1; sh < 16; sh <<= 1) {
        const bool same = col + sh < 16 && ((bits >> (col + 1)) & ((1u << sh) - 1u)) == 0u;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          if (b < B) {
            const float u = __shfl_down(ts[b], sh, 16);
            ts[b] = same ? fmaxf(ts[b], u) : ts[b];
          }
        }
      }
      if (grp == 0 && run_start && row < n_pool) {
        float *dst = starts_doc ? doc_part + (int64_t)d * qs : tile_cont + tile * qs;
        *reinterpret_cast<f32x4 *>(dst) = f32x4{ts[0], ts[1], ts[2], ts[3]};
        if (qs > 4) *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{ts[4], ts[5], ts[6], ts[7]};
      }
    } else if (grp == 0) {
      for (int b = 0; b < B; ++b) {
        float m = -INFINITY;
        for (int t = 0; t < Tq; ++t) {
          const int slot = b * Tq + t;
          float v = ts[0];
#pragma unroll
          for (int q = 1; q < 8; ++q) v = slot == q ? ts[q] : v;
          m = fmaxf(m, v);
        }
#if MSA_SCAN_BUF
        rbuf[(n_buf * 8 + b) * 16 + col] = m;
#else
        if (row < n_pool) row_score[(int64_t)b * n_pool + row] = m;
#endif
      }
    }
#if MSA_SCAN_BUF
    // flush when the buffer is full or this was the wave's last tile: slot j
    // holds tile (tile - (n_buf - 1 - j) * t_step); the 64 lanes store four
    // (slot, query) pieces of 16 rows per instruction
    if constexpr (!DOCS) ++n_buf;
    if (!DOCS && (n_buf == MSA_SCAN_BUF || tile + t_step >= n_tiles)) {
      for (int idx = grp; idx < n_buf * B; idx += 4) {
        const int j = idx / B, b = idx - j * B;
        const int64_t r = (tile - (int64_t)(n_buf - 1 - j) * t_step) * 16 + col;
        if (r < n_pool) row_score[(int64_t)b * n_pool + r] = rbuf[(j * 8 + b) * 16 + col];
      }
      n_buf = 0;
    }
#endif
  }
}

template <int HR, int KS, bool TILED, bool DOCS>
hipError_t launch_scan_mfma_t(const msa_route_args &a, const RouteWs &ws, hipStream_t s) {
  constexpr int HG = HR < MSA_SCAN_HG ? HR : MSA_SCAN_HG;
  const int64_t n_tiles = (a.n_pool + 15) / 16;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, scan_mfma_kernel<HR, KS, HG, TILED, DOCS>, 256, 0) !=
          hipSuccess ||
      occ < 1)
    occ = 1;
  const int64_t want = (int64_t)device_info().n_cu * occ * MSA_SCAN_GRID_MULT;
  const int64_t need = (n_tiles + kWaves - 1) / kWaves;
  const int grid = (int)std::max<int64_t>(1, std::min(want, need));
  hipExtLaunchKernelGGL((scan_mfma_kernel<HR, KS, HG, TILED, DOCS>), dim3(grid), dim3(256), 0, s,
                        prof_event(a.prof_event_begin), prof_event(a.prof_event_end), 0,
                        reinterpret_cast<const uint16_t *>(a.kr_pooled), reinterpret_cast<const uint16_t *>(a.qr),
                        ws.row_score, ws.tile_doc, ws.tile_bits, ws.doc_part, ws.tile_cont, ws.qstride, a.n_docs,
                        a.n_pool, a.batch, a.q_tokens);
  return hipGetLastError();
}

template <int HR, int KS>
hipError_t launch_scan_mfma(const msa_route_args &a, const RouteWs &ws, hipStream_t s) {
  const bool docs = ws.qstride > 0;
  if (a.kr_layout == MSA_KR_TILED)
    return docs ? launch_scan_mfma_t<HR, KS, true, true>(a, ws, s) : launch_scan_mfma_t<HR, KS, true, false>(a, ws, s);
  return docs ? launch_scan_mfma_t<HR, KS, false, true>(a, ws, s) : launch_scan_mfma_t<HR, KS, false, false>(a, ws, s);
}

}  // namespace

hipError_t launch_scan_narrow(const msa_route_args &a, const RouteWs &ws, hipStream_t s) {
  const int ks = a.router_dim / 32;
  switch (a.n_router_heads * 8 + ks) {
    case 1 * 8 + 2: return launch_scan_mfma<1, 2>(a, ws, s);
    case 1 * 8 + 4: return launch_scan_mfma<1, 4>(a, ws, s);
    case 2 * 8 + 2: return launch_scan_mfma<2, 2>(a, ws, s);
    case 2 * 8 + 4: return launch_scan_mfma<2, 4>(a, ws, s);
    case 4 * 8 + 2: return launch_scan_mfma<4, 2>(a, ws, s);
    case 4 * 8 + 4: return launch_scan_mfma<4, 4>(a, ws, s);
    case 8 * 8 + 2: return launch_scan_mfma<8, 2>(a, ws, s);
    case 8 * 8 + 4: return launch_scan_mfma<8, 4>(a, ws, s);
    case 16 * 8 + 2: return launch_scan_mfma<16, 2>(a, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
