// Routing, stage 2 of the method: the bank scan for more than 8 bf16 query
// tokens (prefill routing, or many decode queries batched) on MFMA, and the
// fp32 scan on the VALU.
//
// Method: "EverMind-AI/MSA: Memory Sparse Attention for 100M-Token Contexts"
// (hysenlabs.com), section "How MSA compresses and routes documents": the
// score of a pooled row is the cosine of the routing query and the pooled
// router key, averaged over router heads and maximised over query tokens.
// Output of every scan: row_score[b, j] = max over query b's tokens.
#include "msa_internal.h"

#include <algorithm>

namespace msa {
namespace {

constexpr int kWaves = 4;            // waves per workgroup

// --------------------------------------------------------------------------
// fp32 unit queries (VALU scan, and input of the wide fragments): qhat[m, h*dr + i] =
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
// bf16 MFMA scan for many query tokens (more than 8)
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

// The same fragments straight from the bf16 queries, one launch instead of
// prep_unit + prep_wide: each thread sums the squares of its (token, head)
// row itself (the row's 16 threads read it from L2) and writes its 8
// elements scaled by 1 / (max(|q|, eps) Hr), rounded to bf16 once.
template <int DR>
__global__ __launch_bounds__(256) void prep_wide_direct_kernel(const uint16_t *__restrict__ qr,
                                                               u32x4 *__restrict__ frag, int B, int Tq, int Hr,
                                                               int n_mt) {
  constexpr int KS = DR / 32;
  const int NF = Hr * KS;
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
      const uint16_t *row = qr + ((int64_t)m * Hr + h) * DR;
      u32x4 v[DR / 8];                        // the whole row in flight at once
#pragma unroll
      for (int i = 0; i < DR / 8; ++i) v[i] = ld16(row + 8 * i);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < DR / 8; ++i) {
        float x[8];
        Elt<uint16_t>::unpack(v[i], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
      }
      const float scale = 1.0f / (fmaxf(sqrtf(ss), kEps) * (float)Hr);
      float x[8];
      Elt<uint16_t>::unpack(ld16(row + 32 * s + 8 * (l >> 4)), x);   // this lane's 8 elements (a cached line)
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e >> 1] |= (uint32_t)f32_to_bf16(x[e] * scale) << (16 * (e & 1));
    }
    u32x4 o;
    o.x = w[0]; o.y = w[1]; o.z = w[2]; o.w = w[3];
    frag[idx] = o;
  }
}

// One workgroup of 8 waves per CU (two per SIMD).  The workgroup keeps one
// chunk of NM query M-tiles in LDS (at most 128 KiB) for the whole launch;
// every wave streams 16-row bank tiles from HBM one head at a time, loading
// the next head (or the next tile's first head) into the other of two
// fragment buffers while it computes: per head, 4 MFMAs give the tile's Gram
// matrix (norms on its diagonal) and each of the NM query tiles takes 4
// MFMAs against A-fragments read from LDS, scaled by the head's inverse norm.
// Tiles of a chunk past its last real one are staged as zeros and their
// results dropped, so the MFMA loop has no branches.
// A workgroup that walks only a few groups of bank tiles (a small bank:
// prefill routing), or whose query tiles span several chunks, runs heads
// outer instead, over batches of up to three of the wave's tiles: each
// head's query fragments are read from LDS once per batch into registers
// and applied to all of the batch's tiles, whose accumulators stay live,
// with one bank-fragment slot per tile refilled as it is used.
// When the query tiles span several chunks, chunks go to different
// workgroups of one XCD that walk the same bank tiles in the same order, so
// the bank is fetched from HBM about once and re-read from the XCD's L2 or
// the MALL; workgroups are dispatched round-robin over the 8 XCDs, which the
// XCD-major logical id below follows.
constexpr int kWideWaves = 8;
#ifndef MSA_WIDE_HEAD_OUTER // 1: heads outer when a workgroup walks few bank-tile groups (wide_tmax)
#define MSA_WIDE_HEAD_OUTER 1
#endif
// Tiles per wave the heads-outer loop takes: as many (up to 3; 2 with two or
// four heads, whose loops are unrolled; 1 for chunks of 8 query tiles) as fit its
// registers - a head's query fragments (4 NM KS), per tile a bank-fragment
// slot (4 KS) and 4 NM accumulators, and 4 NM more for the epilogue -
// within a budget of 176 (the caps and the budget are where the compiled
// instantiations stop spilling); 0: never.
template <int HR, int NM, int KS>
constexpr int wide_tmax() {
  int t = NM >= 8 ? 1 : HR <= 4 ? 2 : 3;
  while (t > 0 && 4 * NM * KS + 4 * KS * t + 4 * NM * (t + 1) > 176) --t;
  return t;
}
#ifndef MSA_WIDE_STAGE_ROT // 1: workgroups staging the same query chunk start at different eighths of it
#define MSA_WIDE_STAGE_ROT 1
#endif

// One doubling step of the segmented max over the 16 rows of a tile (lane
// column = row): row r takes row r + SH's running max while no document
// starts in rows r+1 .. r+SH.  The value of row r + SH arrives through a DPP
// row shift (row_shl, within each 16-lane row), so the step costs vector
// instructions only, no LDS permute.
template <int SH>
__device__ __forceinline__ void seg_step(f32x4 &v, int col, uint32_t bits) {
  const bool same = col + SH < 16 && ((bits >> (col + 1)) & ((1u << SH) - 1u)) == 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float u = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v[i]), 0x100 + SH, 0xf, 0xf, false));
    v[i] = same ? fmaxf(v[i], u) : v[i];
  }
}
// Bank layouts of the wide scan: row-major, tiled (plain loads: several
// query chunks share each bank tile through L2) and tiled with non-temporal
// loads (one query chunk: every tile is read once; measured 13-14% faster at
// 16-64 queries, and twice as slow when chunks share tiles).
enum WideBank { kWideRows = 0, kWideTiled = 1, kWideTiledNT = 2 };

// One token per query (the document path): instead of B scores per bank row
// the epilogue writes, per tile and query, the max over each run of rows
// that belongs to one document (a segmented max over the tile's 16 rows,
// runs marked by the document map): doc_part[d] for the document starting
// in the tile, tile_cont[tile] for rows continuing an earlier document.
// Storing B scores per row cost a third of the scan at 64 queries.
template <int HR, int KS, int NM, int BANK>
__global__ __launch_bounds__(kWideWaves * 64) void scan_wide_kernel(
    const uint16_t *__restrict__ kr, const u32x4 *__restrict__ frag, float *__restrict__ row_score,
    const int32_t *__restrict__ tile_doc, const uint32_t *__restrict__ tile_bits, float *__restrict__ doc_part,
    float *__restrict__ tile_cont, int qstride, int n_docs, int64_t n_pool, int B, int Tq) {
  constexpr int NF = HR * KS;
  constexpr int ROW = NF * 32;
  static_assert(NM <= wide_mg(NF, KS), "query chunk exceeds the LDS budget");
  __shared__ u32x4 afrag[NM * NF * 64];
  if (n_pool <= 0) return;              // (rejected by the API; the loads below clamp to row n_pool-1)
  const WideLayout L = wide_layout(B, Tq, wide_mg(NF, KS));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int diag_src = ((col >> 2) << 4) + col;

  const int nwg = gridDim.x, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per = nwg >> 3, rem = nwg & 7;
  const int lid = xcd * per + min(xcd, rem) + slot;
  int S, stream, c0, cstep;
  if (L.n_chunks <= nwg) {
    S = nwg / L.n_chunks;               // bank streams, each scanned once per chunk
    stream = lid / L.n_chunks;
    c0 = lid % L.n_chunks;
    cstep = L.n_chunks;
    if (stream >= S) return;            // whole workgroup: no barrier is left waiting
  } else {
    S = 1; stream = 0; c0 = lid; cstep = nwg;
  }
  const int64_t n_tiles = (n_pool + 15) >> 4;
  const int64_t n_groups = (n_tiles + kWideWaves - 1) / kWideWaves;

  // fragments of head h of this wave's tile in group g (groups past the end
  // read the last group; in the row-major bank rows past the end read its
  // last row, the tiled bank holds whole tiles and the last tile is clamped)
  auto load = [&](int64_t g, int h, u32x4 *dst) {
    g = g < n_groups ? g : n_groups - 1;
    if constexpr (BANK != kWideRows) {
      int64_t tile = g * kWideWaves + wave;
      tile = tile < n_tiles ? tile : n_tiles - 1;
      const uint16_t *rp = kr + tile * (16 * ROW) + h * KS * 512 + 8 * lane;
#pragma unroll
      for (int s = 0; s < KS; ++s) dst[s] = BANK == kWideTiledNT ? ld16_nt(rp + 512 * s) : ld16(rp + 512 * s);
    } else {
      int64_t row = (g * kWideWaves + wave) * 16 + col;
      row = row < n_pool ? row : n_pool - 1;
      const uint16_t *rp = kr + row * ROW + h * KS * 32 + 8 * grp;
#pragma unroll
      for (int s = 0; s < KS; ++s) dst[s] = ld16(rp + 32 * s);
    }
  };
  // One head of the tile: the query fragments are read from LDS in one batch
  // ahead of the MFMAs (the scheduling barrier keeps the compiler from
  // pairing each read with its MFMA), the Gram MFMAs covering their latency.
  auto read_a = [&](int h, u32x4 (&a)[NM][KS]) {
#pragma unroll
    for (int mt = 0; mt < NM; ++mt)
#pragma unroll
      for (int s = 0; s < KS; ++s) a[mt][s] = afrag[(mt * NF + h * KS + s) * 64 + lane];
  };
  auto head_mma = [&](const u32x4 (&a)[NM][KS], const u32x4 *f, f32x4 *acc) {
    f32x4 gm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 bv = __builtin_bit_cast(bf16x8, f[s]);
      gm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv, bv, gm, 0, 0, 0);
    }
    f32x4 d[NM];
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) d[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int mt = 0; mt < NM; ++mt)
        d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mt][s]),
                                                        __builtin_bit_cast(bf16x8, f[s]), d[mt], 0, 0, 0);
    const int di = col & 3;              // selects, not branches: the body stays one basic block
    float mine = gm[0];
    mine = di == 1 ? gm[1] : mine;
    mine = di == 2 ? gm[2] : mine;
    mine = di == 3 ? gm[3] : mine;
    const float inv = rsqrtf(fmaxf(__shfl(mine, diag_src, 64), kEps2));
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) acc[mt] += d[mt] * inv;
  };
  auto head = [&](int h, const u32x4 *f, f32x4 *acc) {
    u32x4 a[NM][KS];
    read_a(h, a);
    __builtin_amdgcn_sched_barrier(0);
    head_mma(a, f, acc);
  };

  // Document path (Tq == 1): lane (col, grp) holds, for bank row col of the
  // tile, the scores of queries 16 (t0 + mt) + 4 grp + i in acc[mt][i].
  // After the segmented max (doubling steps within the 16 lanes of a group,
  // each taken only while no document starts in between), a lane whose row
  // starts a run holds the run's max and stores its 4 queries at once.
  auto epilogue_docs = [&](int t0, int nm, int64_t tile, uint32_t bits, int32_t tdoc, const f32x4 *acc) {
    const int64_t row = tile * 16 + col;
    const bool run_start = col == 0 || ((bits >> col) & 1u);
    const bool starts_doc = (bits >> col) & 1u;
    // document of a run that starts here: the tile's first document plus the
    // starts in rows 1..col (clamped: bad offsets give wrong numbers only)
    int d = tdoc + __popc(bits & ((2u << col) - 2u));
    d = d < 0 ? 0 : (d >= n_docs ? n_docs - 1 : d);
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) {
      if (mt >= nm) break;                // (uniform)
      f32x4 v = acc[mt];
      seg_step<1>(v, col, bits);
      seg_step<2>(v, col, bits);
      seg_step<4>(v, col, bits);
      seg_step<8>(v, col, bits);
      if (run_start && row < n_pool) {
        const int b0 = (t0 + mt) * 16 + 4 * grp;
        float *dst = starts_doc ? doc_part + (int64_t)d * qstride + b0 : tile_cont + tile * qstride + b0;
        *reinterpret_cast<f32x4 *>(dst) = v;
      }
    }
  };
  // row scores of one bank tile (Tq > 1): per query the max over the
  // chunk's tiles of that query
  auto epilogue = [&](int t0, int nm, int part, int64_t row, const f32x4 *acc) {
    {
      float qmax = -INFINITY;         // max over the chunk's tiles of one query
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
        float m = fmaxf(fmaxf(acc[mt][0], acc[mt][1]), fmaxf(acc[mt][2], acc[mt][3]));
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        qmax = fmaxf(qmax, m);
        const int t = t0 + mt;
        if (mt < nm && ((t + 1) % L.mtq == 0 || mt == nm - 1)) {
          if (grp == 0) row_score[((int64_t)(t / L.mtq) * L.n_parts + part) * n_pool + row] = qmax;
          qmax = -INFINITY;
        }
      }
    }
  };

  for (int c = c0; c < L.n_chunks; c += cstep) {
    int t0, t1;
    wide_chunk(L, c, &t0, &t1);
    const int nm = t1 - t0;
    const int part = L.ppq > 1 ? c % L.ppq : 0;
    const int64_t n_my = stream < n_groups ? (n_groups - 1 - stream) / S + 1 : 0;   // groups this workgroup walks
    if (n_my == 0) continue;            // (uniform over the workgroup) no bank tile: nothing to stage or store
    // The chunk into LDS by gfx950's loads straight to LDS (16 bytes a lane,
    // no registers: the first bank loads are issued behind them and land
    // while the chunk does), each wave 1 KiB fragments; tiles past the
    // chunk's last copy its last one (their results are never stored).  The
    // workgroups of one XCD that stage the same chunk start at different
    // eighths of it: each line is fetched from memory by one and found in L2
    // by the others, instead of all of them waiting on the same misses.
    auto stage_chunk = [&]() {
      constexpr int NFR = NM * NF;
      const int rot = MSA_WIDE_STAGE_ROT ? ((L.n_chunks <= nwg ? stream : 0) & 7) * NFR / 8 : 0;
      for (int f0 = wave; f0 < NFR; f0 += kWideWaves) {   // (uniform)
        const int f = (f0 + rot) % NFR, mt = f / NF;
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void *>(frag + ((int64_t)t0 + min(mt, nm - 1)) * NF * 64 + (f % NF) * 64 + lane),
            (__attribute__((address_space(3))) void *)(afrag + f * 64), 16, 0, 0);
      }
    };
    __syncthreads();                    // readers of the previous chunk are done

    // Few bank tiles per wave (a small bank), or several chunks of query
    // tiles (the tile loop would re-read a chunk's fragments from LDS for
    // every bank tile): heads outer over batches of the wave's tiles, so that
    // a head's query fragments are read from LDS once per batch and kept in
    // registers, the batch's accumulators live; the per-head order of the
    // sums is that of the tile loop below, which keeps the one-chunk scans
    // of large banks (bound by HBM, their tiles streamed whole).
    constexpr int TM = wide_tmax<HR, NM, KS>();
    if constexpr (HR > 1 && MSA_WIDE_HEAD_OUTER && TM > 0) {
      if (n_my <= TM || L.n_chunks > 1) {
        // The wave's groups in batches of TM, heads outer within a batch.
        // One fragment slot per tile, refilled with the tile's next head as
        // soon as it is used, and in the batch's last head with the next
        // batch's first: TM loads in flight per wave throughout.  No
        // branches: slots past the workgroup's last group repeat its last
        // group (lines already requested), their results never stored.
        u32x4 fr[TM][KS];
        auto gof = [&](int64_t j) { return stream + (j < n_my ? j : n_my - 1) * S; };
        stage_chunk();
#pragma unroll
        for (int j = 0; j < TM; ++j) load(gof(j), 0, fr[j]);
        __syncthreads();                // the chunk in place (and the first bank fragments landed)
        for (int64_t jb = 0; jb < n_my; jb += TM) {   // (uniform)
          f32x4 acc[TM][NM];
#pragma unroll
          for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int mt = 0; mt < NM; ++mt) acc[j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
          for (int h = 0; h < HR - 1; ++h) {
            u32x4 a[NM][KS];
            read_a(h, a);
#pragma unroll
            for (int j = 0; j < TM; ++j) {
              __builtin_amdgcn_sched_barrier(0);
              head_mma(a, fr[j], acc[j]);
              load(gof(jb + j), h + 1, fr[j]);
            }
          }
          {
            u32x4 a[NM][KS];
            read_a(HR - 1, a);
#pragma unroll
            for (int j = 0; j < TM; ++j) {
              __builtin_amdgcn_sched_barrier(0);
              head_mma(a, fr[j], acc[j]);
              load(gof(jb + TM + j), 0, fr[j]);   // (after the last batch: valid, unused)
            }
          }
#pragma unroll
          for (int j = 0; j < TM; ++j) {
            if (jb + j < n_my) {
              const int64_t tile = (stream + (jb + j) * S) * kWideWaves + wave;
              const int64_t row = tile * 16 + col;
              if (L.tok1) {
                const int64_t tc = tile < n_tiles ? tile : n_tiles - 1;
                const uint32_t bits = tile_bits[tc];
                const int32_t tdoc = tile_doc[tc];
                if (tile < n_tiles) epilogue_docs(t0, nm, tile, bits, tdoc, acc[j]);   // (wave-uniform)
              } else if (row < n_pool) {
                epilogue(t0, nm, part, row, acc[j]);
              }
            }
          }
        }
        continue;
      }
    }

    stage_chunk();
    u32x4 fa[KS], fb[KS];
    load(stream, 0, fa);
    __syncthreads();                    // the chunk in place
    for (int64_t g = stream; g < n_groups; g += S) {
      const int64_t tile = g * kWideWaves + wave;
      const int64_t row = tile * 16 + col;
      // the tile's document map (document path), requested ahead of its use
      uint32_t bits = 0;
      int32_t tdoc = 0;
      if (L.tok1) {
        const int64_t tc = tile < n_tiles ? tile : n_tiles - 1;
        bits = tile_bits[tc];
        tdoc = tile_doc[tc];
      }
      f32x4 acc[NM];
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (HR == 1) {
        load(g + S, 0, fb);
        __builtin_amdgcn_sched_barrier(0);   // the prefetch stays ahead of the compute
        head(0, fa, acc);
#pragma unroll
        for (int s = 0; s < KS; ++s) fa[s] = fb[s];
      } else {
        // two heads per step, fa and fb alternating; fa ends on the next tile's head 0
#pragma unroll 1
        for (int h = 0; h < HR; h += 2) {
          load(g, h + 1, fb);
          __builtin_amdgcn_sched_barrier(0);   // the prefetch stays ahead of the compute
          head(h, fa, acc);
          const bool last = h + 2 >= HR;       // no branch: the loads stay where they are written
          load(last ? g + S : g, last ? 0 : h + 2, fa);
          __builtin_amdgcn_sched_barrier(0);
          head(h + 1, fb, acc);
        }
      }
      if (L.tok1) {
        if (tile < n_tiles) epilogue_docs(t0, nm, tile, bits, tdoc, acc);   // (wave-uniform)
      } else if (row < n_pool) {
        epilogue(t0, nm, part, row, acc);
      }
    }
  }
}

// --------------------------------------------------------------------------
// VALU scan (fp32): one wave per row
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

template <int HR, int KS, int NM, int BANK>
void launch_wide_bank(const msa_route_args &a, const u32x4 *frag, const RouteWs &ws, hipStream_t s) {
  // one workgroup per CU (the query chunk takes most of the LDS)
  hipExtLaunchKernelGGL((scan_wide_kernel<HR, KS, NM, BANK>), dim3(device_info().n_cu), dim3(kWideWaves * 64), 0,
                        s, prof_event(a.prof_event_begin), prof_event(a.prof_event_end), 0,
                        reinterpret_cast<const uint16_t *>(a.kr_pooled), frag, ws.row_score, ws.tile_doc,
                        ws.tile_bits, ws.doc_part, ws.tile_cont, ws.qstride, a.n_docs, a.n_pool, a.batch,
                        a.q_tokens);
}

template <int HR, int KS, int NM>
hipError_t launch_wide_nm(const msa_route_args &a, const u32x4 *frag, const RouteWs &ws, hipStream_t s) {
  if (a.kr_layout != MSA_KR_TILED)
    launch_wide_bank<HR, KS, NM, kWideRows>(a, frag, ws, s);
  else if (wide_layout(a.batch, a.q_tokens, wide_mg(HR * KS, KS)).n_chunks == 1)
    launch_wide_bank<HR, KS, NM, kWideTiledNT>(a, frag, ws, s);
  else
    launch_wide_bank<HR, KS, NM, kWideTiled>(a, frag, ws, s);
  return hipGetLastError();
}

// NM = the largest chunk, rounded up to a power of two (at most the LDS budget)
template <int HR, int KS>
hipError_t launch_wide_t(const msa_route_args &a, const u32x4 *frag, const RouteWs &ws, hipStream_t s) {
  constexpr int MG = wide_mg(HR * KS, KS);
  const WideLayout L = wide_layout(a.batch, a.q_tokens, MG);
  int need = 0;
  for (int c = 0; c < L.n_chunks && need < MG; ++c) {
    int t0, t1;
    wide_chunk(L, c, &t0, &t1);
    need = std::max(need, t1 - t0);
  }
  if (need <= 1) return launch_wide_nm<HR, KS, 1>(a, frag, ws, s);
  if (need <= 2 || MG < 4) return launch_wide_nm<HR, KS, (MG < 2 ? MG : 2)>(a, frag, ws, s);
  if (need <= 4 || MG < 8) return launch_wide_nm<HR, KS, (MG < 4 ? MG : 4)>(a, frag, ws, s);
  return launch_wide_nm<HR, KS, (MG < 8 ? MG : 8)>(a, frag, ws, s);
}

template <typename T, int EPL>
hipError_t launch_valu_t(const msa_route_args &a, const float *qhat, float *row_score, hipStream_t s) {
  const int64_t need = (a.n_pool + kWaves - 1) / kWaves;
  const int64_t want = (int64_t)device_info().n_cu * 8;
  const int grid = (int)std::max<int64_t>(1, std::min(want, need));
  const int lanes_per_head = 64 / a.n_router_heads;
  hipExtLaunchKernelGGL((scan_valu_kernel<T, EPL>), dim3(grid), dim3(256), 0, s, prof_event(a.prof_event_begin),
                        prof_event(a.prof_event_end), 0, reinterpret_cast<const T *>(a.kr_pooled), qhat, row_score,
                        a.n_pool, a.batch, a.q_tokens, lanes_per_head);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_valu(const msa_route_args &a, const float *qhat, float *row_score, hipStream_t s) {
  switch (a.n_router_heads * a.router_dim / 64) {
    case 1: return launch_valu_t<T, 1>(a, qhat, row_score, s);
    case 2: return launch_valu_t<T, 2>(a, qhat, row_score, s);
    case 4: return launch_valu_t<T, 4>(a, qhat, row_score, s);
    case 8: return launch_valu_t<T, 8>(a, qhat, row_score, s);
    case 16: return launch_valu_t<T, 16>(a, qhat, row_score, s);
    case 32: return launch_valu_t<T, 32>(a, qhat, row_score, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prep_unit(const msa_route_args &a, float *qhat, hipStream_t s) {
  const int M = a.batch * a.q_tokens;
  const int n = M * a.n_router_heads;
  const int grid = std::max(1, std::min((n + kWaves - 1) / kWaves, 1024));
  if (a.dtype == MSA_BF16)
    hipLaunchKernelGGL(prep_unit_kernel<uint16_t>, dim3(grid), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t *>(a.qr), qhat, M, a.n_router_heads, a.router_dim);
  else
    hipLaunchKernelGGL(prep_unit_kernel<float>, dim3(grid), dim3(256), 0, s, reinterpret_cast<const float *>(a.qr),
                       qhat, M, a.n_router_heads, a.router_dim);
  return hipGetLastError();
}

hipError_t launch_prep_wide(const msa_route_args &a, const float *qhat, u32x4 *frag, hipStream_t s) {
  const int n_mt = wide_tiles(a.batch, a.q_tokens);
  const int64_t n = (int64_t)n_mt * a.n_router_heads * (a.router_dim / 32) * 64;
  hipLaunchKernelGGL(prep_wide_kernel, dim3((int)std::min<int64_t>((n + 255) / 256, 4096)), dim3(256), 0, s, qhat,
                     frag, a.batch, a.q_tokens, a.n_router_heads, a.router_dim, n_mt);
  return hipGetLastError();
}

hipError_t launch_prep_wide_direct(const msa_route_args &a, u32x4 *frag, hipStream_t s) {
  const int n_mt = wide_tiles(a.batch, a.q_tokens);
  const int64_t n = (int64_t)n_mt * a.n_router_heads * (a.router_dim / 32) * 64;
  const dim3 grid((int)std::min<int64_t>((n + 255) / 256, 4096));
  const uint16_t *qr = reinterpret_cast<const uint16_t *>(a.qr);
  if (a.router_dim == 64)
    hipLaunchKernelGGL(prep_wide_direct_kernel<64>, grid, dim3(256), 0, s, qr, frag, a.batch, a.q_tokens,
                       a.n_router_heads, n_mt);
  else
    hipLaunchKernelGGL(prep_wide_direct_kernel<128>, grid, dim3(256), 0, s, qr, frag, a.batch, a.q_tokens,
                       a.n_router_heads, n_mt);
  return hipGetLastError();
}

hipError_t launch_scan_wide(const msa_route_args &a, const u32x4 *frag, const RouteWs &ws, hipStream_t s) {
  switch (a.n_router_heads * 8 + a.router_dim / 32) {
    case 1 * 8 + 2: return launch_wide_t<1, 2>(a, frag, ws, s);
    case 1 * 8 + 4: return launch_wide_t<1, 4>(a, frag, ws, s);
    case 2 * 8 + 2: return launch_wide_t<2, 2>(a, frag, ws, s);
    case 2 * 8 + 4: return launch_wide_t<2, 4>(a, frag, ws, s);
    case 4 * 8 + 2: return launch_wide_t<4, 2>(a, frag, ws, s);
    case 4 * 8 + 4: return launch_wide_t<4, 4>(a, frag, ws, s);
    case 8 * 8 + 2: return launch_wide_t<8, 2>(a, frag, ws, s);
    case 8 * 8 + 4: return launch_wide_t<8, 4>(a, frag, ws, s);
    case 16 * 8 + 2: return launch_wide_t<16, 2>(a, frag, ws, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan_valu(const msa_route_args &a, const float *qhat, float *row_score, hipStream_t s) {
  return a.dtype == MSA_BF16 ? launch_valu<uint16_t>(a, qhat, row_score, s)
                             : launch_valu<float>(a, qhat, row_score, s);
}

}  // namespace msa
