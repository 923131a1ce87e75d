// Internal declarations shared by the libmsa translation units (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/msa.h"
#include "msa_device.h"

namespace msa {

// Optional profiling events of a call, attached to one kernel's dispatch
// (hipExtLaunchKernel): they time exactly that kernel and add no packets to
// the queue, unlike event records placed around the launch.
inline hipEvent_t prof_event(void *p) { return reinterpret_cast<hipEvent_t>(p); }

// ---------------------------------------------------------------------------
// launchers (validated arguments only)
// ---------------------------------------------------------------------------
struct DeviceInfo {
  int n_cu = 256;
};
const DeviceInfo &device_info();

hipError_t launch_pool(const msa_pool_args &a, hipStream_t s);

// One document's copy in the device-side context assembly.
struct GatherPlan {
  int64_t src_row;         // first pooled row in the host tier
  int32_t rows;            // 0: nothing to copy (dropped or empty)
  int32_t dst_row;         // first row in mem_kv[b]
};

struct RouteWs {  // carved out of the caller's workspace
  // row path (narrow scan, VALU scan, wide scan with several tokens per query)
  float *row_score;        // [B, n_parts, n_pool]
  // document path (one token per query, matrix-core scans): the scan reduces
  // every 16-row tile per document itself
  float *doc_part;         // [n_docs, qstride] max over a document's rows in the tile where it starts
  float *tile_cont;        // [n_tiles, qstride] max over a tile's first rows when they continue a document
  int32_t *tile_doc;       // [n_tiles] document holding the tile's first row
  uint32_t *tile_bits;     // [n_tiles] bit r: row 16 t + r starts a document (or is row n_pool)
  float *qhat;             // [B*Tq, Hr*dr] fp32 unit queries (VALU and wide scans)
  u32x4 *wide_frag;        // [n_mt, Hr*dr/32, 64] bf16 query fragments (wide scan)
  uint64_t *blockmax;      // [B, n_blocks] best document key per block of kDocsPerBlock documents
  GatherPlan *plan;        // [B, k]
  int32_t n_blocks;        // blocks of kDocsPerBlock documents
  int32_t n_parts;         // partial token maxima per query in row_score (wide scan), else 1
  int32_t qstride;         // query stride of doc_part / tile_cont: a multiple of 16 on the wide
                           // scan, B rounded up to 4 on the narrow one; 0 on the row path
  int32_t map_given;       // tile_doc / tile_bits point into a caller's document map
};
// Routing kernels.  The bank scan writes row_score[b, j] (max over query b's
// tokens of the head-mean cosine) or, on the document path, per-document
// parts of each tile; selection reduces them per document, takes the exact
// top-k and plans/performs the device-side assembly.
constexpr int kDocsPerBlock = 256;    // documents per block of the top-k bound

// v_mfma_f32_16x16x32_bf16 scan shapes: router dim 64 or 128, heads a power
// of two up to 8 (16 with dim 64)
inline bool mfma_shape(int32_t hr, int32_t dr) {
  const int ks = dr / 32;
  return (ks == 2 || ks == 4) && (hr == 1 || hr == 2 || hr == 4 || hr == 8 || (hr == 16 && ks == 2));
}
// query M-tiles of 16 rows in the wide scan
__host__ __device__ inline int wide_tiles(int32_t batch, int32_t q_tokens) {
  return q_tokens == 1 ? (batch + 15) / 16 : batch * ((q_tokens + 15) / 16);
}
// Query M-tiles the wide scan keeps in LDS at once, for ks = dr/32
// fragments per head and nf = Hr*ks per tile: at most 128 KiB of bf16
// fragments, at most 8 tiles, and at most 16/ks tiles, so one head's query
// fragments (NM*ks*4 registers) fit beside the accumulators at two waves
// per SIMD.
__host__ __device__ constexpr int wide_mg(int nf, int ks) {
  return (128 / nf < 16 / ks ? 128 / nf : 16 / ks) < 8 ? (128 / nf < 16 / ks ? 128 / nf : 16 / ks) : 8;
}
// How the wide scan splits the query tiles into chunks of at most mg tiles.
// Tq == 1: a tile holds 16 queries; chunk c = tiles [c*mg, (c+1)*mg).
// Tq > 1: query b owns mtq = ceil(Tq/16) tiles.  If mtq <= mg a chunk holds
// qpc = mg/mtq whole queries; otherwise query b is cut into ppq parts of at
// most mg tiles, each scanned by its own workgroup, and row_score gets one
// partial max per part: row_score[(b*n_parts + part)*n_pool + j].
struct WideLayout {
  int tok1;        // Tq == 1
  int mg, mtq, n_mt, qpc, ppq, n_chunks, n_parts;
};
__host__ __device__ inline WideLayout wide_layout(int32_t batch, int32_t q_tokens, int mg) {
  WideLayout L;
  L.mg = mg;
  L.tok1 = q_tokens == 1;
  L.n_mt = wide_tiles(batch, q_tokens);
  if (L.tok1) {
    L.mtq = 1; L.qpc = 16; L.ppq = 1;
    L.n_chunks = (L.n_mt + mg - 1) / mg;
  } else {
    L.mtq = (q_tokens + 15) / 16;
    if (L.mtq <= mg) {
      L.qpc = mg / L.mtq; L.ppq = 1;
      L.n_chunks = (batch + L.qpc - 1) / L.qpc;
    } else {
      L.qpc = 0; L.ppq = (L.mtq + mg - 1) / mg;
      L.n_chunks = batch * L.ppq;
    }
  }
  L.n_parts = L.ppq;
  return L;
}
// tiles [t0, t1) of chunk c
__host__ __device__ inline void wide_chunk(const WideLayout &L, int c, int *t0, int *t1) {
  if (L.tok1) {
    *t0 = c * L.mg;
    *t1 = c * L.mg + L.mg < L.n_mt ? c * L.mg + L.mg : L.n_mt;
  } else if (L.ppq == 1) {
    *t0 = c * L.qpc * L.mtq;
    *t1 = (c + 1) * L.qpc * L.mtq < L.n_mt ? (c + 1) * L.qpc * L.mtq : L.n_mt;
  } else {
    const int q = c / L.ppq, p = c % L.ppq;
    *t0 = q * L.mtq + p * L.mg;
    *t1 = q * L.mtq + ((p + 1) * L.mg < L.mtq ? (p + 1) * L.mg : L.mtq);
  }
}
// bf16, at most 8 query tokens (route_scan.hip)
hipError_t launch_scan_narrow(const msa_route_args &a, const RouteWs &ws, hipStream_t s);
// fp32 unit queries (route_scan_wide.hip)
hipError_t launch_prep_unit(const msa_route_args &a, float *qhat, hipStream_t s);
// bf16 query fragments and the MFMA scan for more than 8 tokens
hipError_t launch_prep_wide(const msa_route_args &a, const float *qhat, u32x4 *frag, hipStream_t s);
// the same fragments straight from bf16 queries (norms included), one launch
hipError_t launch_prep_wide_direct(const msa_route_args &a, u32x4 *frag, hipStream_t s);
hipError_t launch_scan_wide(const msa_route_args &a, const u32x4 *frag, const RouteWs &ws, hipStream_t s);
// fp32 (any token count): one wave per bank row
hipError_t launch_scan_valu(const msa_route_args &a, const float *qhat, float *row_score, hipStream_t s);
// document map of the document path, per-document scores, exact top-k,
// assembly plan and device-side gather (route_select.hip)
hipError_t launch_doc_map(const int64_t *pool_off, int32_t n_docs, int64_t n_pool, int32_t *tile_doc,
                          uint32_t *tile_bits, hipStream_t s);
// the document map's layout (msa_doc_map): tile_doc at 0, tile_bits here
inline size_t doc_map_bits_offset(int64_t n_pool) {
  return ((size_t)4 * (size_t)((n_pool + 15) / 16) + 255) & ~(size_t)255;
}
hipError_t launch_select(const msa_route_args &a, const RouteWs &ws, const void *host_kv_dev, hipStream_t s);
// msa_assemble in the device-side mode: the copy plan from given top-k ids,
// then the gather (plan: [B, k] in the caller's workspace)
hipError_t launch_assemble(const msa_assemble_args &a, GatherPlan *plan, const void *host_kv_dev, hipStream_t s);

size_t route_ws_layout(int32_t dtype, int32_t batch, int32_t q_tokens, int32_t hr, int32_t dr,
                       int32_t n_docs, int64_t n_pool, int32_t top_k, void *base, RouteWs *ws);
// host_kv_dev: device address of the pinned host tier for device-side
// assembly, or NULL (no assembly, or host-driven copies)
hipError_t launch_route(const msa_route_args &a, const RouteWs &ws, const void *host_kv_dev, hipStream_t s);

size_t decode_ws_layout(int32_t batch, int32_t hq, int32_t d, int32_t mem_cap, int32_t local_cap,
                        void *base, float **part_acc, float **part_ml, int32_t *n_split);
hipError_t launch_decode(const msa_decode_args &a, float *part_acc, float *part_ml, int32_t n_split,
                         hipStream_t s);

// Block attention: work items (query, KV head, 16-row query tile, key split).
struct AttendPlan {
  int32_t n_mt;            // 16-row tiles of (token, head) rows per KV head
  int32_t rps;             // rows kept per partial slot: min(16, Tq * G)
  int32_t split_len;       // keys per split, a multiple of 64
  int32_t n_split;
};
void attend_plan(int32_t batch, int32_t q_tokens, int32_t hq, int32_t hkv, int32_t mem_cap, int32_t local_cap,
                 AttendPlan *p);
// Attention workspace: split partials, and the local keys and the query
// block rotated once when several query tiles per KV head read them (else
// rot_k and rot_q are null).
struct AttendWs {
  float *part_acc;
  float *part_ml;
  uint16_t *rot_k;         // [B, local_cap, Hkv, D] bf16 or null
  float *rot_q;            // [B, Tq, Hq, D] fp32, rotated and scaled, or null (with rot_k)
};
size_t attend_ws_layout(int32_t batch, int32_t q_tokens, int32_t hq, int32_t hkv, int32_t d, int32_t mem_cap,
                        int32_t local_cap, void *base, AttendWs *ws);
hipError_t launch_attend(const msa_attend_args &a, const AttendWs &ws, hipStream_t s);

}  // namespace msa
