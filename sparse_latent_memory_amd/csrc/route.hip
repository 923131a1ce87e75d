// Routing, stage 2 of the method: workspace layout and kernel dispatch.
//
// Method: "EverMind-AI/MSA: Memory Sparse Attention for 100M-Token Contexts"
// (hysenlabs.com), section "How MSA compresses and routes documents"; stage 2
// of "EverMind Releases Memory-Sparse Attention Code for Long-Context AI
// Models" (toolmesh.ai), section "Architectural Design and Inference".
//
// One call runs, on one stream:
//  * the bank scan, row_score[b, j] = max over query b's tokens of the
//    head-mean cosine of pooled row j:
//      bf16, at most 8 tokens   scan_mfma_kernel (route_scan.hip), query prep
//                               fused in;
//      bf16, more tokens        prep_wide_direct + scan_wide_kernel
//                               (route_scan_wide.hip);
//      fp32                     prep_unit + scan_valu_kernel;
//  * selection (route_select.hip): per-document max, exact top-k, and with
//    device-side assembly the copy plan and the gather.
// The optional profiling events bracket the scan launch alone.
#include "msa_internal.h"

#include <algorithm>

#ifndef MSA_ROUTE_NARROW_DOCS   // 1: one-token batches of up to 8 queries also take the document path
#define MSA_ROUTE_NARROW_DOCS 1
#endif
#ifndef MSA_ROUTE_PREP_DIRECT   // 1: the wide scan's query fragments in one launch from the bf16 queries
#define MSA_ROUTE_PREP_DIRECT 1
#endif

namespace msa {
namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// bf16, at most 8 query tokens: fused-prep scan with hi/lo query rows
bool narrow_path(int32_t dtype, int32_t M, int32_t hr, int32_t dr) {
  return dtype == MSA_BF16 && M <= 8 && mfma_shape(hr, dr);
}
// bf16, more query tokens: query M-tiles streamed through LDS
bool wide_path(int32_t dtype, int32_t M, int32_t hr, int32_t dr) {
  return dtype == MSA_BF16 && M > 8 && mfma_shape(hr, dr);
}

}  // namespace

bool route_shape_supported(int32_t hr, int32_t dr) {
  if (dr != 64 && dr != 128) return false;
  if (hr < 1 || hr > 64 || (hr & (hr - 1)) != 0) return false;
  const int epl = hr * dr / 64;
  return epl <= 32 && (64 % hr) == 0;
}

size_t route_ws_layout(int32_t dtype, int32_t batch, int32_t q_tokens, int32_t hr, int32_t dr, int32_t n_docs,
                       int64_t n_pool, int32_t top_k, void *base, RouteWs *ws) {
  const int32_t M = batch * q_tokens;
  const int32_t n_blocks = (n_docs + kDocsPerBlock - 1) / kDocsPerBlock;
  const bool wide = wide_path(dtype, M, hr, dr);
  const bool narrow = narrow_path(dtype, M, hr, dr);
  const bool docs = (wide || (narrow && MSA_ROUTE_NARROW_DOCS)) && q_tokens == 1;   // the document path
  const int32_t n_parts = wide ? wide_layout(batch, q_tokens, wide_mg(hr * dr / 32, dr / 32)).n_parts : 1;
  const int64_t n_tiles = (n_pool + 15) / 16;
  const int32_t qstride = !docs ? 0 : wide ? wide_tiles(batch, 1) * 16 : (batch + 3) / 4 * 4;
  size_t off = 0;
  const size_t o_rs = off;
  if (!docs) off = align256(off + sizeof(float) * (size_t)batch * n_parts * (size_t)n_pool);
  const size_t o_dp = off;
  off = align256(off + sizeof(float) * (size_t)n_docs * qstride);
  const size_t o_tc = off;
  off = align256(off + sizeof(float) * (size_t)n_tiles * qstride);
  const size_t o_td = off;
  if (docs) off = align256(off + sizeof(int32_t) * (size_t)n_tiles);
  const size_t o_tb = off;
  if (docs) off = align256(off + sizeof(uint32_t) * (size_t)n_tiles);
  const size_t o_q = off;
  if (!narrow && !(wide && MSA_ROUTE_PREP_DIRECT)) off = align256(off + sizeof(float) * (size_t)M * hr * dr);
  const size_t o_w = off;
  if (wide) off = align256(off + sizeof(u32x4) * 64 * (size_t)hr * (dr / 32) * wide_tiles(batch, q_tokens));
  const size_t o_bm = off;
  off = align256(off + sizeof(uint64_t) * (size_t)batch * n_blocks);
  const size_t o_plan = off;
  off = align256(off + sizeof(GatherPlan) * (size_t)batch * top_k);
  if (ws) {
    char *p = reinterpret_cast<char *>(base);
    ws->row_score = reinterpret_cast<float *>(p + o_rs);
    ws->doc_part = reinterpret_cast<float *>(p + o_dp);
    ws->tile_cont = reinterpret_cast<float *>(p + o_tc);
    ws->tile_doc = reinterpret_cast<int32_t *>(p + o_td);
    ws->tile_bits = reinterpret_cast<uint32_t *>(p + o_tb);
    ws->qhat = reinterpret_cast<float *>(p + o_q);
    ws->wide_frag = reinterpret_cast<u32x4 *>(p + o_w);
    ws->blockmax = reinterpret_cast<uint64_t *>(p + o_bm);
    ws->plan = reinterpret_cast<GatherPlan *>(p + o_plan);
    ws->n_blocks = n_blocks;
    ws->n_parts = n_parts;
    ws->qstride = qstride;
    ws->map_given = 0;
  }
  return off;
}

hipError_t launch_route(const msa_route_args &a, const RouteWs &ws, const void *host_kv_dev, hipStream_t s) {
  const int M = a.batch * a.q_tokens;
  hipError_t e = hipSuccess;
  // the scan launchers attach a.prof_event_begin / _end to the scan kernel
  if (narrow_path(a.dtype, M, a.n_router_heads, a.router_dim)) {
    if (ws.qstride > 0 && !ws.map_given &&
        (e = launch_doc_map(a.doc_pool_off, a.n_docs, a.n_pool, ws.tile_doc, ws.tile_bits, s)) != hipSuccess)
      return e;
    e = launch_scan_narrow(a, ws, s);
  } else {
    if (wide_path(a.dtype, M, a.n_router_heads, a.router_dim)) {
#if MSA_ROUTE_PREP_DIRECT
      if ((e = launch_prep_wide_direct(a, ws.wide_frag, s)) != hipSuccess) return e;
#else
      if ((e = launch_prep_unit(a, ws.qhat, s)) != hipSuccess) return e;
      if ((e = launch_prep_wide(a, ws.qhat, ws.wide_frag, s)) != hipSuccess) return e;
#endif
      if (ws.qstride > 0 && !ws.map_given &&
          (e = launch_doc_map(a.doc_pool_off, a.n_docs, a.n_pool, ws.tile_doc, ws.tile_bits, s)) != hipSuccess)
        return e;
      e = launch_scan_wide(a, ws.wide_frag, ws, s);
    } else {
      if ((e = launch_prep_unit(a, ws.qhat, s)) != hipSuccess) return e;
      e = launch_scan_valu(a, ws.qhat, ws.row_score, s);
    }
  }
  if (e != hipSuccess) return e;
  return launch_select(a, ws, host_kv_dev, s);
}

}  // namespace msa
