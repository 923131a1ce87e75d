// C ABI entry points of libmsa: argument checks, workspace carving, the
// host-driven context assembly, and error reporting.  Kernels live in
// pool.hip, route.hip and decode.hip.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "msa_internal.h"

namespace msa {

bool route_shape_supported(int32_t hr, int32_t dr);

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(MSA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int32_t d) { return d == MSA_F32 || d == MSA_BF16; }
size_t elt_size(int32_t d) { return d == MSA_BF16 ? 2 : 4; }
bool dim_ok(int32_t d) { return d == 64 || d == 128; }

// per-thread, per-device events for the assembly path
struct ThreadEvents {
  int device = -1;
  hipEvent_t topk = nullptr, copies = nullptr;
  ~ThreadEvents() {
    if (topk) (void)hipEventDestroy(topk);
    if (copies) (void)hipEventDestroy(copies);
  }
};
thread_local ThreadEvents g_ev;

hipError_t thread_events(ThreadEvents **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (g_ev.device != dev) {
    if (g_ev.topk) (void)hipEventDestroy(g_ev.topk);
    if (g_ev.copies) (void)hipEventDestroy(g_ev.copies);
    g_ev.topk = g_ev.copies = nullptr;
    if ((e = hipEventCreateWithFlags(&g_ev.topk, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&g_ev.copies, hipEventDisableTiming)) != hipSuccess) return e;
    g_ev.device = dev;
  }
  *out = &g_ev;
  return hipSuccess;
}

// The assembly half of msa_route's arguments, as msa_assemble takes them.
msa_assemble_args assembly_of(const msa_route_args &a) {
  msa_assemble_args x = {};
  x.batch = a.batch;
  x.top_k = a.top_k;
  x.n_docs = a.n_docs;
  x.kv_dtype = a.kv_dtype;
  x.n_pool = a.n_pool;
  x.topk_idx = a.topk_idx;
  x.doc_pool_off = a.doc_pool_off;
  x.host_kv = a.host_kv;
  x.host_doc_pool_off = a.host_doc_pool_off;
  x.n_kv_heads = a.n_kv_heads;
  x.head_dim = a.head_dim;
  x.mem_cap = a.mem_cap;
  x.append = a.append;
  x.gather_mode = a.gather_mode;
  x.mem_kv = a.mem_kv;
  x.mem_len = a.mem_len;
  x.host_topk_idx = a.host_topk_idx;
  x.host_mem_len = a.host_mem_len;
  x.host_mem_docs = a.host_mem_docs;
  x.copy_stream = a.copy_stream;
  return x;
}

// Checks of the assembly arguments (msa_route with assembly, msa_assemble);
// the kernel mode also needs host_kv's device mapping, returned in *host_kv_dev.
int check_assembly(const char *who, const msa_assemble_args &x, void **host_kv_dev) {
  const bool kernel_gather = x.gather_mode == MSA_GATHER_KERNEL;
  if (x.gather_mode != MSA_GATHER_COPIES && !kernel_gather)
    return fail(MSA_ERR_INVALID_ARG, "%s: bad gather_mode %d", who, x.gather_mode);
  if (!x.host_doc_pool_off || !x.mem_kv || !x.mem_len)
    return fail(MSA_ERR_INVALID_ARG, "%s: assembly needs host_doc_pool_off, mem_kv and mem_len", who);
  if (!kernel_gather && (!x.host_topk_idx || !x.host_mem_len))
    return fail(MSA_ERR_INVALID_ARG, "%s: copy assembly needs host_topk_idx and host_mem_len", who);
  if (!dtype_ok(x.kv_dtype)) return fail(MSA_ERR_INVALID_ARG, "%s: bad kv_dtype %d", who, x.kv_dtype);
  if (x.n_kv_heads < 1 || x.head_dim < 1 || x.mem_cap < 0)
    return fail(MSA_ERR_INVALID_ARG, "%s: assembly needs n_kv_heads, head_dim >= 1, mem_cap >= 0", who);
  if (x.append && !kernel_gather) {
    for (int b = 0; b < x.batch; ++b)
      if (x.host_mem_len[b] < 0 || x.host_mem_len[b] > x.mem_cap)
        return fail(MSA_ERR_INVALID_ARG, "%s: host_mem_len[%d] = %d outside [0, mem_cap]", who, b, x.host_mem_len[b]);
  }
  *host_kv_dev = nullptr;
  if (kernel_gather) {
    const size_t row_bytes = 2 * (size_t)x.n_kv_heads * x.head_dim * elt_size(x.kv_dtype);
    if (!aligned16(x.host_kv) || !aligned16(x.mem_kv) || row_bytes % 16 != 0)
      return fail(MSA_ERR_INVALID_ARG, "%s: kernel assembly needs 16-byte aligned host_kv, mem_kv and rows", who);
    if (hipHostGetDevicePointer(host_kv_dev, const_cast<void *>(x.host_kv), 0) != hipSuccess || !*host_kv_dev) {
      (void)hipGetLastError();
      return fail(MSA_ERR_INVALID_ARG, "%s: host_kv is not device-mapped pinned memory", who);
    }
  }
  return MSA_OK;
}

// Host-driven assembly: the top-k ids to the host (after the work queued on
// s), then one hipMemcpyAsync per document on the copy stream, and s waits
// for the copies.  Blocks the calling thread until the ids have landed.
int copy_assembly(const char *who, const msa_assemble_args &x, hipStream_t s) {
  ThreadEvents *ev = nullptr;
  hipError_t e;
  if ((e = thread_events(&ev)) != hipSuccess) return fail(MSA_ERR_HIP, "%s events: %s", who, hipGetErrorString(e));
  const size_t idx_bytes = sizeof(int32_t) * (size_t)x.batch * x.top_k;
  if ((e = hipMemcpyAsync(x.host_topk_idx, x.topk_idx, idx_bytes, hipMemcpyDeviceToHost, s)) != hipSuccess)
    return fail(MSA_ERR_HIP, "%s top-k to host: %s", who, hipGetErrorString(e));
  if ((e = hipEventRecord(ev->topk, s)) != hipSuccess)
    return fail(MSA_ERR_HIP, "%s event record: %s", who, hipGetErrorString(e));
  if ((e = hipEventSynchronize(ev->topk)) != hipSuccess)
    return fail(MSA_ERR_HIP, "%s wait for top-k: %s", who, hipGetErrorString(e));

  hipStream_t cs = reinterpret_cast<hipStream_t>(x.copy_stream);
  const size_t row_bytes = 2 * (size_t)x.n_kv_heads * x.head_dim * elt_size(x.kv_dtype);
  const char *src = reinterpret_cast<const char *>(x.host_kv);
  char *dst = reinterpret_cast<char *>(x.mem_kv);
  const int64_t *off = x.host_doc_pool_off;
  for (int b = 0; b < x.batch; ++b) {
    int64_t len = x.append ? x.host_mem_len[b] : 0;
    int taken = 0;
    for (int r = 0; r < x.top_k; ++r) {
      const int32_t d = x.host_topk_idx[(size_t)b * x.top_k + r];
      if (d < 0 || d >= x.n_docs) break;
      const int64_t r0 = off[d], r1 = off[d + 1];
      if (r0 < 0 || r1 < r0 || r1 > x.n_pool) break;
      const int64_t rows = r1 - r0;
      if (len + rows > x.mem_cap) break;
      if (rows > 0) {
        e = hipMemcpyAsync(dst + ((size_t)b * x.mem_cap + len) * row_bytes, src + (size_t)r0 * row_bytes,
                           (size_t)rows * row_bytes, hipMemcpyHostToDevice, cs);
        if (e != hipSuccess) return fail(MSA_ERR_HIP, "%s gather copy: %s", who, hipGetErrorString(e));
      }
      len += rows;
      ++taken;
    }
    x.host_mem_len[b] = (int32_t)len;
    if (x.host_mem_docs) x.host_mem_docs[b] = taken;
  }
  if ((e = hipMemcpyAsync(x.mem_len, x.host_mem_len, sizeof(int32_t) * x.batch, hipMemcpyHostToDevice, cs)) !=
      hipSuccess)
    return fail(MSA_ERR_HIP, "%s mem_len copy: %s", who, hipGetErrorString(e));
  if ((e = hipEventRecord(ev->copies, cs)) != hipSuccess)
    return fail(MSA_ERR_HIP, "%s event record: %s", who, hipGetErrorString(e));
  if ((e = hipStreamWaitEvent(s, ev->copies, 0)) != hipSuccess)
    return fail(MSA_ERR_HIP, "%s stream wait: %s", who, hipGetErrorString(e));
  return MSA_OK;
}

}  // namespace

const DeviceInfo &device_info() {
  static DeviceInfo info[64];
  static std::once_flag once[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::call_once(once[dev], [dev] {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess && p.multiProcessorCount > 0)
      info[dev].n_cu = p.multiProcessorCount;
  });
  return info[dev];
}

}  // namespace msa

using namespace msa;

extern "C" {

const char *msa_last_error(void) { return g_err; }

int msa_version(void) { return 100; }

int msa_pool_encode(const msa_pool_args *a, void *stream) {
  if (!a) return fail(MSA_ERR_INVALID_ARG, "msa_pool_encode: args is NULL");
  if (!dtype_ok(a->dtype)) return fail(MSA_ERR_INVALID_ARG, "msa_pool_encode: bad dtype %d", a->dtype);
  if (a->n_docs < 1 || a->n_tokens < a->n_docs || a->n_pool < a->n_docs || a->pool_size < 1 ||
      a->n_kv_heads < 1 || a->n_router_heads < 1 || !(a->rope_theta > 0.0))
    return fail(MSA_ERR_INVALID_ARG,
                "msa_pool_encode: need n_docs >= 1, n_tokens >= n_docs, n_pool >= n_docs, pool_size >= 1, "
                "heads >= 1, rope_theta > 0");
  if (a->n_pool > a->n_tokens)
    return fail(MSA_ERR_INVALID_ARG, "msa_pool_encode: n_pool (%lld) exceeds n_tokens (%lld)",
                (long long)a->n_pool, (long long)a->n_tokens);
  if (!dim_ok(a->head_dim) || !dim_ok(a->router_dim))
    return fail(MSA_ERR_UNSUPPORTED, "msa_pool_encode: head_dim and router_dim must be 64 or 128");
  if (a->kr_layout != MSA_KR_ROWS && a->kr_layout != MSA_KR_TILED)
    return fail(MSA_ERR_INVALID_ARG, "msa_pool_encode: bad kr_layout %d", a->kr_layout);
  if (a->kr_layout == MSA_KR_TILED && a->dtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "msa_pool_encode: the tiled router-bank layout is bf16 only");
  if (a->kr_row_base < 0)
    return fail(MSA_ERR_INVALID_ARG, "msa_pool_encode: kr_row_base must be >= 0");
  const int vw = a->dtype == MSA_BF16 ? 8 : 4;
  const int tasks = a->n_kv_heads * a->head_dim / 2 / vw + a->n_kv_heads * a->head_dim / vw +
                    a->n_router_heads * a->router_dim / vw;
  if (tasks > 4096) return fail(MSA_ERR_UNSUPPORTED, "msa_pool_encode: too many heads (%d vector tasks)", tasks);
  if (!a->doc_tok_off || !a->doc_pool_off || !a->k || !a->v || !a->kr || !a->kv_pooled || !a->kr_pooled)
    return fail(MSA_ERR_INVALID_ARG, "msa_pool_encode: NULL pointer");
  if (!aligned16(a->k) || !aligned16(a->v) || !aligned16(a->kr) || !aligned16(a->kv_pooled) ||
      !aligned16(a->kr_pooled))
    return fail(MSA_ERR_INVALID_ARG, "msa_pool_encode: tensors must be 16-byte aligned");
  // an output in pinned host memory (the content tier) is written through its
  // device mapping, straight over the host link.  Anything else that is not
  // this device's memory (pageable host memory reports "unregistered") is
  // refused before any launch: the kernel could not store to it.
  msa_pool_args t = *a;
  void *outs[2] = {t.kv_pooled, t.kr_pooled};
  int cur_dev = -1;
  if (hipError_t ge = hipGetDevice(&cur_dev); ge != hipSuccess) return hip_fail(ge, "msa_pool_encode: hipGetDevice");
  for (int i = 0; i < 2; ++i) {
    hipPointerAttribute_t attr;
    const bool known = hipPointerGetAttributes(&attr, outs[i]) == hipSuccess;
    if (!known) (void)hipGetLastError();
    const bool on_device = known && attr.type == hipMemoryTypeDevice && attr.device == cur_dev;
    const bool pinned = known && attr.type == hipMemoryTypeHost;
    if (!on_device && !pinned)
      return fail(MSA_ERR_INVALID_ARG,
                  "msa_pool_encode: %s must be device memory (of the current device) or pinned host memory",
                  i ? "kr_pooled" : "kv_pooled");
    if (pinned) {
      void *dev = nullptr;
      if (hipHostGetDevicePointer(&dev, outs[i], 0) != hipSuccess || !dev || !aligned16(dev)) {
        (void)hipGetLastError();
        return fail(MSA_ERR_INVALID_ARG,
                    "msa_pool_encode: %s must be device memory or pinned host memory (no device mapping)",
                    i ? "kr_pooled" : "kv_pooled");
      }
      outs[i] = dev;
    }
  }
  t.kv_pooled = outs[0];
  t.kr_pooled = outs[1];
  hipError_t e = launch_pool(t, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e, "msa_pool_encode launch");
}

size_t msa_route_workspace_bytes(int32_t dtype, int32_t batch, int32_t q_tokens, int32_t n_router_heads,
                                 int32_t router_dim, int32_t n_docs, int64_t n_pool, int32_t top_k) {
  if (!dtype_ok(dtype) || batch < 1 || q_tokens < 1 || n_router_heads < 1 || router_dim < 1 || n_docs < 1 ||
      n_pool < n_docs || top_k < 1)
    return 0;
  return route_ws_layout(dtype, batch, q_tokens, n_router_heads, router_dim, n_docs, n_pool, top_k, nullptr,
                         nullptr);
}

size_t msa_doc_map_bytes(int64_t n_pool) {
  if (n_pool < 1) return 0;
  return doc_map_bits_offset(n_pool) + (((size_t)4 * (size_t)((n_pool + 15) / 16) + 255) & ~(size_t)255);
}

int msa_doc_map(const int64_t *doc_pool_off, int32_t n_docs, int64_t n_pool, void *doc_map, size_t doc_map_bytes,
                void *stream) {
  if (!doc_pool_off || !doc_map) return fail(MSA_ERR_INVALID_ARG, "msa_doc_map: NULL pointer");
  if (n_docs < 1 || n_pool < n_docs || n_docs > 0x7ffffffe)
    return fail(MSA_ERR_INVALID_ARG, "msa_doc_map: need 1 <= n_docs <= n_pool");
  if (!aligned16(doc_map) || doc_map_bytes < msa_doc_map_bytes(n_pool))
    return fail(MSA_ERR_INVALID_ARG, "msa_doc_map: doc_map needs %zu bytes (16-byte aligned), got %zu",
                msa_doc_map_bytes(n_pool), doc_map_bytes);
  char *m = reinterpret_cast<char *>(doc_map);
  const hipError_t e = launch_doc_map(doc_pool_off, n_docs, n_pool, reinterpret_cast<int32_t *>(m),
                                      reinterpret_cast<uint32_t *>(m + doc_map_bits_offset(n_pool)),
                                      reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e, "msa_doc_map launch");
}

int msa_route(const msa_route_args *a, void *stream) {
  if (!a) return fail(MSA_ERR_INVALID_ARG, "msa_route: args is NULL");
  if (!dtype_ok(a->dtype)) return fail(MSA_ERR_INVALID_ARG, "msa_route: bad dtype %d", a->dtype);
  if (a->batch < 1 || a->q_tokens < 1 || a->n_docs < 1 || a->n_pool < a->n_docs)
    return fail(MSA_ERR_INVALID_ARG, "msa_route: need batch, q_tokens, n_docs >= 1 and n_pool >= n_docs");
  if (a->n_docs > 0x7ffffffe) return fail(MSA_ERR_UNSUPPORTED, "msa_route: too many documents");
  if (a->top_k < 1 || a->top_k > a->n_docs)
    return fail(MSA_ERR_INVALID_ARG, "msa_route: need 1 <= top_k (%d) <= n_docs (%d)", a->top_k, a->n_docs);
  if (a->top_k > kMaxTopK) return fail(MSA_ERR_UNSUPPORTED, "msa_route: top_k > %d", kMaxTopK);
  if (!route_shape_supported(a->n_router_heads, a->router_dim))
    return fail(MSA_ERR_UNSUPPORTED,
                "msa_route: router_dim must be 64 or 128 and n_router_heads a power of two dividing 64 with "
                "n_router_heads * router_dim <= 2048");
  if (a->kr_layout != MSA_KR_ROWS && a->kr_layout != MSA_KR_TILED)
    return fail(MSA_ERR_INVALID_ARG, "msa_route: bad kr_layout %d", a->kr_layout);
  if (a->kr_layout == MSA_KR_TILED && (a->dtype != MSA_BF16 || !mfma_shape(a->n_router_heads, a->router_dim)))
    return fail(MSA_ERR_UNSUPPORTED, "msa_route: the tiled router-bank layout needs bf16 and a matrix-core "
                                     "router shape (dr 64 with Hr <= 16, or dr 128 with Hr <= 8)");
  if (!a->qr || !a->kr_pooled || !a->doc_pool_off || !a->doc_scores || !a->topk_idx || !a->topk_score)
    return fail(MSA_ERR_INVALID_ARG, "msa_route: NULL pointer");
  if (!aligned16(a->qr) || !aligned16(a->kr_pooled))
    return fail(MSA_ERR_INVALID_ARG, "msa_route: qr and kr_pooled must be 16-byte aligned");
  const size_t need = route_ws_layout(a->dtype, a->batch, a->q_tokens, a->n_router_heads, a->router_dim,
                                      a->n_docs, a->n_pool, a->top_k, nullptr, nullptr);
  if (!a->workspace || a->workspace_bytes < need || !aligned16(a->workspace))
    return fail(MSA_ERR_WORKSPACE, "msa_route: workspace needs %zu bytes (16-byte aligned), got %zu", need,
                a->workspace ? a->workspace_bytes : (size_t)0);
  if (a->doc_map && !aligned16(a->doc_map))
    return fail(MSA_ERR_INVALID_ARG, "msa_route: doc_map must be 16-byte aligned");
  const bool assemble = a->host_kv != nullptr;
  const bool kernel_gather = assemble && a->gather_mode == MSA_GATHER_KERNEL;
  void *host_kv_dev = nullptr;
  const msa_assemble_args x = assembly_of(*a);
  if (assemble) {
    const int st = check_assembly("msa_route", x, &host_kv_dev);
    if (st != MSA_OK) return st;
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  RouteWs ws;
  route_ws_layout(a->dtype, a->batch, a->q_tokens, a->n_router_heads, a->router_dim, a->n_docs, a->n_pool,
                  a->top_k, a->workspace, &ws);
  if (a->doc_map) {
    char *m = reinterpret_cast<char *>(const_cast<void *>(a->doc_map));
    ws.tile_doc = reinterpret_cast<int32_t *>(m);
    ws.tile_bits = reinterpret_cast<uint32_t *>(m + doc_map_bits_offset(a->n_pool));
    ws.map_given = 1;
  }
  hipError_t e = launch_route(*a, ws, host_kv_dev, s);
  if (e != hipSuccess) return hip_fail(e, "msa_route launch");
  if (!assemble || kernel_gather) return MSA_OK;
  return copy_assembly("msa_route", x, s);
}

size_t msa_assemble_workspace_bytes(int32_t batch, int32_t top_k) {
  if (batch < 1 || top_k < 1) return 0;
  return ((size_t)batch * top_k * sizeof(GatherPlan) + 255) & ~(size_t)255;
}

int msa_assemble(const msa_assemble_args *a, void *stream) {
  if (!a) return fail(MSA_ERR_INVALID_ARG, "msa_assemble: args is NULL");
  if (a->batch < 1 || a->n_docs < 1 || a->n_pool < a->n_docs || !a->topk_idx || !a->host_kv)
    return fail(MSA_ERR_INVALID_ARG, "msa_assemble: need batch, n_docs >= 1, n_pool >= n_docs, topk_idx, host_kv");
  if (a->n_docs > 0x7ffffffe) return fail(MSA_ERR_UNSUPPORTED, "msa_assemble: too many documents");
  if (a->top_k < 1 || a->top_k > a->n_docs)
    return fail(MSA_ERR_INVALID_ARG, "msa_assemble: need 1 <= top_k (%d) <= n_docs (%d)", a->top_k, a->n_docs);
  if (a->top_k > kMaxTopK) return fail(MSA_ERR_UNSUPPORTED, "msa_assemble: top_k > %d", kMaxTopK);
  void *host_kv_dev = nullptr;
  const int st = check_assembly("msa_assemble", *a, &host_kv_dev);
  if (st != MSA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a->gather_mode == MSA_GATHER_COPIES) return copy_assembly("msa_assemble", *a, s);
  const size_t need = msa_assemble_workspace_bytes(a->batch, a->top_k);
  if (!a->doc_pool_off) return fail(MSA_ERR_INVALID_ARG, "msa_assemble: kernel assembly needs doc_pool_off");
  if (!a->workspace || a->workspace_bytes < need || !aligned16(a->workspace))
    return fail(MSA_ERR_WORKSPACE, "msa_assemble: workspace needs %zu bytes (16-byte aligned), got %zu", need,
                a->workspace ? a->workspace_bytes : (size_t)0);
  const hipError_t e = launch_assemble(*a, reinterpret_cast<GatherPlan *>(a->workspace), host_kv_dev, s);
  return e == hipSuccess ? MSA_OK : hip_fail(e, "msa_assemble launch");
}

// bf16 decode runs the block-attention kernel with one query token (fp32
// keeps the split-KV VALU kernel); the KV head count is not an argument
// here, so the size covers every Hkv that divides Hq.
size_t msa_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t head_dim, int32_t mem_cap,
                                  int32_t local_cap) {
  if (batch < 1 || n_q_heads < 1 || !dim_ok(head_dim) || mem_cap < 0 || local_cap < 0) return 0;
  size_t need = decode_ws_layout(batch, n_q_heads, head_dim, mem_cap, local_cap, nullptr, nullptr, nullptr, nullptr);
  if ((int64_t)mem_cap + local_cap <= (1LL << 30))
    for (int32_t hkv = 1; hkv <= n_q_heads; ++hkv)
      if (n_q_heads % hkv == 0 && n_q_heads / hkv <= 16)
        need = std::max(need, attend_ws_layout(batch, 1, n_q_heads, hkv, head_dim, mem_cap, local_cap, nullptr,
                                               nullptr));
  return need;
}

}  // extern "C"

namespace {

// Device scratch of msa_sparse_decode_noalloc: the split partials that
// msa_sparse_decode keeps in the caller's workspace.  Every device the
// library runs on holds its own copy for the life of the process; calls on
// one device share it.
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

// The device address of `scratch` on the current device, looked up once per
// device while that device is current.  In host code `scratch` names a host
// stand-in, never the device array, so only this address reaches a kernel.
hipError_t scratch_address(void **out) {
  static void *addr[64];
  static hipError_t err[64];
  static std::once_flag once[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    err[dev] = hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(scratch));
    if (err[dev] == hipSuccess && !addr[dev]) err[dev] = hipErrorInvalidSymbol;
  });
  if (err[dev] != hipSuccess) return err[dev];
  *out = addr[dev];
  return hipSuccess;
}

// Shared body of msa_sparse_decode and msa_sparse_decode_noalloc: `ws` holds
// `ws_bytes` bytes for the split partials (the caller's workspace, or the
// static scratch when `noalloc`); `who` names the entry point in messages.
int sparse_decode_with(const char *who, const msa_decode_args *a, void *ws, size_t ws_bytes, bool noalloc,
                       void *stream) {
  if (!a) return fail(MSA_ERR_INVALID_ARG, "%s: args is NULL", who);
  if (!dtype_ok(a->dtype)) return fail(MSA_ERR_INVALID_ARG, "%s: bad dtype %d", who, a->dtype);
  if (a->batch < 1 || a->n_q_heads < 1 || a->n_kv_heads < 1 || a->mem_cap < 0 || a->local_cap < 0 ||
      !(a->rope_theta > 0.0))
    return fail(MSA_ERR_INVALID_ARG, "%s: need batch, heads >= 1, caps >= 0, rope_theta > 0", who);
  if (a->n_q_heads % a->n_kv_heads != 0)
    return fail(MSA_ERR_INVALID_ARG, "%s: n_q_heads (%d) not a multiple of n_kv_heads (%d)", who, a->n_q_heads,
                a->n_kv_heads);
  if (a->n_q_heads / a->n_kv_heads > 8)
    return fail(MSA_ERR_UNSUPPORTED, "%s: more than 8 query heads per KV head", who);
  if (!dim_ok(a->head_dim)) return fail(MSA_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128", who);
  if ((int64_t)a->mem_cap + a->local_cap > (1LL << 30))
    return fail(MSA_ERR_UNSUPPORTED, "%s: context capacity too large", who);
  if (!a->q || !a->mem_len || !a->local_len || !a->pos_offset || !a->out || (a->mem_cap > 0 && !a->mem_kv) ||
      (a->local_cap > 0 && (!a->local_k || !a->local_v)))
    return fail(MSA_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if ((a->mem_kv && !aligned16(a->mem_kv)) || (a->local_k && !aligned16(a->local_k)) ||
      (a->local_v && !aligned16(a->local_v)))
    return fail(MSA_ERR_INVALID_ARG, "%s: K/V tensors must be 16-byte aligned", who);
  if (a->dtype == MSA_BF16 && (!aligned16(a->q) || !aligned16(a->out)))
    return fail(MSA_ERR_INVALID_ARG, "%s: bf16 q and out must be 16-byte aligned", who);
  // bf16: the block-attention kernel with one query token; fp32: split-KV
  size_t need = 0;
  int32_t n_split = 0;
  if (a->dtype == MSA_BF16)
    need = attend_ws_layout(a->batch, 1, a->n_q_heads, a->n_kv_heads, a->head_dim, a->mem_cap, a->local_cap, nullptr,
                            nullptr);
  else
    need = decode_ws_layout(a->batch, a->n_q_heads, a->head_dim, a->mem_cap, a->local_cap, nullptr, nullptr, nullptr,
                            &n_split);
  if (noalloc) {
    if (need > kDecodeScratchBytes)
      return fail(MSA_ERR_WORKSPACE, "%s: this call needs %zu bytes of scratch; the static scratch holds %zu", who,
                  need, kDecodeScratchBytes);
    const hipError_t se = scratch_address(&ws);
    if (se != hipSuccess) return hip_fail(se, "msa_sparse_decode_noalloc: scratch address");
    ws_bytes = kDecodeScratchBytes;
  } else if (!ws || ws_bytes < need || !aligned16(ws)) {
    return fail(MSA_ERR_WORKSPACE, "%s: workspace needs %zu bytes (16-byte aligned), got %zu", who, need,
                ws ? ws_bytes : (size_t)0);
  }
  hipError_t e = hipSuccess;
  if (a->dtype == MSA_BF16) {
    msa_attend_args t = {};
    t.dtype = a->dtype;
    t.batch = a->batch;
    t.q_tokens = 1;
    t.n_q_heads = a->n_q_heads;
    t.n_kv_heads = a->n_kv_heads;
    t.head_dim = a->head_dim;
    t.mem_cap = a->mem_cap;
    t.local_cap = a->local_cap;
    t.q = a->q;
    t.mem_kv = a->mem_kv;
    t.mem_len = a->mem_len;
    t.local_k = a->local_k;
    t.local_v = a->local_v;
    t.local_len = a->local_len;
    t.pos_offset = a->pos_offset;
    t.rope_theta = a->rope_theta;
    t.softmax_scale = a->softmax_scale;
    t.out = a->out;
    t.lse = a->lse;
    t.prof_event_begin = a->prof_event_begin;
    t.prof_event_end = a->prof_event_end;
    AttendWs aws;
    attend_ws_layout(t.batch, 1, t.n_q_heads, t.n_kv_heads, t.head_dim, t.mem_cap, t.local_cap, ws, &aws);
    e = launch_attend(t, aws, reinterpret_cast<hipStream_t>(stream));
  } else {
    float *part_acc = nullptr, *part_ml = nullptr;
    decode_ws_layout(a->batch, a->n_q_heads, a->head_dim, a->mem_cap, a->local_cap, ws, &part_acc, &part_ml,
                     &n_split);
    e = launch_decode(*a, part_acc, part_ml, n_split, reinterpret_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "%s launch: %s (%d)", who, hipGetErrorString(e), (int)e);
  return MSA_OK;
}

}  // namespace

extern "C" {

int msa_sparse_decode(const msa_decode_args *a, void *stream) {
  return sparse_decode_with("msa_sparse_decode", a, a ? a->workspace : nullptr, a ? a->workspace_bytes : 0, false,
                            stream);
}

int msa_sparse_decode_noalloc(const msa_decode_args *a, void *stream) {
  return sparse_decode_with("msa_sparse_decode_noalloc", a, nullptr, 0, true, stream);
}

size_t msa_attend_workspace_bytes(int32_t batch, int32_t q_tokens, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t head_dim, int32_t mem_cap, int32_t local_cap) {
  if (batch < 1 || q_tokens < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0 ||
      n_q_heads / n_kv_heads > 16 || !dim_ok(head_dim) || mem_cap < 0 || local_cap < 0 ||
      (int64_t)mem_cap + local_cap > (1LL << 30))
    return 0;
  return attend_ws_layout(batch, q_tokens, n_q_heads, n_kv_heads, head_dim, mem_cap, local_cap, nullptr, nullptr);
}

int msa_sparse_attend(const msa_attend_args *a, void *stream) {
  if (!a) return fail(MSA_ERR_INVALID_ARG, "msa_sparse_attend: args is NULL");
  if (!dtype_ok(a->dtype)) return fail(MSA_ERR_INVALID_ARG, "msa_sparse_attend: bad dtype %d", a->dtype);
  if (a->dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_attend: bf16 only");
  if (a->batch < 1 || a->q_tokens < 1 || a->n_q_heads < 1 || a->n_kv_heads < 1 || a->mem_cap < 0 ||
      a->local_cap < 0 || !(a->rope_theta > 0.0))
    return fail(MSA_ERR_INVALID_ARG,
                "msa_sparse_attend: need batch, q_tokens, heads >= 1, caps >= 0, rope_theta > 0");
  if (a->n_q_heads % a->n_kv_heads != 0)
    return fail(MSA_ERR_INVALID_ARG, "msa_sparse_attend: n_q_heads (%d) not a multiple of n_kv_heads (%d)",
                a->n_q_heads, a->n_kv_heads);
  if (a->n_q_heads / a->n_kv_heads > 16)
    return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_attend: more than 16 query heads per KV head");
  if (!dim_ok(a->head_dim)) return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_attend: head_dim must be 64 or 128");
  if ((int64_t)a->mem_cap + a->local_cap > (1LL << 30))
    return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_attend: context capacity too large");
  if (!a->q || !a->mem_len || !a->local_len || !a->pos_offset || !a->out || (a->mem_cap > 0 && !a->mem_kv) ||
      (a->local_cap > 0 && (!a->local_k || !a->local_v)))
    return fail(MSA_ERR_INVALID_ARG, "msa_sparse_attend: NULL pointer");
  if (!aligned16(a->q) || !aligned16(a->out) || (a->mem_kv && !aligned16(a->mem_kv)) ||
      (a->local_k && !aligned16(a->local_k)) || (a->local_v && !aligned16(a->local_v)))
    return fail(MSA_ERR_INVALID_ARG, "msa_sparse_attend: q, out and K/V tensors must be 16-byte aligned");
  const size_t need = attend_ws_layout(a->batch, a->q_tokens, a->n_q_heads, a->n_kv_heads, a->head_dim,
                                       a->mem_cap, a->local_cap, nullptr, nullptr);
  if (!a->workspace || a->workspace_bytes < need || !aligned16(a->workspace))
    return fail(MSA_ERR_WORKSPACE, "msa_sparse_attend: workspace needs %zu bytes (16-byte aligned), got %zu",
                need, a->workspace ? a->workspace_bytes : (size_t)0);
  AttendWs aws;
  attend_ws_layout(a->batch, a->q_tokens, a->n_q_heads, a->n_kv_heads, a->head_dim, a->mem_cap, a->local_cap,
                   a->workspace, &aws);
  hipError_t e = launch_attend(*a, aws, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e, "msa_sparse_attend launch");
}

}  // extern "C"
