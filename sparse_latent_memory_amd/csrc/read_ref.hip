// Reference streaming read in the tiled router bank's pattern (measurement
// only; see include/msa_readref.h).  Each wave walks 32 KiB tiles
// grid-stride; lane l reads 16-byte vector l of each of the tile's 32
// contiguous KiB, eight loads in flight, and XOR-folds them.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/msa_readref.h"

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kTileVecs = 2048;   // 32 KiB
constexpr int kInflight = 8;

template <bool NT>
__global__ __launch_bounds__(256) void read_tiles_kernel(const u32x4 *__restrict__ p, int64_t n_tiles,
                                                         u32x4 *__restrict__ sink) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n_waves = (int64_t)gridDim.x * 4;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t < n_tiles; t += n_waves) {
    const u32x4 *rp = p + t * kTileVecs + lane;
#pragma unroll
    for (int s0 = 0; s0 < kTileVecs / 64; s0 += kInflight) {
      u32x4 v[kInflight];
#pragma unroll
      for (int u = 0; u < kInflight; ++u) {
        const u32x4 *a = rp + 64 * (s0 + u);
        v[u] = NT ? __builtin_nontemporal_load(a) : *a;
      }
#pragma unroll
      for (int u = 0; u < kInflight; ++u) acc ^= v[u];
    }
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" int msa_ref_read_tiles(const void *buf, int64_t n_bytes, int32_t grid, int32_t nontemporal, void *sink,
                                  void *stream, void *ev_begin, void *ev_end) {
  if (!buf || !sink || n_bytes <= 0 || n_bytes % (kTileVecs * 16) != 0 || grid < 1 ||
      (reinterpret_cast<uintptr_t>(buf) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 15) != 0)
    return -1;
  const int64_t n_tiles = n_bytes / (kTileVecs * 16);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t a = reinterpret_cast<hipEvent_t>(ev_begin), b = reinterpret_cast<hipEvent_t>(ev_end);
  const u32x4 *p = reinterpret_cast<const u32x4 *>(buf);
  u32x4 *o = reinterpret_cast<u32x4 *>(sink);
  if (nontemporal)
    hipExtLaunchKernelGGL((read_tiles_kernel<true>), dim3((unsigned)grid), dim3(256), 0, s, a, b, 0, p, n_tiles, o);
  else
    hipExtLaunchKernelGGL((read_tiles_kernel<false>), dim3((unsigned)grid), dim3(256), 0, s, a, b, 0, p, n_tiles, o);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
