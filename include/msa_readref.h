/* libmsa_readref: a reference streaming-read kernel, for measurement only.
 *
 * It reads device memory in the access pattern of the route bank scan over
 * the tiled router bank at 8 heads x 128 bf16 (2 KiB rows, 16-row tiles of
 * 32 KiB): one wave per tile, 32 loads of 1 KiB of contiguous memory each.
 * It computes nothing but an XOR fold, so its time is the read ceiling that
 * the scan can be compared with on the same device and buffer.  Not part of
 * the method: no passage defines it.
 *
 * msa_ref_read_tiles
 *   buf          device memory, 16-byte aligned, n_bytes readable
 *   n_bytes      > 0, a multiple of 32768 (whole tiles)
 *   grid         >= 1 workgroups of 256 threads (4 waves); tile t is read by
 *                wave (t mod 4*grid) of the grid-stride walk
 *   nontemporal  != 0: non-temporal loads (as the scan uses on this layout)
 *   sink         device, grid*256 entries of 16 bytes, written: the XOR of
 *                all entries equals the XOR of all 16-byte vectors of buf
 *   stream       hipStream_t (NULL: the null stream)
 *   ev_begin/end optional hipEvent_t pair attached to the dispatch
 *                (hipExtLaunchKernel); NULL to skip
 * Returns 0; -1 for invalid arguments (nothing enqueued); -5 when the launch
 * fails.  The library allocates nothing.
 */
#ifndef MSA_READREF_H
#define MSA_READREF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int msa_ref_read_tiles(const void *buf, int64_t n_bytes, int32_t grid, int32_t nontemporal, void *sink,
                       void *stream, void *ev_begin, void *ev_end);

#ifdef __cplusplus
}
#endif

#endif
