/*
 * gp_probe.h - HBM bandwidth probes exported by libgrowpage.so.
 *
 * Measurement helpers, not part of the boundary event: they give the
 * practical HBM ceilings the event's kernels are compared with beside the
 * device's published peak.  The read probe has the shape of the demand
 * kernel's key stream (reads only), the copy probe that of the compaction
 * (every byte read once and written once).  Each wave moves whole 16 KiB
 * blocks with 16-byte non-temporal loads.
 *
 * Both calls enqueue one kernel on `stream` (a hipStream_t, NULL for the
 * null stream) and return the hipError_t of the launch as an int (0 on
 * success).  `bytes` must be a positive multiple of GP_PROBE_BLOCK_BYTES and
 * the pointers 16-byte aligned device addresses, else hipErrorInvalidValue is
 * returned and nothing is enqueued.  The caller owns every buffer.
 */
#ifndef GP_PROBE_H
#define GP_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GP_PROBE_BLOCK_BYTES ((size_t)16384)

/* Reads `bytes` of src once; writes at most one word to sink (device, 4
 * bytes), so that the loads cannot be dropped. */
int gp_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Copies `bytes` from src to dst (device, not overlapping). */
int gp_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GP_PROBE_H */
