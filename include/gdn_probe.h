/*
 * gdn_probe.h -- measurement probes in libgdn (AMD Instinct MI355X, gfx950):
 * what this GPU attains on plain matrix-core work and on a plain device
 * memory stream, so that the library's kernels can be set beside a measured
 * attainable rate as well as the datasheet peaks.  Neither call takes part in
 * the Gated DeltaNet computation.
 *
 * Conventions are those of gdn.h: device pointers owned by the caller, work
 * enqueued on `stream` (a hipStream_t, NULL for the default stream), host-side
 * argument checks returning a gdn_status, message in gdn_last_error().
 */
#ifndef GDN_PROBE_H
#define GDN_PROBE_H

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * gdn_probe_mfma -- matrix-core rate.  n_workgroups workgroups of four waves;
 * each wave runs `iters` rounds of four independent 32x32x16 bf16 MFMAs
 * (fp32 accumulators) on register operands whose elements are all 1.0:
 * n_workgroups * 4 * iters * 4 * 32768 flops.  sink: device fp32 array of
 * n_workgroups * 256 entries; entry i receives the sum of thread i's 64
 * accumulator elements, which is exactly 4 * 16 * 16 * iters = 1024 * iters.
 * Errors: GDN_ERR_SHAPE unless 1 <= n_workgroups <= 2^20 and iters is a
 * multiple of 4 in [4, 65536]; GDN_ERR_NULL without sink; GDN_ERR_ALIGN unless sink is
 * 4-byte aligned; GDN_ERR_DEVICE on a launch failure.
 */
gdn_status gdn_probe_mfma(int32_t n_workgroups, int32_t iters, float* sink, void* stream);

/*
 * gdn_probe_copy -- device-memory stream: copies `bytes` from src to dst with
 * 16-byte loads, eight per thread in flight (bytes read + bytes written).
 * bytes must be a multiple of 32768 and below 2^46; src and dst 16-byte
 * aligned and not overlapping.  Errors: GDN_ERR_SHAPE, GDN_ERR_NULL,
 * GDN_ERR_ALIGN, GDN_ERR_DEVICE as above.  bytes = 0 does nothing.
 */
gdn_status gdn_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_PROBE_H */
