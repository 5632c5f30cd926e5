/*
 * pa_probe.h - measurement kernel: the achievable HBM read bandwidth on this
 * GPU, as a reference for the decode kernels' roofline (C ABI).
 *
 * pa_probe_stream_read reads `bytes` bytes of device memory at `buf` once,
 * front to back, with 16-byte non-temporal lane loads (the decode kernels' load
 * width and cache hint), spread evenly over `num_waves` single-wave work-groups
 * that keep several loads in flight each. Nothing is computed from the data but
 * an XOR of all of it per work-group, stored to sink[work-group] (uint32, so the
 * loads are not removed); callers only time the kernel. `buf` must be 16-byte
 * aligned, bytes a multiple of 16 and num_waves in [1, 65536]; sink holds
 * num_waves uint32. Enqueued on `stream` (NULL = the default stream); the
 * profiling hook of pa.h (pa_set_kernel_timing_events) applies to it. Returns
 * PA_ERR_NULL_POINTER / PA_ERR_INVALID_ARGUMENT for bad arguments, PA_ERR_HIP
 * if the launch fails.
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

pa_status pa_probe_stream_read(const void* buf, size_t bytes, int32_t num_waves, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
