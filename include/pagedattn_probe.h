/*
 * pagedattn_probe.h -- measurement kernels shipped with the paged-attention
 * library. They compute nothing of attention; the benchmark uses them to
 * put the attention kernels' bandwidth next to what the device delivers.
 * Pointers are device pointers owned by the caller; calls only enqueue on
 * `stream` (hipStream_t as void*, NULL = null stream). Return PA_OK or a
 * negative pa_status (pagedattn.h).
 */
#ifndef PAGEDATTN_PROBE_H
#define PAGEDATTN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "pagedattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16, 16-byte aligned) of `buf` once with
 * nontemporal 16-byte loads (the load kind the attention kernels use for
 * K/V), one wave per SIMD, each wave reading whole contiguous 8 KB chunks:
 * the fastest plain read of this device, an upper bound for the gathers of
 * the attention kernels. `sink` receives at most a few words so the loads
 * cannot be optimized away (it needs room for 8 words per compute unit). */
int pa_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Copy `bytes` (a multiple of 16, 16-byte aligned) from src to dst: a plain
 * kernel of known traffic (bytes read + bytes written) for calibrating the
 * profiler's byte counters. */
int pa_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_PROBE_H */
