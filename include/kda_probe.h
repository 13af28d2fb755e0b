/*
 * kda_probe.h -- measurement-only C ABI (libkda_probe.so): HBM streaming
 * probes that state the achievable ceiling of the decode step's access
 * contract and calibrate the profiler's byte counters.  Not part of the KDA
 * decode step.
 *
 * Both take DEVICE pointers the caller owns (16-byte aligned), enqueue one
 * kernel on `stream` (a hipStream_t; NULL = default stream) and return
 * 0 = enqueued, 1 = NULL pointer, 4 = misaligned, 5 = src and dst overlap,
 * 6 = bytes is 0, not a multiple of 8192, or too large, 7 = launch refused.
 * Nothing is allocated, freed or synchronised.
 */
#ifndef KDA_PROBE_H
#define KDA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In place: buf[i] = buf[i] * scale over `bytes` bytes of f32, each 16-byte
 * chunk read once and written once (the state update's read-once/write-once
 * contract): non-temporal loads, non-temporal agent-scope stores, as the
 * decode kernel's state accesses on large grids.  HBM traffic: 2 * bytes. */
int kda_probe_rmw(void *buf, size_t bytes, float scale, void *stream);

/* dst = src over `bytes` bytes, 16-byte accesses with the same cache policy
 * as kda_probe_rmw; the buffers must not overlap.  HBM traffic: 2 * bytes. */
int kda_probe_copy(const void *src, void *dst, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_PROBE_H */
