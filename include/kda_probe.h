/*
 * kda_probe.h -- measurement-only C ABI (libkda_probe.so): HBM streaming
 * probes that state the achievable ceiling of the decode step's access
 * contract and calibrate the profiler's byte counters.  Not part of the KDA
 * decode step.
 *
 * All take DEVICE pointers the caller owns (16-byte aligned), enqueue one
 * kernel on `stream` (a hipStream_t; NULL = default stream) and return
 * 0 = enqueued, 1 = NULL pointer, 4 = misaligned, 5 = src and dst overlap
 * (or, in place, differ), 6 = bytes is 0, not a multiple of the tile, or too
 * large, or an unknown shape, 7 = launch refused.  Nothing is allocated,
 * freed or synchronised.
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

/* The ceiling sweep: one launch over `bytes` bytes in 16-byte chunks.
 *   kind             0 in place (dst must equal src: read once, written once),
 *                    1 read only (src; dst unused), 2 write only (dst is
 *                    filled with `scale`; src unused), 3 copy (no overlap)
 *   threads          256, 512 or 1024 per workgroup
 *   chunks_per_lane  1, 2 or 4: a tile is threads * chunks_per_lane chunks;
 *                    a lane issues all its loads before its first store
 *   persistent       0: one workgroup per tile; 1: a grid of every wave slot
 *                    of the device (32 waves per CU) walks the tiles
 * bytes must be a multiple of the tile (threads * chunks_per_lane * 16).
 * Same cache policy as kda_probe_rmw.  HBM traffic: 2 * bytes for kinds 0
 * and 3, bytes for kinds 1 and 2.  In place multiplies by `scale`. */
int kda_probe_stream(int kind, int threads, int chunks_per_lane, int persistent, const void *src, void *dst,
                     size_t bytes, float scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_PROBE_H */
