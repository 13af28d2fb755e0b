// kda_probe.hip -- HBM streaming probes for measurement (libkda_probe.so).
//
// Not part of the decode step.  They state what a plain stream of the same
// access contract achieves on the device, and give rocprofv3's byte counters
// a kernel of exactly known traffic to be calibrated against:
//  * rmw:  in place, every 16-byte chunk read once and written once
//          (the state update's contract), 512 threads per workgroup, one
//          chunk per lane;
//  * copy: 16-byte chunks from src to dst, same shape;
//  * stream: the ceiling sweep -- in place, read only, write only or copy,
//          256 / 512 / 1024 threads per workgroup, 1, 2 or 4 chunks per lane
//          (all loads of a lane issued before its first store), and either
//          one workgroup per tile or a persistent grid that walks the tiles.
// Loads are non-temporal; stores are non-temporal with agent scope (sc1), the
// fastest of the cache-policy combinations measured on MI355X (an in-place
// stream over 128 MiB: 6.56 TB/s; 6.41 TB/s with non-temporal stores alone;
// 5.6-5.7 TB/s with a plain load or a plain store) and the policy of the
// decode kernel's state stores on large grids.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda_probe.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 512;
constexpr size_t kChunk = 16;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// `bytes` starting at base as a raw buffer (stride 0, 32-bit data format):
// hipcc exposes the agent-scope cache-policy bit on buffer accesses only.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(void* base) {
    return span_rsrc(base, (int)(kThreads * kChunk));
}

// a 16-byte chunk at byte offset off of a buffer, agent scope (sc1 = 16) +
// non-temporal (nt = 2)
__device__ __forceinline__ void store_sc1_nt(__amdgpu_buffer_rsrc_t rs, int off, const f32x4& v) {
    const u32x4 r = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(r, rs, off, 0, 16 | 2);
}

__global__ __launch_bounds__(kThreads) void rmw_kernel(f32x4* __restrict__ a, float scale) {
    f32x4* const blk = a + (size_t)blockIdx.x * kThreads;
    const f32x4 v = __builtin_nontemporal_load(blk + threadIdx.x) * scale;
    store_sc1_nt(block_rsrc(blk), (int)(threadIdx.x * kChunk), v);
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst) {
    const size_t b = (size_t)blockIdx.x * kThreads;
    store_sc1_nt(block_rsrc(dst + b), (int)(threadIdx.x * kChunk), __builtin_nontemporal_load(src + b + threadIdx.x));
}

// The sweep.  A tile is NT * APL chunks (contiguous); access a of a lane is
// chunk a * NT + tid of the tile, so every access instruction of the
// workgroup covers NT consecutive chunks.  KIND 0: in place (dst == src),
// 1: read only, 2: write only, 3: copy.  PERSIST: the grid walks the tiles
// with a stride of its own size; otherwise one workgroup per tile.
template <int NT, int APL, int KIND, bool PERSIST>
__global__ __launch_bounds__(NT) void stream_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                    unsigned tiles, float scale) {
    constexpr unsigned TILE = (unsigned)NT * APL;
    const unsigned stride = PERSIST ? gridDim.x : tiles;
    for (unsigned t = blockIdx.x; t < tiles; t += stride) {
        const size_t base = (size_t)t * TILE;
        f32x4 v[APL];
        if constexpr (KIND != 2) {
#pragma unroll
            for (int a = 0; a < APL; ++a) v[a] = __builtin_nontemporal_load(src + base + a * NT + threadIdx.x);
        }
        const auto rs = span_rsrc(dst + base, (int)(TILE * kChunk));
        if constexpr (KIND == 1) {
            // read only: the sum is stored only if it equals a value the
            // probe's data (finite, non-negative) never sums to, which keeps
            // the loads without writing
            f32x4 s = v[0];
#pragma unroll
            for (int a = 1; a < APL; ++a) s += v[a];
            if (s.x == -1.0f) store_sc1_nt(rs, (int)(threadIdx.x * kChunk), s);
        } else {
#pragma unroll
            for (int a = 0; a < APL; ++a) {
                const f32x4 w = KIND == 0 ? v[a] * scale : (KIND == 3 ? v[a] : f32x4{scale, scale, scale, scale});
                store_sc1_nt(rs, (int)((a * NT + threadIdx.x) * kChunk), w);
            }
        }
    }
}

bool bad_size(size_t bytes) {
    return bytes == 0 || bytes % (kThreads * kChunk) != 0 || bytes / (kThreads * kChunk) > 0x7fffffffu;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

template <int NT, int APL, int KIND>
const void* pick_kernel(bool persistent) {
    return persistent ? reinterpret_cast<const void*>(&stream_kernel<NT, APL, KIND, true>)
                      : reinterpret_cast<const void*>(&stream_kernel<NT, APL, KIND, false>);
}

template <int NT, int KIND>
const void* pick_apl(int apl, bool persistent) {
    switch (apl) {
    case 1: return pick_kernel<NT, 1, KIND>(persistent);
    case 2: return pick_kernel<NT, 2, KIND>(persistent);
    case 4: return pick_kernel<NT, 4, KIND>(persistent);
    default: return nullptr;
    }
}

template <int KIND>
const void* pick_threads(int threads, int apl, bool persistent) {
    switch (threads) {
    case 256: return pick_apl<256, KIND>(apl, persistent);
    case 512: return pick_apl<512, KIND>(apl, persistent);
    case 1024: return pick_apl<1024, KIND>(apl, persistent);
    default: return nullptr;
    }
}

}  // namespace

extern "C" {

int kda_probe_rmw(void* buf, size_t bytes, float scale, void* stream) {
    if (!buf) return 1;
    if (misaligned(buf)) return 4;
    if (bad_size(bytes)) return 6;
    const dim3 grid((unsigned)(bytes / (kThreads * kChunk)));
    hipLaunchKernelGGL(rmw_kernel, grid, dim3(kThreads), 0, (hipStream_t)stream, (f32x4*)buf, scale);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

int kda_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst) return 1;
    if (misaligned(src) || misaligned(dst)) return 4;
    if (bad_size(bytes)) return 6;
    const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
    if (s < d + bytes && d < s + bytes) return 5;
    const dim3 grid((unsigned)(bytes / (kThreads * kChunk)));
    hipLaunchKernelGGL(copy_kernel, grid, dim3(kThreads), 0, (hipStream_t)stream, (const f32x4*)src,
                       (f32x4*)dst);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

int kda_probe_stream(int kind, int threads, int chunks_per_lane, int persistent, const void* src, void* dst,
                     size_t bytes, float scale, void* stream) {
    if (kind < 0 || kind > 3) return 6;
    const bool reads = kind != 2, writes = kind != 1;
    if ((reads && !src) || (writes && !dst)) return 1;
    if ((reads && misaligned(src)) || (writes && misaligned(dst))) return 4;
    if (kind == 0 && src != dst) return 5;
    if (kind == 3) {
        const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
        if (s < d + bytes && d < s + bytes) return 5;
    }
    const void* fn = nullptr;
    switch (kind) {
    case 0: fn = pick_threads<0>(threads, chunks_per_lane, persistent != 0); break;
    case 1: fn = pick_threads<1>(threads, chunks_per_lane, persistent != 0); break;
    case 2: fn = pick_threads<2>(threads, chunks_per_lane, persistent != 0); break;
    default: fn = pick_threads<3>(threads, chunks_per_lane, persistent != 0); break;
    }
    if (!fn) return 6;
    const size_t tile = (size_t)threads * chunks_per_lane * kChunk;
    if (bytes == 0 || bytes % tile != 0 || bytes / tile > 0x7fffffffu) return 6;
    unsigned tiles = (unsigned)(bytes / tile);
    unsigned grid = tiles;
    if (persistent) {
        // every wave slot of the device: 32 waves per CU
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
            return 7;
        const unsigned slots = (unsigned)ncu * (unsigned)(2048 / threads);
        grid = tiles < slots ? tiles : slots;
    }
    const f32x4* s = static_cast<const f32x4*>(reads ? src : dst);
    f32x4* d = static_cast<f32x4*>(writes ? dst : const_cast<void*>(src));
    void* args[] = {(void*)&s, (void*)&d, (void*)&tiles, (void*)&scale};
    if (hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, (hipStream_t)stream) != hipSuccess) return 7;
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
