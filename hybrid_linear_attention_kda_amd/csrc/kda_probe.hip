// kda_probe.hip -- HBM streaming probes for measurement (libkda_probe.so).
//
// Not part of the decode step.  They state what a plain stream of the same
// access contract achieves on the device, and give rocprofv3's byte counters
// a kernel of exactly known traffic to be calibrated against:
//  * rmw:  in place, every 16-byte chunk read once and written once
//          (the state update's contract), 512 threads per workgroup, one
//          chunk per lane;
//  * copy: 16-byte chunks from src to dst, same shape.
// Loads are non-temporal; stores are non-temporal with agent scope (sc1), the
// fastest of the cache-policy combinations measured on MI355X (an in-place
// stream over 128 MiB: 6.56 TB/s; 6.41 TB/s with non-temporal stores alone;
// 5.6-5.7 TB/s with a plain load or a plain store) and the policy of the
// decode kernel's state stores on large grids.
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "kda_probe.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 512;
constexpr size_t kChunk = 16;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// A workgroup's kThreads chunks starting at base, as a raw buffer (stride 0,
// 32-bit data format): hipcc exposes the agent-scope cache-policy bit on
// buffer accesses only.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)(kThreads * kChunk), 0x00020000);
}

// lane's 16-byte chunk of the workgroup's buffer, agent scope (sc1 = 16) +
// non-temporal (nt = 2)
__device__ __forceinline__ void store_sc1_nt(__amdgpu_buffer_rsrc_t rs, const f32x4& v) {
    const u32x4 r = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(r, rs, (int)(threadIdx.x * kChunk), 0, 16 | 2);
}

__global__ __launch_bounds__(kThreads) void rmw_kernel(f32x4* __restrict__ a, float scale) {
    f32x4* const blk = a + (size_t)blockIdx.x * kThreads;
    const f32x4 v = __builtin_nontemporal_load(blk + threadIdx.x) * scale;
    store_sc1_nt(block_rsrc(blk), v);
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst) {
    const size_t b = (size_t)blockIdx.x * kThreads;
    store_sc1_nt(block_rsrc(dst + b), __builtin_nontemporal_load(src + b + threadIdx.x));
}

bool bad_size(size_t bytes) {
    return bytes == 0 || bytes % (kThreads * kChunk) != 0 || bytes / (kThreads * kChunk) > 0x7fffffffu;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

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

}  // extern "C"
