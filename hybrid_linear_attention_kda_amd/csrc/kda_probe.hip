// kda_probe.hip -- HBM streaming probes for measurement (libkda_probe.so).
//
// Not part of the decode step.  They state what a plain stream of the same
// access contract achieves on the device, and give rocprofv3's byte counters
// a kernel of exactly known traffic to be calibrated against:
//  * rmw:  in place, every 16-byte chunk read once and written once
//          (the state update's contract), non-temporal, 512 threads per
//          workgroup, one chunk per lane;
//  * copy: 16-byte chunks from src to dst, non-temporal, same shape.
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "kda_probe.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 512;
constexpr size_t kChunk = 16;

__global__ __launch_bounds__(kThreads) void rmw_kernel(f32x4* __restrict__ a, float scale) {
    f32x4* p = a + (size_t)blockIdx.x * kThreads + threadIdx.x;
    f32x4 v = __builtin_nontemporal_load(p);
    __builtin_nontemporal_store(v * scale, p);
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst) {
    const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
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
