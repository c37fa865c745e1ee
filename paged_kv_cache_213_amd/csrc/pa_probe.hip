// pa_probe.hip -- measurement kernels that sit beside the attention path:
// a streaming read of a large buffer (the achievable HBM read rate that
// the attention kernels are compared with) and a plain copy of known size
// (to calibrate the byte counters of the profiler).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "pagedattn_probe.h"

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Nontemporal 16-byte load: the same load kind the attention kernels use for
// the K/V bytes they read once.
__device__ __forceinline__ u32x4_t ld_stream(const u32x4_t* p) {
    return __builtin_nontemporal_load(p);
}

// One wave per workgroup; wave w reads 8 KB chunks w, w + grid, ... whole
// (eight 16-byte loads per lane, all requested before any is used), then
// the bytes past the last whole chunk. Contiguous 8 KB per wave is the read
// shape this device serves fastest (a grid-stride loop of 16-byte loads,
// each wave touching four places 16 MB apart, reads about 15% slower).
constexpr int kChunk16 = 512;  // 16-byte elements per 8 KB chunk
__global__ __launch_bounds__(64) void stream_read_kernel(const u32x4_t* __restrict__ src,
                                                         int64_t n16, uint32_t* sink) {
    const int lane = threadIdx.x;
    uint32_t acc = 0;
    const int64_t nchunks = n16 / kChunk16;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const u32x4_t* p = src + c * kChunk16 + lane;
        u32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = ld_stream(p + 64 * u);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (int64_t i = nchunks * kChunk16 + (int64_t)blockIdx.x * 64 + lane; i < n16;
         i += (int64_t)gridDim.x * 64) {
        const u32x4_t a = ld_stream(src + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;  // keeps the loads live
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

int grid_for(int64_t n16) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    int64_t g = (int64_t)cus * 8;
    const int64_t need = (n16 + 255) / 256;
    return (int)(need < g ? (need > 0 ? need : 1) : g);
}

}  // namespace

extern "C" int pa_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink || (bytes & 15) || ((uintptr_t)buf & 15)) return PA_EINVAL;
    const int64_t n16 = (int64_t)(bytes / 16);
    // one wave per SIMD
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t need = (n16 + 63) / 64;
    const int grid = (int)std::min<int64_t>((int64_t)cus * 4, need > 0 ? need : 1);
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(64), 0, (hipStream_t)stream,
                       (const u32x4_t*)buf, n16, sink);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_EHIP;
}

extern "C" int pa_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || (bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
        return PA_EINVAL;
    const int64_t n16 = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n16)), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)src, (uint4*)dst, n16);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_EHIP;
}
