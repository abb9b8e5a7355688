// probe_kernels.hip -- plain streaming kernels used to calibrate measurements:
// a device copy of a known number of bytes (the reference for scaling the
// rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes) and a device read (the
// achievable read bandwidth of the HBM on this machine, the practical ceiling
// of the decode sweep).  Both use 16-byte loads, grid-stride over the whole
// buffer: the copy with four loads in flight per lane and 8 workgroups per
// compute unit, the read with eight non-temporal loads in flight per lane and
// 32 workgroups per compute unit (the fastest plain read measured on MI355X).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gqa_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4 *__restrict__ src,
                                                        uint4 *__restrict__ dst, size_t n16) {
    const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
    size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        uint4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) dst[i + u * stride] = x[u];
    }
    for (; i < n16; i += stride) dst[i] = src[i];
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Non-temporal 16-byte load (the same cache policy the decode sweep uses for K/V).
__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}

__global__ __launch_bounds__(kThreads) void read_kernel(const uint4 *__restrict__ src, size_t n16,
                                                        uint32_t *sink) {
    constexpr int kReadUnroll = 8;
    const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
    size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
        uint4 x[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) x[u] = load_nt(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 x = load_nt(src + i);
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), d));
    // Spread the atomics over the sink words so they do not serialise on one address.
    if ((threadIdx.x & 63) == 0) atomicXor(sink + (blockIdx.x % GQA_PROBE_SINK_WORDS), acc);
}

int grid_for(size_t n16, int per_cu) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    const size_t want = (n16 + kThreads - 1) / kThreads;
    const size_t cap = static_cast<size_t>(cus) * per_cu;
    return static_cast<int>(want < cap ? (want > 0 ? want : 1) : cap);
}

}  // namespace

extern "C" {

int gqa_probe_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (!src || !dst) return 1;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | bytes) % 16) return 4;
    const size_t n16 = bytes / 16;
    const int grid = grid_for(n16, 8);
    if (grid < 0) return 7;
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

int gqa_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    if (!src || !sink) return 1;
    if ((reinterpret_cast<uintptr_t>(src) | bytes) % 16 || reinterpret_cast<uintptr_t>(sink) % 4) return 4;
    const size_t n16 = bytes / 16;
    const int grid = grid_for(n16, 32);
    if (grid < 0) return 7;
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(src), n16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
