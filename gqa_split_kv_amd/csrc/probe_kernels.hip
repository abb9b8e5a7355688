// probe_kernels.hip -- plain streaming kernels used to calibrate measurements:
// a device copy of a known number of bytes (the reference for scaling the
// rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes) and a device read (the
// achievable read bandwidth of the HBM on this machine, the practical ceiling
// of the decode sweep).  The copy is grid-stride with four 16-byte loads in
// flight per lane and 8 workgroups per compute unit.  The read is grid-stride
// over 8 KiB chunks, one wavefront per SIMD, each chunk read as eight 1 KiB
// non-temporal wavefront loads in flight: the fastest of the plain reads
// measured on MI355X over a 4 GiB buffer (7.27 TB/s; a contiguous slab per
// wavefront 7.19 TB/s at one and 7.00 at two wavefronts per SIMD; 16 KiB or
// more in flight per wavefront, or loads without the non-temporal policy,
// slower).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
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

constexpr int kReadUnroll = 8;
constexpr int kReadWavesPerCu = 4;
constexpr int kReadCpol = 2;   // non-temporal, the policy the decode sweep uses for K/V
constexpr size_t kReadChunk = kReadUnroll * 1024;   // bytes per wavefront per round

// Wavefront w of W reads the chunks w, w + W, w + 2W, ... of kReadChunk bytes of
// src (the last one cut at `bytes`), 1 KiB per wavefront load.
__global__ __launch_bounds__(kThreads) void read_kernel(const uint8_t *__restrict__ src, size_t bytes,
                                                        uint32_t *sink) {
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const size_t waves = static_cast<size_t>(gridDim.x) * (kThreads / 64);
    const size_t w = static_cast<size_t>(blockIdx.x) * (kThreads / 64) + threadIdx.x / 64;
    uint32_t acc = 0;
    for (size_t beg = w * kReadChunk; beg < bytes; beg += waves * kReadChunk) {
        const size_t left = bytes - beg;
        const auto r = gqa::dev::make_rsrc(src + beg, static_cast<uint32_t>(left < kReadChunk ? left : kReadChunk));
        uint4 x[kReadUnroll];   // loads past the chunk's range read zero
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            x[u] = gqa::dev::buffer_load16<kReadCpol>(r, static_cast<uint32_t>(lane) * 16 + u * 1024);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), d));
    // Spread the atomics over the sink words so they do not serialise on one address.
    if (lane == 0) atomicXor(sink + (w % GQA_PROBE_SINK_WORDS), acc);
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
    if (bytes == 0) return 0;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 7;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 7;
    // One workgroup of kReadWavesPerCu wavefronts per compute unit (fewer for a
    // buffer of fewer chunks).
    const size_t chunks = (bytes + kReadChunk - 1) / kReadChunk;
    const size_t want = (chunks + kThreads / 64 - 1) / (kThreads / 64);
    const size_t cap = static_cast<size_t>(cus) * kReadWavesPerCu / (kThreads / 64);
    const unsigned grid = static_cast<unsigned>(want < cap ? want : cap);
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<const uint8_t *>(src), bytes, sink);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
