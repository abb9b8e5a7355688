// probe_kernels.hip -- plain streaming kernels used to calibrate measurements:
// a device copy of a known number of bytes (the reference for scaling the
// rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes) and a device read (the
// achievable read bandwidth of the HBM on this machine, the practical ceiling
// of the decode sweep).  The copy is grid-stride with four 16-byte loads in
// flight per lane and 8 workgroups per compute unit.  The read gives every
// wavefront one contiguous slab and streams it with non-temporal 16-byte buffer
// loads, eight 1 KiB wavefront loads in flight, two wavefronts per SIMD (the
// fastest plain read measured on MI355X: ~7.06 TB/s, where a grid-stride read
// with the same policy reached ~5.7 TB/s).
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
constexpr int kReadWavesPerCu = 8;
constexpr int kReadCpol = 2;   // non-temporal, the policy the decode sweep uses for K/V

// Wavefront w reads the 16-byte units [w per, min((w + 1) per, n16)) of src
// (per: a multiple of 64, at most 2^27 units so that a slab's byte count fits a
// buffer resource), 1 KiB per wavefront load.
__global__ __launch_bounds__(kThreads) void read_kernel(const uint8_t *__restrict__ src, size_t n16, size_t per,
                                                        uint32_t *sink) {
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const size_t w = static_cast<size_t>(blockIdx.x) * (kThreads / 64) + threadIdx.x / 64;
    const size_t beg = w * per;
    uint32_t acc = 0;
    if (beg < n16) {
        const size_t end = beg + per < n16 ? beg + per : n16;
        const uint32_t bytes = static_cast<uint32_t>((end - beg) * 16);
        const auto r = gqa::dev::make_rsrc(src + beg * 16, bytes);
        for (uint32_t off = static_cast<uint32_t>(lane) * 16; off < bytes; off += kReadUnroll * 1024) {
            uint4 x[kReadUnroll];   // loads past the slab's end read zero
#pragma unroll
            for (int u = 0; u < kReadUnroll; ++u) x[u] = gqa::dev::buffer_load16<kReadCpol>(r, off + u * 1024);
#pragma unroll
            for (int u = 0; u < kReadUnroll; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
        }
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
    const size_t n16 = bytes / 16;
    if (n16 == 0) return 0;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 7;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 7;
    const size_t waves = static_cast<size_t>(cus) * kReadWavesPerCu;
    size_t per = ((n16 + waves - 1) / waves + 63) & ~static_cast<size_t>(63);
    if (per > (static_cast<size_t>(1) << 27)) per = static_cast<size_t>(1) << 27;
    const size_t grid = ((n16 + per - 1) / per + kThreads / 64 - 1) / (kThreads / 64);
    if (grid > 0x7fffffffu) return 7;
    hipLaunchKernelGGL(read_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const uint8_t *>(src), n16, per, sink);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
