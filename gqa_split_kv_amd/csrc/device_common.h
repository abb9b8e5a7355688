// device_common.h -- device helpers shared by the decode (sweep, merge) and
// prefill kernels: wavefront scans over seq_lens, the stream-K range arithmetic
// the sweep and merge kernels must agree on, buffer loads, and 16-bit rounding.
// Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {
namespace dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;


__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

// Maximum of x over the four lanes l mod 16 + 16 r (r = 0..3) that share l's
// position within a 16-lane row, with the two row-swap permutes of gfx950:
// permlane16_swap with both operands x returns rows (0, 0, 2, 2) in one half of
// its result and (1, 1, 3, 3) in the other, permlane32_swap rows (0, 1, 0, 1)
// and (2, 3, 2, 3).  No LDS traffic.
__device__ __forceinline__ float max_over_rows(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ int64_t shfl64(int64_t x, int src) {
    const int lo = __shfl(static_cast<int>(static_cast<uint32_t>(x)), src);
    const int hi = __shfl(static_cast<int>(x >> 32), src);
    return (static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo);
}

__device__ __forceinline__ int64_t shfl_up64(int64_t x, int d) {
    const int lo = __shfl_up(static_cast<int>(static_cast<uint32_t>(x)), d);
    const int hi = __shfl_up(static_cast<int>(x >> 32), d);
    return (static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo);
}

__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const int lo = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(x)));
    const int hi = __builtin_amdgcn_readfirstlane(static_cast<int>(x >> 32));
    return (static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo);
}

__device__ __forceinline__ int uniform32(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int64_t inclusive_scan64(int64_t x) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int64_t y = shfl_up64(x, d);
        if (lane >= d) x += y;
    }
    return x;
}

__device__ __forceinline__ int seq_len_at(const int32_t *seq_lens, int i) {
    const int v = seq_lens[i];
    return v > 0 ? v : 0;   // a negative length counts as empty
}

// Sum of the (clamped) sequence lengths; the same value in every lane.
__device__ int64_t total_len(const int32_t *seq_lens, int batch) {
    const int lane = lane_id();
    int64_t acc = 0;
    for (int base = 0; base < batch; base += kWave) {
        const int i = base + lane;
        const int64_t len = (i < batch) ? seq_len_at(seq_lens, i) : 0;
        acc += shfl64(inclusive_scan64(len), kWave - 1);
    }
    return uniform64(acc);
}

// Sum of the lengths of sequences [0, b).
__device__ int64_t prefix_len(const int32_t *seq_lens, int b) {
    const int lane = lane_id();
    int64_t acc = 0;
    for (int base = 0; base < b; base += kWave) {
        const int i = base + lane;
        const int64_t len = (i < b) ? seq_len_at(seq_lens, i) : 0;
        acc += shfl64(inclusive_scan64(len), kWave - 1);
    }
    return uniform64(acc);
}

// The sequence b holding flat key `pos` (0 <= pos < h_kv * total), with
// off = lengths before b and len = its length.
__device__ void locate(const int32_t *seq_lens, int batch, int h_kv, int64_t pos, int &b,
                       int64_t &off, int &len) {
    const int lane = lane_id();
    int64_t run = 0;
    for (int base = 0; base < batch; base += kWave) {
        const int i = base + lane;
        const int64_t li = (i < batch) ? seq_len_at(seq_lens, i) : 0;
        const int64_t incl = inclusive_scan64(li);
        const bool hit = (i < batch) && ((run + incl) * h_kv > pos);
        const unsigned long long mask = __ballot(hit);
        if (mask) {
            const int src = __ffsll(static_cast<long long>(mask)) - 1;
            b = base + src;
            const int64_t inc_s = shfl64(incl, src);
            const int64_t len_s = shfl64(li, src);
            off = uniform64(run + inc_s - len_s);
            len = uniform32(static_cast<int>(len_s));
            return;
        }
        run += shfl64(incl, kWave - 1);
    }
    b = batch;
    off = run;
    len = 0;
}

// Value of x in lane src (src the same in every lane), as a wave-uniform value.
__device__ __forceinline__ int64_t lane64(int64_t x, int src) {
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x)), src);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(x >> 32), src);
    return (static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo);
}

// The lengths of a batch of at most 64 sequences held in registers: lane i has
// sequence i's clamped length li (0 past the batch) and the inclusive sum incl of
// lengths 0 .. i.  One load and one scan answer every seq_lens question the
// decode kernels ask (the total, a sequence's length and offset, and which
// sequence holds a key), where the loops above would each read seq_lens again.
struct FirstLens {
    int64_t li = 0, incl = 0;
    __device__ void load(const int32_t *seq_lens, int batch) {
        const int i = lane_id();
        li = (i < batch) ? seq_len_at(seq_lens, i) : 0;
        // One sequence: every lane's inclusive prefix is lane 0's length (no scan).
        incl = batch == 1 ? static_cast<int64_t>(__builtin_amdgcn_readlane(static_cast<int>(li), 0))
                          : inclusive_scan64(li);
    }
    __device__ int64_t total() const { return lane64(incl, kWave - 1); }
    __device__ int len(int b) const { return static_cast<int>(lane64(li, b)); }      // b < 64
    __device__ int64_t prefix(int b) const { return lane64(incl, b) - lane64(li, b); }   // b < 64
    // locate() over these lengths.
    __device__ void locate(int batch, int h_kv, int64_t pos, int &b, int64_t &off, int &len) const {
        const unsigned long long mask = __ballot(lane_id() < batch && incl * h_kv > pos);
        if (mask) {
            b = __ffsll(static_cast<long long>(mask)) - 1;
            len = static_cast<int>(lane64(li, b));
            off = lane64(incl, b) - len;
        } else {
            b = batch;
            off = total();
            len = 0;
        }
    }
};

// Quotient of non-negative a by positive b; a 32-bit division when both fit (a
// few tens of instructions instead of the few hundred of a 64-bit one).
__device__ __forceinline__ int64_t div_nonneg(int64_t a, int64_t b) {
    if (((a | b) >> 32) == 0) return static_cast<int64_t>(static_cast<uint32_t>(a) / static_cast<uint32_t>(b));
    return a / b;
}

// Keys per range: max(min_chunk, ceil(total / num_chunks)).  The partial and the
// merge kernel must agree on it exactly.
__device__ __forceinline__ int64_t chunk_keys(int64_t total, int num_chunks, int min_chunk) {
    const int64_t c = div_nonneg(total + num_chunks - 1, num_chunks);
    return c > min_chunk ? c : static_cast<int64_t>(min_chunk);
}

// Buffer resource over `bytes` bytes at `base` (raw, stride 0): loads at offsets
// at or beyond `bytes` return zero without touching memory.  Both inputs must be
// wave-uniform; readfirstlane makes that visible so the resource sits in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const int64_t a = uniform64(reinterpret_cast<int64_t>(base));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(a), 0,
                                             uniform32(static_cast<int>(bytes)), 0x00020000);
}

// 16-byte buffer load with the given cache-policy bits.
template <int kCpol>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpol);
    return make_uint4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two outputs rounded to nearest even, packed (the first in the low half):
// bf16 (kHalf = false) or IEEE fp16 (kHalf = true).
template <bool kHalf>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (kHalf) {
        const f32x2_t v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
    } else {
        return bf16_rne(a) | (bf16_rne(b) << 16);
    }
}

}  // namespace dev
}  // namespace gqa
