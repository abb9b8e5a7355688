// decode_kernels.hip -- gfx950 (CDNA4) kernels of split-KV GQA decode.
//
// Method (kernbench2 page "_gqa_attention_decode_long.py"): the keys of every
// (sequence, kv head) are swept in tiles; each tile gives a partial online-softmax
// triple (m, l, O) for all G query heads that share the kv head ("M-fold": the G
// heads are the rows of one product with the key tile), tiles are folded with
// `_merge_running` (m = max; both sides rescaled by exp(m_side - m); l and O
// summed), ranges handled by different workers are reduced with the same merge,
// and the owner stores O / l ("Final normalise + store").
//
// Mapping to one MI355X:
//   * The page's ranks become wavefronts.  The flattened key axis -- the keys of
//     all (sequence, kv head) pairs end to end -- is cut into equal ranges, one
//     per wavefront (stream-K style), so ragged lengths cost no load imbalance.
//     A range that covers a whole pair stores o itself; a pair cut across ranges
//     leaves one partial triple per piece in a workspace, merged by merge_kernel.
//   * A wavefront sweeps its piece in 16-key blocks.  Q K^T for the block is one
//     to four v_mfma_f32_16x16x32_bf16 (or 16x16x4_f32 for fp32 input) with the
//     16 keys as the M axis and the (up to 16) query heads as the N axis; K rows
//     are loaded straight into the MFMA A-operand layout with 16-byte loads, so
//     no LDS round trip is needed.  The d axis of the contraction is permuted
//     (the same permutation on Q and K) so each load instruction reads 64
//     contiguous bytes of 16 key rows.
//   * P V runs as v_mfma_f32_16x16x4_f32 with V^T as the A operand and P^T as the
//     B operand: each lane contributes one key per MFMA, so V rows need no
//     transpose and P stays in fp32 (no rounding of the softmax weights).  The
//     V loads read 4 whole key rows per instruction.
//   * The softmax state of query head g lives in lanes with lane % 16 == g; the
//     block maximum is reduced across the 4 lane groups with two cross-lane
//     exchanges, l is kept per lane and reduced once per piece.  Scores are kept
//     in the log2 domain (scale * log2 e folded in) and exponentiated with
//     v_exp_f32; the partial m is stored in that domain and merged with exp2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace gqa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlockKeys = 16;

// ------------------------------------------------------------------ wave helpers

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

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

// Keys per range: max(min_chunk, ceil(total / num_chunks)).  The partial and the
// merge kernel must agree on it exactly.
__device__ __forceinline__ int64_t chunk_keys(int64_t total, int num_chunks, int min_chunk) {
    const int64_t c = (total + num_chunks - 1) / num_chunks;
    return c > min_chunk ? c : static_cast<int64_t>(min_chunk);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ------------------------------------------------------------------ per-type shape

template <bool kBf16In, int D>
struct Shape {
    static constexpr int ES = kBf16In ? 2 : 4;   // input element bytes
    static constexpr int ROWB = D * ES;          // one key row of one kv head
    static constexpr int NKP = ROWB / 64;        // 16-byte K pieces per lane per block
    static constexpr int VEC = D / 16;           // V elements per lane per key row
    static constexpr int VW = VEC * ES / 4;      // V 32-bit words per lane per key row
    static constexpr int QOPS = kBf16In ? NKP : NKP * 4;   // MFMAs for Q K^T per block
};

template <bool kBf16In, int D>
struct Block {
    uint4 k[Shape<kBf16In, D>::NKP];
    uint32_t v[4][Shape<kBf16In, D>::VW];
};

template <int NW>
__device__ __forceinline__ void load_words(uint32_t (&dst)[NW], const uint8_t *p) {
    if constexpr (NW == 2) {
        const uint2 x = *reinterpret_cast<const uint2 *>(p);
        dst[0] = x.x;
        dst[1] = x.y;
    } else {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const uint4 x = *reinterpret_cast<const uint4 *>(p + 16 * i);
            dst[4 * i + 0] = x.x;
            dst[4 * i + 1] = x.y;
            dst[4 * i + 2] = x.z;
            dst[4 * i + 3] = x.w;
        }
    }
}

// Loads one 16-key block (keys [16*blk, 16*blk + 16) of the piece, clamped to the
// last valid key so every address stays inside the piece).  The block base is
// wave-uniform and the lane offsets are 32-bit, so the loads take the
// scalar-base + vector-offset form.
template <bool kBf16In, int D>
__device__ __forceinline__ void load_block(Block<kBf16In, D> &B, const uint8_t *kbase,
                                           const uint8_t *vbase, int rowstride, int blk, int nkeys) {
    using S = Shape<kBf16In, D>;
    const int lane = lane_id();
    const int m = lane & 15;
    const int kg = lane >> 4;
    const int last = min(kBlockKeys, nkeys - blk * kBlockKeys) - 1;
    const int64_t boff = static_cast<int64_t>(blk) * kBlockKeys * rowstride;
    const uint8_t *kb = kbase + boff;
    const uint8_t *vb = vbase + boff;
    // K: lane -> key m of the block, bytes [64p + 16kg, +16) of the row.
    const uint32_t koff = static_cast<uint32_t>(min(m, last) * rowstride + 16 * kg);
#pragma unroll
    for (int p = 0; p < S::NKP; ++p) B.k[p] = *reinterpret_cast<const uint4 *>(kb + koff + 64 * p);
    // V: lane -> key 4kg + r of the block, elements [VEC*m, VEC*m + VEC) of the row.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t voff = static_cast<uint32_t>(min(4 * kg + r, last) * rowstride + m * S::VEC * S::ES);
        load_words<S::VW>(B.v[r], vb + voff);
    }
}

// Q K^T of one block: s[q] = score of key 4*kg + q against query head lane%16.
template <bool kBf16In, int D>
__device__ __forceinline__ f32x4_t qk_block(const Block<kBf16In, D> &B,
                                            const uint4 (&qop)[Shape<kBf16In, D>::NKP]) {
    using S = Shape<kBf16In, D>;
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < S::NKP; ++p) {
        if constexpr (kBf16In) {
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, B.k[p]),
                                                        __builtin_bit_cast(bf16x8_t, qop[p]), s, 0,
                                                        0, 0);
        } else {
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(B.k[p].x),
                                                     __uint_as_float(qop[p].x), s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(B.k[p].y),
                                                     __uint_as_float(qop[p].y), s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(B.k[p].z),
                                                     __uint_as_float(qop[p].z), s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(B.k[p].w),
                                                     __uint_as_float(qop[p].w), s, 0, 0, 0);
        }
    }
    return s;
}

// O[c] += V^T P^T for one block: acc[c][q] holds O[g = lane%16][d = VEC*(4kg+q) + c].
template <bool kBf16In, int D>
__device__ __forceinline__ void pv_block(const Block<kBf16In, D> &B, const float (&p)[4],
                                         f32x4_t (&acc)[Shape<kBf16In, D>::VEC]) {
    using S = Shape<kBf16In, D>;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float vf[S::VEC];
        if constexpr (kBf16In) {
#pragma unroll
            for (int w = 0; w < S::VW; ++w) {
                vf[2 * w] = bf16_lo(B.v[r][w]);
                vf[2 * w + 1] = bf16_hi(B.v[r][w]);
            }
        } else {
#pragma unroll
            for (int w = 0; w < S::VW; ++w) vf[w] = __uint_as_float(B.v[r][w]);
        }
#pragma unroll
        for (int c = 0; c < S::VEC; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[c], p[r], acc[c], 0, 0, 0);
    }
}

// One block of the sweep: scores, online-softmax update (the page's running
// merge of the block's (m, l, O) into the state), and P V.
template <bool kBf16In, int D>
__device__ __forceinline__ void block_step(const Block<kBf16In, D> &B,
                                           const uint4 (&qop)[Shape<kBf16In, D>::NKP], int nvalid,
                                           int kg, float sl2, float &m_run, float &l_run,
                                           f32x4_t (&acc)[Shape<kBf16In, D>::VEC]) {
    using S = Shape<kBf16In, D>;
    const f32x4_t s = qk_block<kBf16In, D>(B, qop);
    float sv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sv[q] = (4 * kg + q < nvalid) ? s[q] * sl2 : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first block
    float p[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) p[q] = __builtin_amdgcn_exp2f(sv[q] - m_new);
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int c = 0; c < S::VEC; ++c) acc[c] *= alpha;
    m_run = m_new;
    pv_block<kBf16In, D>(B, p, acc);
}

template <bool kBf16Out>
__device__ __forceinline__ void store_row(uint8_t *dst, const float *x, int n);

// Stores n (multiple of 8) consecutive values.
template <>
__device__ __forceinline__ void store_row<true>(uint8_t *dst, const float *x, int n) {
    for (int i = 0; i < n; i += 8) {
        uint4 w;
        w.x = bf16_rne(x[i + 0]) | (bf16_rne(x[i + 1]) << 16);
        w.y = bf16_rne(x[i + 2]) | (bf16_rne(x[i + 3]) << 16);
        w.z = bf16_rne(x[i + 4]) | (bf16_rne(x[i + 5]) << 16);
        w.w = bf16_rne(x[i + 6]) | (bf16_rne(x[i + 7]) << 16);
        *reinterpret_cast<uint4 *>(dst + 2 * i) = w;
    }
}

template <>
__device__ __forceinline__ void store_row<false>(uint8_t *dst, const float *x, int n) {
    for (int i = 0; i < n; i += 4)
        *reinterpret_cast<float4 *>(dst + 4 * i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
}

// One piece: keys [t0, t1) of (sequence b, kv head j); off = keys before b.
template <bool kBf16In, bool kBf16Out, int D>
__device__ __forceinline__ void process_piece(const DecodeParams &P, int b, int j, int64_t off,
                                              int t0, int t1, int len, int w) {
    using S = Shape<kBf16In, D>;
    const int lane = lane_id();
    const int g = lane & 15;
    const int kg = lane >> 4;
    const int G = P.G;
    const int rowstride = P.h_kv * S::ROWB;

    // Q operand: query head j*G + g, bytes [64p + 16kg, +16) of its row (zero for g >= G).
    uint4 qop[S::NKP];
    {
        const int gq = g < G ? g : G - 1;
        const uint8_t *qrow = P.q + (static_cast<int64_t>(b) * P.h_q + j * G + gq) * S::ROWB + 16 * kg;
#pragma unroll
        for (int p = 0; p < S::NKP; ++p) {
            qop[p] = *reinterpret_cast<const uint4 *>(qrow + 64 * p);
            if (g >= G) qop[p] = make_uint4(0, 0, 0, 0);
        }
    }

    f32x4_t acc[S::VEC];
#pragma unroll
    for (int c = 0; c < S::VEC; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    const int nkeys = t1 - t0;
    const int nblk = (nkeys + kBlockKeys - 1) / kBlockKeys;
    const int64_t row0 = (off + t0) * P.h_kv + j;
    const uint8_t *kbase = P.k + row0 * S::ROWB;
    const uint8_t *vbase = P.v + row0 * S::ROWB;
    const float sl2 = P.scale_log2;

    // Software pipeline over two register buffers: the loads of block blk+1 are in
    // flight while block blk is computed.  The prefetch index is clamped so the
    // loads are unconditional (the last block is fetched twice, from cache).
    Block<kBf16In, D> bufA, bufB;
    load_block<kBf16In, D>(bufA, kbase, vbase, rowstride, 0, nkeys);
    int blk = 0;
    while (true) {
        load_block<kBf16In, D>(bufB, kbase, vbase, rowstride, min(blk + 1, nblk - 1), nkeys);
        __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the compute
        block_step<kBf16In, D>(bufA, qop, min(kBlockKeys, nkeys - blk * kBlockKeys), kg, sl2, m_run,
                               l_run, acc);
        if (++blk == nblk) break;
        load_block<kBf16In, D>(bufA, kbase, vbase, rowstride, min(blk + 1, nblk - 1), nkeys);
        __builtin_amdgcn_sched_barrier(0);
        block_step<kBf16In, D>(bufB, qop, min(kBlockKeys, nkeys - blk * kBlockKeys), kg, sl2, m_run,
                               l_run, acc);
        if (++blk == nblk) break;
    }

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);

    // The lane's outputs: d in [4*VEC*kg, 4*VEC*kg + 4*VEC), index q*VEC + c.
    float out[4 * S::VEC];
    if (t0 == 0 && t1 == len) {
        // The whole (sequence, kv head) was in this range: normalise and store.
        const float inv = 1.0f / l_tot;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < S::VEC; ++c) out[q * S::VEC + c] = acc[c][q] * inv;
        if (g < G) {
            const int64_t orow = static_cast<int64_t>(b) * P.h_q + j * G + g;
            uint8_t *dst = P.o + (orow * D + 4 * S::VEC * kg) * (kBf16Out ? 2 : 4);
            store_row<kBf16Out>(dst, out, 4 * S::VEC);
        }
    } else {
        // Slot 0: a piece of a pair that began before this range; slot 1: the
        // first piece of a pair that continues past it.
        const int slot = (t0 > 0) ? 0 : 1;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < S::VEC; ++c) out[q * S::VEC + c] = acc[c][q];
        if (g < G) {
            const int64_t srow = (static_cast<int64_t>(w) * 2 + slot) * G + g;
            store_row<false>(reinterpret_cast<uint8_t *>(P.ws_o + srow * D + 4 * S::VEC * kg), out,
                             4 * S::VEC);
            if (kg == 0) P.ws_ml[srow] = make_float2(m_run, l_tot);
        }
    }
}

template <bool kBf16In, bool kBf16Out, int D>
__global__ __launch_bounds__(kThreads) void split_kernel(DecodeParams P) {
    const int w = uniform32(static_cast<int>(blockIdx.x) * kWavesPerBlock +
                            static_cast<int>(threadIdx.x) / kWave);
    if (w >= P.num_chunks) return;
    const int64_t total = static_cast<int64_t>(P.h_kv) * total_len(P.seq_lens, P.batch);
    const int64_t chunk = chunk_keys(total, P.num_chunks, P.min_chunk);
    int64_t pos = static_cast<int64_t>(w) * chunk;
    if (pos >= total) return;
    const int64_t end = pos + chunk < total ? pos + chunk : total;
    int b, len;
    int64_t off;
    locate(P.seq_lens, P.batch, P.h_kv, pos, b, off, len);
    while (true) {
        const int64_t seq_start = off * P.h_kv;
        const int j = uniform32(static_cast<int>((pos - seq_start) / len));
        const int64_t ustart = seq_start + static_cast<int64_t>(j) * len;
        const int t0 = uniform32(static_cast<int>(pos - ustart));
        const int64_t lim = end - ustart;
        const int t1 = uniform32(static_cast<int>(lim < len ? lim : len));
        process_piece<kBf16In, kBf16Out, D>(P, b, j, off, t0, t1, len, w);
        pos = ustart + t1;
        if (pos >= end) break;
        if (j + 1 == P.h_kv) {   // next non-empty sequence (one exists: pos < total)
            off += len;
            do {
                ++b;
                len = uniform32(seq_len_at(P.seq_lens, b));
            } while (len == 0);
        }
    }
}

// Merge of the pieces of one (sequence, kv head): for every query head g and
// element d, M = max m_s, L = sum l_s 2^(m_s - M), o = sum O_s 2^(m_s - M) / L,
// pieces in ascending order.  Also writes zeros for an empty sequence.
template <bool kBf16Out, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeParams P) {
    const int b = static_cast<int>(blockIdx.x) / P.h_kv;
    const int j = static_cast<int>(blockIdx.x) % P.h_kv;
    const int G = P.G;
    const int len = uniform32(seq_len_at(P.seq_lens, b));
    uint8_t *obase = P.o + (static_cast<int64_t>(b) * P.h_q + j * G) * D * (kBf16Out ? 2 : 4);
    const int n = G * D;
    if (len == 0) {
        for (int e = threadIdx.x; e < n; e += kThreads) {
            if constexpr (kBf16Out)
                reinterpret_cast<uint16_t *>(obase)[e] = 0;
            else
                reinterpret_cast<float *>(obase)[e] = 0.f;
        }
        return;
    }
    const int64_t total = static_cast<int64_t>(P.h_kv) * total_len(P.seq_lens, P.batch);
    const int64_t chunk = chunk_keys(total, P.num_chunks, P.min_chunk);
    const int64_t ustart = prefix_len(P.seq_lens, b) * P.h_kv + static_cast<int64_t>(j) * len;
    const int64_t wa = ustart / chunk;
    const int64_t wb = (ustart + len - 1) / chunk;
    if (wa == wb) return;   // written whole by the partial kernel
    for (int e = threadIdx.x; e < n; e += kThreads) {
        const int g = e / D;
        const int d = e - g * D;
        float M = -INFINITY;
        for (int64_t s = wa; s <= wb; ++s) {
            const int64_t srow = (s * 2 + (s == wa ? 1 : 0)) * G + g;
            M = fmaxf(M, P.ws_ml[srow].x);
        }
        float L = 0.f, acc = 0.f;
        for (int64_t s = wa; s <= wb; ++s) {
            const int64_t srow = (s * 2 + (s == wa ? 1 : 0)) * G + g;
            const float2 ml = P.ws_ml[srow];
            const float f = __builtin_amdgcn_exp2f(ml.x - M);
            L += f * ml.y;
            acc += f * P.ws_o[srow * D + d];
        }
        const float r = acc / L;
        if constexpr (kBf16Out)
            reinterpret_cast<uint16_t *>(obase)[e] = static_cast<uint16_t>(bf16_rne(r));
        else
            reinterpret_cast<float *>(obase)[e] = r;
    }
}

template <bool kBf16In, bool kBf16Out, int D>
hipError_t launch_variant(const DecodeParams &P, int split_blocks, int merge_blocks,
                          hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
    hipError_t e;
    if (ev_begin && (e = hipEventRecord(ev_begin, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL((split_kernel<kBf16In, kBf16Out, D>), dim3(split_blocks), dim3(kThreads), 0,
                       stream, P);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_end && (e = hipEventRecord(ev_end, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL((merge_kernel<kBf16Out, D>), dim3(merge_blocks), dim3(kThreads), 0, stream, P);
    return hipGetLastError();
}

template <bool kBf16In, bool kBf16Out, int D>
hipError_t occupancy_variant(int *blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu,
                                                        split_kernel<kBf16In, kBf16Out, D>, kThreads, 0);
}

}  // namespace

hipError_t launch_decode(const DecodeParams &P, int in_bf16, int out_bf16, int D, int split_blocks,
                         int merge_blocks, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
    if (in_bf16 && out_bf16) {
        return D == 128 ? launch_variant<true, true, 128>(P, split_blocks, merge_blocks, stream, ev_begin, ev_end)
                        : launch_variant<true, true, 64>(P, split_blocks, merge_blocks, stream, ev_begin, ev_end);
    }
    if (in_bf16) {
        return D == 128 ? launch_variant<true, false, 128>(P, split_blocks, merge_blocks, stream, ev_begin, ev_end)
                        : launch_variant<true, false, 64>(P, split_blocks, merge_blocks, stream, ev_begin, ev_end);
    }
    return D == 128 ? launch_variant<false, false, 128>(P, split_blocks, merge_blocks, stream, ev_begin, ev_end)
                    : launch_variant<false, false, 64>(P, split_blocks, merge_blocks, stream, ev_begin, ev_end);
}

hipError_t split_occupancy(int in_bf16, int out_bf16, int D, int *blocks_per_cu) {
    if (in_bf16 && out_bf16)
        return D == 128 ? occupancy_variant<true, true, 128>(blocks_per_cu)
                        : occupancy_variant<true, true, 64>(blocks_per_cu);
    if (in_bf16)
        return D == 128 ? occupancy_variant<true, false, 128>(blocks_per_cu)
                        : occupancy_variant<true, false, 64>(blocks_per_cu);
    return D == 128 ? occupancy_variant<false, false, 128>(blocks_per_cu)
                    : occupancy_variant<false, false, 64>(blocks_per_cu);
}

}  // namespace gqa
