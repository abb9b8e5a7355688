// merge_kernel.hip -- log-sum-exp merge of the partial triples a sequence left in
// the workspace when its keys were cut across several sweep ranges.
//
// For row (query token t, query head g) of (sequence b, kv head j) with pieces
// s = ca .. cb (range s
// was swept by wavefront s*h_kv + j; the first piece sits in slot 1 of its
// wavefront, the rest in slot 0):
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  o = sum_s O_s 2^(m_s - M) / L
// (kernbench2 page "_gqa_attention_decode_long.py", `_merge_running`: the
// pairwise rule applied to all pieces at once with their common maximum, which
// is the same reduction its chain and centre-root trees compute), then the final
// normalise and store.  m is in log2 units (the sweep folds log2 e into the
// scale), so the weights are exp2.
//
// Layout: a workgroup covers (sequence, kv head), a group of rows (query token,
// query head) and a slice of d.  Thread (pl, h, eq) owns four consecutive
// elements d = 4eq .. 4eq+3 of row h and the pieces s = ca + pl, ca + pl + PL,
// ...; it loads eight pieces at a time and folds them into a running (M, L, acc)
// with the merge rule; the piece lanes are then folded in a fixed tree (lanes of
// a wavefront by shuffles, then the wavefronts through LDS in ascending order),
// so the result is deterministic.  Three layouts: narrow (one piece lane, up to
// 8 rows of all of d per workgroup at d 128) for sequences cut into few pieces;
// wide (one row, all of d, 32 piece lanes at d 128) for long sequences cut into
// many; split (one row, 32 elements of d, 128 piece lanes) for a few units cut
// into very many pieces, where the wide layout would leave most of the GPU idle.
// Also writes zeros for an empty sequence.  With a single sequence and a length
// bound from the caller, the pieces are read for a length of exactly the bound
// while seq_lens is read, and the two lengths are compared before any store (a
// mismatch takes the general path; the result is the same either way).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace gqa {
namespace {

using namespace dev;

constexpr int kF32 = 1;
constexpr int kF16 = 2;

// Stores four consecutive outputs of one head, rounded to the output type.
template <int kOut>
__device__ __forceinline__ void store_quad(uint8_t *row, int eq, float4 x) {
    if constexpr (kOut == kF32)
        reinterpret_cast<float4 *>(row)[eq] = x;
    else
        reinterpret_cast<uint2 *>(row)[eq] = make_uint2(pack2<kOut == kF16>(x.x, x.y), pack2<kOut == kF16>(x.z, x.w));
}

// Folds a batch of pieces into a running (M, L, acc) with the merge rule: the new
// maximum, both sides rescaled by 2^(old - new), sums added.  Every multiply-add
// is written as one fused operation (nothing is left to contraction), so each
// inlined copy of the merge rounds alike.
struct Running {
    float M, L;
    float4 acc;
};

__device__ __forceinline__ void fold(Running &r, float m, float l, float4 o) {
    const float Mn = fmaxf(r.M, m);
    // Both sides empty (-inf): exponentiate against 0 so the identity stays NaN-free.
    const float Mr = Mn == -INFINITY ? 0.f : Mn;
    const float a = __builtin_amdgcn_exp2f(r.M - Mr);   // 0 when r is empty
    const float f = __builtin_amdgcn_exp2f(m - Mr);     // 0 for an empty side
    r.L = __builtin_fmaf(r.L, a, l * f);
    r.acc.x = __builtin_fmaf(r.acc.x, a, o.x * f);
    r.acc.y = __builtin_fmaf(r.acc.y, a, o.y * f);
    r.acc.z = __builtin_fmaf(r.acc.z, a, o.z * f);
    r.acc.w = __builtin_fmaf(r.acc.w, a, o.w * f);
    r.M = Mn;
}

__device__ __forceinline__ Running shfl_xor_running(const Running &r, int mask) {
    Running o;
    o.M = __shfl_xor(r.M, mask);
    o.L = __shfl_xor(r.L, mask);
    o.acc.x = __shfl_xor(r.acc.x, mask);
    o.acc.y = __shfl_xor(r.acc.y, mask);
    o.acc.z = __shfl_xor(r.acc.z, mask);
    o.acc.w = __shfl_xor(r.acc.w, mask);
    return o;
}

// Workgroup layout: kRows rows x PL piece lanes x kQuads element quads (one d
// slice of 4 kQuads elements; D / (4 kQuads) slices per row); a row is one
// (query token, query head) of the kv head, row = t * G + g.
template <int kThreadsM, int kRows, int kQuads>
struct MergeLayout {
    static constexpr int TP = kQuads * kRows;        // threads per piece lane
    static constexpr int PL = kThreadsM / TP;        // piece lanes
    static constexpr int kWaves = kThreadsM / kWave;
    static_assert(PL >= 1 && PL * TP == kThreadsM, "layout");
    static_assert(PL == 1 || TP <= kWave, "piece lanes are folded within and across wavefronts");
    // LDS of the fold across wavefronts: lanes [0, TP) of every wavefront.
    static constexpr int kRunRows = PL > 1 ? kWaves : 1;
    static constexpr int kRunCols = PL > 1 ? TP : 1;
};

// Merges the pieces of (sequence b, kv head j) for the thread's row g and element
// quad eq, given the sequence's length, the total over the batch and the keys
// before it, and stores o.  With kCheck (one sequence whose length was
// predicted), the pieces are read at once and the stored length `got` (as read:
// a negative value never equals the positive prediction), read before them, is
// compared with the prediction before anything is stored: on a mismatch
// every wavefront returns false having stored nothing (the slots read lie inside
// the workspace either way).  Otherwise returns true.
template <int kOut, int D, int kThreadsM, int kRows, int kQuads, bool kCheck>
__device__ __forceinline__ bool merge_pieces(const DecodeParams &P,
                                             Running (*s_run)[MergeLayout<kThreadsM, kRows, kQuads>::kRunCols],
                                             int j, int g, int eq, bool active, uint8_t *orow, int len,
                                             int64_t total, int64_t ustart, int got) {
    using Lay = MergeLayout<kThreadsM, kRows, kQuads>;
    constexpr int TP = Lay::TP;
    constexpr int PL = Lay::PL;
    constexpr int kBatch = 8;                        // pieces in flight per thread
    const int R = P.R;
    const int tid = static_cast<int>(threadIdx.x);
    const int pl = tid / TP;
    const int64_t chunk = chunk_keys(total, P.num_chunks / P.h_kv, P.min_chunk);
    const int64_t ca = ustart / chunk;   // token ranges holding this sequence
    const int64_t cb = (ustart + len - 1) / chunk;
    // The prediction held: the same test in every wavefront (each read the length).
    auto confirmed = [&]() { return !kCheck || uniform32(got) == len; };
    if (ca == cb) return confirmed();    // written whole by the sweep kernel

    Running r = {-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
    if (active) {
        for (int64_t s0 = ca + pl; s0 <= cb; s0 += static_cast<int64_t>(PL) * kBatch) {
            float2 ml[kBatch];
            float4 ov[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                const int64_t s = s0 + static_cast<int64_t>(i) * PL;
                if (s <= cb) {
                    const int64_t row = ((s * P.h_kv + j) * 2 + (s == ca ? 1 : 0)) * R + g;
                    ml[i] = P.ws_ml[row];
                    ov[i] = reinterpret_cast<const float4 *>(P.ws_o + row * D)[eq];
                } else {
                    ml[i] = make_float2(-INFINITY, 0.f);
                    ov[i] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
            float mb = ml[0].x;
#pragma unroll
            for (int i = 1; i < kBatch; ++i) mb = fmaxf(mb, ml[i].x);
            // One rescale per batch: fold the batch at its own maximum, then into r
            // (an all-empty batch, e.g. a query token that sees none of these keys,
            // is exponentiated against 0 and stays the identity).
            const float mbr = mb == -INFINITY ? 0.f : mb;
            Running bt = {mb, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                const float f = __builtin_amdgcn_exp2f(ml[i].x - mbr);   // 0 for the padding
                bt.L = __builtin_fmaf(f, ml[i].y, bt.L);
                bt.acc.x = __builtin_fmaf(f, ov[i].x, bt.acc.x);
                bt.acc.y = __builtin_fmaf(f, ov[i].y, bt.acc.y);
                bt.acc.z = __builtin_fmaf(f, ov[i].z, bt.acc.z);
                bt.acc.w = __builtin_fmaf(f, ov[i].w, bt.acc.w);
            }
            fold(r, bt.M, bt.L, bt.acc);
        }
    }
    if (!confirmed()) return false;      // before any barrier or store: uniform over the workgroup
    if constexpr (PL > 1) {
        // Piece lanes of one wavefront sit TP lanes apart: fold them pairwise.
#pragma unroll
        for (int mask = TP; mask < kWave; mask <<= 1) {
            const Running x = shfl_xor_running(r, mask);
            fold(r, x.M, x.L, x.acc);
        }
        const int wv = tid / kWave;
        const int ln = tid % kWave;
        if (ln < TP) s_run[wv][ln] = r;
        __syncthreads();
        if (wv != 0 || ln >= TP) return true;
#pragma unroll
        for (int i = 1; i < Lay::kWaves; ++i) {
            const Running x = s_run[i][ln];
            fold(r, x.M, x.L, x.acc);
        }
    }
    if (active) {
        const float inv = r.L > 0.f ? 1.0f / r.L : 0.f;   // a query token with no key gives 0
        store_quad<kOut>(orow, eq, make_float4(r.acc.x * inv, r.acc.y * inv, r.acc.z * inv, r.acc.w * inv));
    }
    return true;
}

template <int kOut, int D, int kThreadsM, int kRows, int kQuads>
__global__ __launch_bounds__(kThreadsM) void merge_kernel(DecodeParams P) {
    using Lay = MergeLayout<kThreadsM, kRows, kQuads>;
    constexpr int kSlices = D / (4 * kQuads);
    static_assert(kSlices * 4 * kQuads == D, "layout");
    __shared__ Running s_run[Lay::kRunRows][Lay::kRunCols];

    const int G = P.G;
    const int R = P.R;
    const int groups = (R + kRows - 1) / kRows;
    const int blk = static_cast<int>(blockIdx.x) / kSlices;
    const int slice = static_cast<int>(blockIdx.x) - blk * kSlices;
    const int unit = blk / groups;
    const int r0 = (blk - unit * groups) * kRows;
    const int b = unit / P.h_kv;
    const int j = unit - b * P.h_kv;
    const int tid = static_cast<int>(threadIdx.x);
    const int eq = slice * kQuads + tid % kQuads;    // element quad within the row
    const int hh = (tid / kQuads) % kRows;
    const int pl = tid / Lay::TP;
    const int g = r0 + hh;                           // row within the kv head
    const bool active = g < R;
    const int tq = (active ? g : R - 1) / G;
    const int gh = (active ? g : R - 1) - tq * G;
    uint8_t *orow = P.o + ((static_cast<int64_t>(b) * P.t_q + tq) * P.h_q + j * G + gh) * D *
                              (kOut == kF32 ? 4 : 2);
    if (P.expect_len > 0) {
        // One sequence, its length predicted by the caller's bound: the piece loads
        // need not wait for the read of seq_lens (a buffer load, so that it stays a
        // vector load, waited for only where the length is compared).  A wrong
        // prediction continues below with the length as stored.
        const int got = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(P.seq_lens, 4), 0, 0, 0));
        if (merge_pieces<kOut, D, kThreadsM, kRows, kQuads, true>(P, s_run, j, g, eq, active, orow, P.expect_len,
                                                                   P.expect_len, 0, got))
            return;
    }
    // Up to 64 sequences: one read of seq_lens gives the length, total and prefix.
    const bool few = P.batch <= kWave;
    FirstLens fl;
    if (few) fl.load(P.seq_lens, P.batch);
    const int len = few ? fl.len(b) : uniform32(seq_len_at(P.seq_lens, b));
    if (len == 0) {
        if (pl == 0 && active) store_quad<kOut>(orow, eq, make_float4(0.f, 0.f, 0.f, 0.f));
        return;
    }
    const int64_t total = few ? fl.total() : total_len(P.seq_lens, P.batch);
    const int64_t ustart = few ? fl.prefix(b) : prefix_len(P.seq_lens, b);
    merge_pieces<kOut, D, kThreadsM, kRows, kQuads, false>(P, s_run, j, g, eq, active, orow, len, total, ustart, 0);
}

template <int kOut, int D>
void launch_d(const DecodeParams &P, int blocks, int threads, int slices, hipStream_t stream) {
    constexpr int QD = D / 4;
    if (slices > 1)          // split: one row, kMergeSliceQuads quads, 1024 threads
        hipLaunchKernelGGL((merge_kernel<kOut, D, kMergeThreadsWide, 1, kMergeSliceQuads>), dim3(blocks),
                           dim3(kMergeThreadsWide), 0, stream, P);
    else if (threads == kMergeThreadsWide)   // wide: one row, all of d
        hipLaunchKernelGGL((merge_kernel<kOut, D, kMergeThreadsWide, 1, QD>), dim3(blocks),
                           dim3(kMergeThreadsWide), 0, stream, P);
    else                     // narrow: kMergeThreadsNarrow / QD rows, one piece lane
        hipLaunchKernelGGL((merge_kernel<kOut, D, kMergeThreadsNarrow, kMergeThreadsNarrow / QD, QD>),
                           dim3(blocks), dim3(kMergeThreadsNarrow), 0, stream, P);
}

template <int kOut>
hipError_t launch_out(const DecodeParams &P, int D, int blocks, int threads, int slices, hipStream_t stream) {
    if (D == 128)
        launch_d<kOut, 128>(P, blocks, threads, slices, stream);
    else
        launch_d<kOut, 64>(P, blocks, threads, slices, stream);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const DecodeParams &P, int out_dtype, int D, int blocks, int threads, int slices,
                        hipStream_t stream) {
    if (out_dtype == kF32) return launch_out<kF32>(P, D, blocks, threads, slices, stream);
    if (out_dtype == kF16) return launch_out<kF16>(P, D, blocks, threads, slices, stream);
    return launch_out<0>(P, D, blocks, threads, slices, stream);
}

}  // namespace gqa
