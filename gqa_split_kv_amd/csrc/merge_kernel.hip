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
// Layout: a workgroup covers (sequence, kv head) and a group of rows (query
// token, query head).  Thread (pl, h, eq) owns four consecutive elements
// d = 4eq .. 4eq+3 of row h
// and the pieces s = ca + pl, ca + pl + PL, ...; it loads eight pieces at a time
// and folds them into a running (M, L, acc) with the merge rule; the piece lanes
// are then folded through LDS in ascending order, so the result is
// deterministic.  The narrow layout (one piece lane, up to 8 heads per
// workgroup at d 128) serves sequences cut into few pieces; the wide one (one
// head, 32 piece lanes at d 128) serves a long sequence cut into many.  Also
// writes zeros for an empty sequence.
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
// maximum, both sides rescaled by 2^(old - new), sums added.
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
    r.L = r.L * a + l * f;
    r.acc.x = r.acc.x * a + o.x * f;
    r.acc.y = r.acc.y * a + o.y * f;
    r.acc.z = r.acc.z * a + o.z * f;
    r.acc.w = r.acc.w * a + o.w * f;
    r.M = Mn;
}

// Workgroup layout: kRows rows x PL piece lanes x QD element quads; a row is one
// (query token, query head) of the kv head, row = t * G + g.
template <int kOut, int D, int kThreadsM, int kRows>
__global__ __launch_bounds__(kThreadsM) void merge_kernel(DecodeParams P) {
    constexpr int QD = D / 4;                        // element quads per row
    constexpr int PL = kThreadsM / (QD * kRows);     // piece lanes
    constexpr int kBatch = 8;                        // pieces in flight per thread
    static_assert(PL >= 1 && PL * QD * kRows == kThreadsM, "layout");
    __shared__ Running s_run[PL > 1 ? PL : 1][kRows][QD];

    const int G = P.G;
    const int R = P.R;
    const int groups = (R + kRows - 1) / kRows;
    const int unit = static_cast<int>(blockIdx.x) / groups;
    const int r0 = (static_cast<int>(blockIdx.x) - unit * groups) * kRows;
    const int b = unit / P.h_kv;
    const int j = unit - b * P.h_kv;
    const int tid = static_cast<int>(threadIdx.x);
    const int eq = tid % QD;
    const int hh = (tid / QD) % kRows;
    const int pl = tid / (QD * kRows);
    const int g = r0 + hh;                           // row within the kv head
    const bool active = g < R;
    const int tq = (active ? g : R - 1) / G;
    const int gh = (active ? g : R - 1) - tq * G;
    const int len = uniform32(seq_len_at(P.seq_lens, b));
    uint8_t *orow = P.o + ((static_cast<int64_t>(b) * P.t_q + tq) * P.h_q + j * G + gh) * D *
                              (kOut == kF32 ? 4 : 2);
    if (len == 0) {
        if (pl == 0 && active) store_quad<kOut>(orow, eq, make_float4(0.f, 0.f, 0.f, 0.f));
        return;
    }
    const int64_t total = total_len(P.seq_lens, P.batch);
    const int64_t chunk = chunk_keys(total, P.num_chunks / P.h_kv, P.min_chunk);
    const int64_t ustart = prefix_len(P.seq_lens, b);
    const int64_t ca = ustart / chunk;   // token ranges holding this sequence
    const int64_t cb = (ustart + len - 1) / chunk;
    if (ca == cb) return;                // written whole by the sweep kernel

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
                bt.L += f * ml[i].y;
                bt.acc.x += f * ov[i].x;
                bt.acc.y += f * ov[i].y;
                bt.acc.z += f * ov[i].z;
                bt.acc.w += f * ov[i].w;
            }
            fold(r, bt.M, bt.L, bt.acc);
        }
    }
    if constexpr (PL > 1) {
        s_run[pl][hh][eq] = r;
        __syncthreads();
        if (pl != 0) return;
#pragma unroll
        for (int i = 1; i < PL; ++i) {
            const Running x = s_run[i][hh][eq];
            fold(r, x.M, x.L, x.acc);
        }
    }
    if (active) {
        const float inv = r.L > 0.f ? 1.0f / r.L : 0.f;   // a query token with no key gives 0
        store_quad<kOut>(orow, eq, make_float4(r.acc.x * inv, r.acc.y * inv, r.acc.z * inv, r.acc.w * inv));
    }
}

template <int kOut>
hipError_t launch_out(const DecodeParams &P, int D, int blocks, int threads, hipStream_t stream) {
    // Narrow: 256 threads covering 256/(D/4) heads with one piece lane each
    // (few pieces per sequence).  Wide: 1024 threads, one head, 1024/(D/4) piece lanes.
    if (threads == kMergeThreadsWide) {
        if (D == 128)
            hipLaunchKernelGGL((merge_kernel<kOut, 128, kMergeThreadsWide, 1>), dim3(blocks), dim3(kMergeThreadsWide), 0, stream, P);
        else
            hipLaunchKernelGGL((merge_kernel<kOut, 64, kMergeThreadsWide, 1>), dim3(blocks), dim3(kMergeThreadsWide), 0, stream, P);
    } else {
        if (D == 128)
            hipLaunchKernelGGL((merge_kernel<kOut, 128, kMergeThreadsNarrow, 8>), dim3(blocks), dim3(kMergeThreadsNarrow), 0, stream, P);
        else
            hipLaunchKernelGGL((merge_kernel<kOut, 64, kMergeThreadsNarrow, 16>), dim3(blocks), dim3(kMergeThreadsNarrow), 0, stream, P);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const DecodeParams &P, int out_dtype, int D, int blocks, int threads,
                        hipStream_t stream) {
    if (out_dtype == kF32) return launch_out<kF32>(P, D, blocks, threads, stream);
    if (out_dtype == kF16) return launch_out<kF16>(P, D, blocks, threads, stream);
    return launch_out<0>(P, D, blocks, threads, stream);
}

}  // namespace gqa
