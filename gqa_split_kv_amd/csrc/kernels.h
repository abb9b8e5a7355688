// kernels.h -- parameters and launchers of the gfx950 kernels (sweep_kernel.hip,
// merge_kernel.hip, prefill_kernel.hip).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host.h"

namespace gqa {

struct DecodeParams {
    const uint8_t *q;          // [batch, t_q, h_q, D] in_dtype
    const uint8_t *k;          // [sum(seq_lens), h_kv, D] in_dtype
    const uint8_t *v;
    uint8_t *o;                // [batch, t_q, h_q, D] out_dtype
    const int32_t *seq_lens;   // [batch]
    float *ws_o;               // [num_chunks][2][R][D]   unnormalised O of a piece
    float2 *ws_ml;             // [num_chunks][2][R]      (m in log2 units, l)
    // Fused merge only (fused_kernel): the workgroup-level pieces and the tree's counters.
    float *ws2_o;              // [num_chunks / kWavesPerBlock][2][R][D]
    float2 *ws2_ml;            // [num_chunks / kWavesPerBlock][2][R]
    uint32_t *counters;        // [levels][num_chunks / kWavesPerBlock][2], zero before and after a call
    int32_t fold_k_log2;       // fan-in of the tree: 2^fold_k_log2
    int32_t batch, h_q, h_kv, G;
    int32_t t_q;               // query tokens per sequence
    int32_t R;                 // rows per kv head: G * t_q (row = t * G + g), up to 64
    int32_t num_chunks, min_chunk;
    int32_t expect_len;        // one sequence: the length the caller's bound predicts, else 0
    float scale_log2;          // scale * log2(e)
};

// Enqueues the sweep (partial) kernel: `blocks` workgroups of kThreads.  Dtypes
// are GQA_DTYPE_* codes.  With `fused`, the single-kernel form (fused_kernel:
// the merge runs inside the sweep, no merge kernel follows; blocks =
// num_chunks / kWavesPerBlock).
hipError_t launch_sweep(const DecodeParams &P, int in_dtype, int out_dtype, int D, int blocks, bool fused,
                        hipStream_t stream);

// Resident workgroups of the sweep kernel per compute unit.
hipError_t sweep_occupancy(int in_dtype, int out_dtype, int D, int *blocks_per_cu);

// Enqueues the merge kernel: `blocks` workgroups of `threads` (kMergeThreadsNarrow
// or kMergeThreadsWide), each row's d cut into `slices` slices (1, or d / 32 for
// the split layout), as the plan sets them.
hipError_t launch_merge(const DecodeParams &P, int out_dtype, int D, int blocks, int threads, int slices,
                        hipStream_t stream);

// Causal prefill: every token of every sequence attends to keys 0 .. itself.
struct PrefillParams {
    const uint8_t *q;          // [sum(seq_lens), h_q, D] in_dtype
    const uint8_t *k;          // [sum(seq_lens), h_kv, D] in_dtype
    const uint8_t *v;
    uint8_t *o;                // [sum(seq_lens), h_q, D] out_dtype
    const int32_t *seq_lens;   // [batch]
    int32_t batch, h_q, h_kv, G;
    float scale_log2;          // scale * log2(e)
    int32_t split_pv;          // 1: split P V products everywhere
    const uint8_t *vt;         // [h_kv][nvb][D][64] fp16: V^T of every sequence's 64-key steps, or null
    const uint8_t *vflags;     // [h_kv][nvb] 1 = that step's V is not fit for fp16 (bf16 input)
    int64_t nvb;               // step blocks per kv head in vt (0: no copy)
    // Tile queue: the next work item to take, zeroed by the V copy kernel before
    // the prefill kernel starts; null = the fixed snake order (no workspace).
    unsigned long long *queue;
};

// Transposed fp16 copy of V for the prefill's fast loop (vprep_kernel).
struct VprepParams {
    const uint8_t *v;          // [sum(seq_lens), h_kv, D] in_dtype
    uint8_t *vt;               // [h_kv][nvb][D][64] fp16
    uint8_t *flags;            // [h_kv][nvb]
    const int32_t *seq_lens;   // [batch]
    int32_t batch, h_kv;
    int64_t nvb;               // >= sum over sequences of ceil(len / 64)
    unsigned long long *queue; // set to 0 (the prefill's tile queue)
};

// Enqueues vprep_kernel over h_kv * nvb workgroups.
hipError_t launch_vprep(const VprepParams &p, int in_dtype, int D, hipStream_t stream);

// Enqueues the prefill kernel: `blocks` workgroups of kPrefillThreads.
hipError_t launch_prefill(const PrefillParams &P, int in_dtype, int out_dtype, int D, int blocks,
                          hipStream_t stream);

// Resident workgroups of the prefill kernel per compute unit.
hipError_t prefill_occupancy(int in_dtype, int out_dtype, int D, int *blocks_per_cu);

}  // namespace gqa
