// host.h -- internal host-side declarations shared by the C-ABI layer (api.cpp),
// the pure-C++ validation/planning (plan.cpp) and the kernel launchers
// (sweep_kernel.hip, merge_kernel.hip, prefill_kernel.hip).  Not part of the
// public interface.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gqa_decode.h"
#include "gqa_prefill.h"

namespace gqa {

#ifndef GQA_SWEEP_WAVES
#define GQA_SWEEP_WAVES 4
#endif
// Wavefronts per workgroup of the sweep kernel.
constexpr int kWavesPerBlock = GQA_SWEEP_WAVES;
constexpr int kThreads = 64 * kWavesPerBlock;
// Merge kernel layouts.  Narrow: 256 threads over whole rows with one piece lane
// (8 rows at d_head 128), for sequences cut into few pieces.  Wide: 1024 threads,
// one row, 1024 / (d_head / 4) piece lanes, for sequences cut into many.  Split:
// 1024 threads, one row, a slice of kMergeSliceQuads * 4 elements of d, 128 piece
// lanes, when the wide layout would launch fewer than kSplitMergeBelowBlocks
// workgroups (a few long sequences: most of the GPU would sit idle).
constexpr int kMergeThreadsNarrow = 256;
constexpr int kMergeThreadsWide = 1024;
constexpr int kMergeSliceQuads = 8;
constexpr int kWideMergePieces = 32;   // expected pieces per sequence above which the merge is wide
constexpr int kSplitMergeBelowBlocks = 256;
// Prefill kernel: workgroups of GQA_PREFILL_THREADS threads owning GQA_PREFILL_ROWS
// rows (GQA_PREFILL_ROWS / G tokens x G heads), 32 rows per wavefront.
#ifndef GQA_PREFILL_THREADS
#define GQA_PREFILL_THREADS 512
#endif
#ifndef GQA_PREFILL_ROWS
#define GQA_PREFILL_ROWS 256
#endif
constexpr int kPrefillThreads = GQA_PREFILL_THREADS;
constexpr int kPrefillRows = GQA_PREFILL_ROWS;
// Keys per step of the prefill (one block of its transposed V copy), and the
// workgroup size of the kernel that makes the copy.
constexpr int kPrefillStepKeys = 64;
constexpr int kVprepThreads = 256;
constexpr int kMaxRows = 64;        // decode: rows per kv head, G * t_q (up to four 16-row tiles per wavefront)
constexpr int kMaxChunks = 1 << 24;
constexpr int kMaxPrefillBlocks = 1 << 20;
constexpr int kMaxHeadsKv = 1 << 16;   // keeps 16 key rows of lane offsets within 32 bits
constexpr int kMaxMinChunk = 1 << 30;
constexpr int kAutoMinChunk = 64;   // default smallest token range (two 32-key steps)
// Automatic plan: at most this many sweep wavefronts per compute unit, i.e. one
// per SIMD.  Measured on MI355X (70B-shaped ragged batch): with the MFMA-based
// step the SIMD is lightly loaded, one wavefront per SIMD with one step of
// prefetch saturates HBM, and a second wavefront on the same SIMD only competes
// for issue (the younger one is served later, which leaves a tail at the end of
// the equal-work stream-K sweep).
constexpr int kAutoWavesPerCu = 4;

// Sets the thread-local error message and returns `status`.
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Argument checks in a fixed order (null, shape, support, alignment, scale,
// tuning ranges, and the caller workspace when num_chunks is explicit).
int validate(const gqa_decode_args *a);

// Host checks of a prefill call (status, message via fail()); the caller
// workspace is checked too unless `check_workspace` is false.
int validate_prefill(const gqa_prefill_args *a, bool check_workspace = true);

// Prefill workspace: the transposed fp16 copy of V, [h_kv][nvb][D][64], at 0 and
// the step flags [h_kv][nvb] (bytes) at flags_offset, nvb = ceil(total_tokens /
// 64) + batch (at least the number of 64-key steps over all sequences).  bytes = 0
// (and nvb = 0) when the call makes no copy (split_pv = 1 or total_tokens = 0).
struct PrefillWorkspace {
    size_t flags_offset;
    size_t queue_offset;   // the tile queue's counter (zeroed by the V copy kernel)
    size_t bytes;
    int64_t nvb;
};
PrefillWorkspace prefill_workspace(const gqa_prefill_args *a);
constexpr int64_t kMaxPrefillRowsHeads = int64_t(1) << 37;   // total_tokens * h_kv limit

// Workspace layout for `num_chunks` wavefronts: the fused merge's counters in a
// fixed reserve at the start (every plan keeps it, so no call's partials ever
// land on another's counters), then two partial-triple slots per wavefront, each
// R = G * t_q rows of (O[D] fp32) plus (m, l) fp32, and for the fused merge two
// more slots per workgroup.
constexpr size_t kCounterBytes = GQA_DECODE_COUNTER_BYTES;
constexpr int64_t kCounterWords = static_cast<int64_t>(kCounterBytes / 4);
struct WorkspaceLayout {
    size_t counter_offset;   // uint32 [levels][num_chunks / kWavesPerBlock][2]  (0)
    size_t o_offset;         // float  [num_chunks][2][R][D]
    size_t ml_offset;        // float2 [num_chunks][2][R]
    size_t o2_offset;        // float  [num_chunks / kWavesPerBlock][2][R][D]   (fused)
    size_t ml2_offset;       // float2 [num_chunks / kWavesPerBlock][2][R]      (fused)
    size_t bytes;
};
WorkspaceLayout workspace_layout(int64_t num_chunks, int rows, int D, bool fused);

// Fused merge: chosen automatically for at most this many (sequence, kv head)
// units when the caller's max_seq_len hint shows that every sequence fits in one
// workgroup's key span (kWavesPerBlock * min_chunk keys), so that no sequence
// needs more than one exchange between workgroups; measured on MI355X, the
// fused form then saves the merge launch (tiny workload 10.6 -> 8.4 us), while
// for long sequences over few units each level of its tree (a device-coherent
// store, an atomic and a coherent load, ~3 us) costs as much as the merge kernel.
// Also the bound on the tree's fold volume per node (fan-in K = the largest power
// of two with K * R * d_head * 4 bytes within it, clamped to [2, 64]).
constexpr int kFusedMaxUnits = 16;
constexpr int kFoldBytes = 64 * 1024;
constexpr int kMaxFanIn = 64;

int make_plan(const gqa_decode_args *a, int num_cus, int waves_per_cu, gqa_decode_plan *plan);

}  // namespace gqa
