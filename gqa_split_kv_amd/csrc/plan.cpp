// plan.cpp -- argument validation and launch planning.  Pure C++: no HIP
// header, no device access, so every rule here is testable on a host without a
// GPU through gqa_decode_validate / gqa_decode_make_plan.
//
// The rules follow the launch-argument checks of the pages' kernels: reject
// bad arguments before any work is enqueued (kernbench2 page
// "_gqa_attention_decode_long.py", the `sub_w` check that raises before the
// kernel body; sglang page "tp_qknorm.cuh", the host launcher's shape, dtype and
// 16-byte alignment checks).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "host.h"

namespace gqa {

namespace {
thread_local std::string g_last_error;
}

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

void clear_error() { g_last_error.clear(); }

const char *last_error() { return g_last_error.c_str(); }

static bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

WorkspaceLayout workspace_layout(int64_t num_chunks, int rows, int D, bool fused) {
    WorkspaceLayout L;
    const size_t slots = static_cast<size_t>(num_chunks) * 2 * static_cast<size_t>(rows);
    L.counter_offset = 0;
    L.o_offset = kCounterBytes;
    L.ml_offset = round_up(L.o_offset + slots * static_cast<size_t>(D) * sizeof(float), 256);
    L.bytes = round_up(L.ml_offset + slots * 2 * sizeof(float), 256);
    L.o2_offset = L.ml2_offset = L.bytes;
    if (fused) {
        const size_t slots2 = static_cast<size_t>(num_chunks / kWavesPerBlock) * 2 * static_cast<size_t>(rows);
        L.o2_offset = L.bytes;
        L.ml2_offset = round_up(L.o2_offset + slots2 * static_cast<size_t>(D) * sizeof(float), 256);
        L.bytes = round_up(L.ml2_offset + slots2 * 2 * sizeof(float), 256);
    }
    return L;
}

// Fan-in of the fused merge's tree for R rows of d_head: the largest power of two
// K with K * R * D * 4 <= kFoldBytes, within [2, kMaxFanIn].
static int fold_fanin(int rows, int D) {
    int k = 2;
    while (k < kMaxFanIn && static_cast<int64_t>(2 * k) * rows * D * 4 <= kFoldBytes) k *= 2;
    return k;
}

// Tree levels over at most `pieces` pieces per sequence with fan-in k.
static int fold_levels(int64_t pieces, int k) {
    int levels = 1;
    for (int64_t span = k; span < pieces; span *= k) ++levels;
    return levels;
}

// Rows of the MFMA N axis per kv head: G query heads x t_q query tokens.
static int rows_per_kv_head(const gqa_decode_args *a) {
    return (a->h_q / a->h_kv) * (a->t_q > 0 ? a->t_q : 1);
}

static int check_basic(const gqa_decode_args *a) {
    if (!a) return fail(GQA_ERR_NULL, "args is NULL");
    if (!a->q || !a->k || !a->v || !a->o || !a->seq_lens)
        return fail(GQA_ERR_NULL, "q, k, v, o and seq_lens must be non-NULL");
    if (a->batch <= 0 || a->h_q <= 0 || a->h_kv <= 0)
        return fail(GQA_ERR_SHAPE, "batch (%d), h_q (%d) and h_kv (%d) must be positive", a->batch,
                    a->h_q, a->h_kv);
    if (a->h_q % a->h_kv != 0)
        return fail(GQA_ERR_SHAPE, "h_q (%d) is not a multiple of h_kv (%d)", a->h_q, a->h_kv);
    if (static_cast<int64_t>(a->batch) * a->h_q > 0x7fffffff)
        return fail(GQA_ERR_SHAPE, "batch * h_q exceeds 2^31-1");
    if (a->h_kv > kMaxHeadsKv)
        return fail(GQA_ERR_UNSUPPORTED, "h_kv %d exceeds %d", a->h_kv, kMaxHeadsKv);
    const int G = a->h_q / a->h_kv;
    if (G > kMaxRows)
        return fail(GQA_ERR_UNSUPPORTED, "G = h_q/h_kv = %d exceeds %d", G, kMaxRows);
    if (a->t_q < 0) return fail(GQA_ERR_SHAPE, "t_q %d is negative", a->t_q);
    const int tq = a->t_q > 0 ? a->t_q : 1;
    if (static_cast<int64_t>(G) * tq > kMaxRows)
        return fail(GQA_ERR_UNSUPPORTED, "G * t_q = %d * %d exceeds %d rows", G, tq, kMaxRows);
    if (static_cast<int64_t>(a->batch) * tq * a->h_q > 0x7fffffff)
        return fail(GQA_ERR_SHAPE, "batch * t_q * h_q exceeds 2^31-1");
    if (a->d_head != 64 && a->d_head != 128)
        return fail(GQA_ERR_UNSUPPORTED, "d_head %d not supported (64 or 128)", a->d_head);
    const bool pair_ok = (a->in_dtype == GQA_DTYPE_BF16 && a->out_dtype == GQA_DTYPE_BF16) ||
                         (a->in_dtype == GQA_DTYPE_BF16 && a->out_dtype == GQA_DTYPE_F32) ||
                         (a->in_dtype == GQA_DTYPE_F32 && a->out_dtype == GQA_DTYPE_F32) ||
                         (a->in_dtype == GQA_DTYPE_F16 && a->out_dtype == GQA_DTYPE_F16) ||
                         (a->in_dtype == GQA_DTYPE_F16 && a->out_dtype == GQA_DTYPE_F32);
    if (!pair_ok)
        return fail(GQA_ERR_UNSUPPORTED, "dtype pair (in %d, out %d) not supported", a->in_dtype,
                    a->out_dtype);
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->o, 16))
        return fail(GQA_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
    if (!aligned(a->seq_lens, 4)) return fail(GQA_ERR_ALIGN, "seq_lens must be 4-byte aligned");
    if (!std::isfinite(a->scale)) return fail(GQA_ERR_SCALE, "scale is not finite");
    if (a->num_chunks < 0 || a->num_chunks > kMaxChunks)
        return fail(GQA_ERR_ARG, "num_chunks %d out of range [0, %d]", a->num_chunks, kMaxChunks);
    if (a->min_chunk < 0 || a->min_chunk > kMaxMinChunk)
        return fail(GQA_ERR_ARG, "min_chunk %d out of range [0, %d]", a->min_chunk, kMaxMinChunk);
    if (a->max_seq_len < 0) return fail(GQA_ERR_ARG, "max_seq_len %d is negative", a->max_seq_len);
    if (a->merge < GQA_MERGE_AUTO || a->merge > GQA_MERGE_FUSED)
        return fail(GQA_ERR_ARG, "merge %d is not GQA_MERGE_AUTO, GQA_MERGE_KERNEL or GQA_MERGE_FUSED", a->merge);
    return GQA_OK;
}

// Wavefront count and merge form of a call: `chunks` requested (explicit or
// automatic) -> the count launched, and whether the merge is fused (with its
// fan-in and levels).  Returns a status.
struct Shape {
    int64_t chunks;
    bool fused;
    int fanin, levels;
};

static int resolve_shape(const gqa_decode_args *a, int64_t chunks, Shape *out) {
    const int R = rows_per_kv_head(a);
    const int64_t units = static_cast<int64_t>(a->batch) * a->h_kv;
    // One wavefront per kv head of every token range: a multiple of h_kv.
    int64_t plain = chunks / a->h_kv * a->h_kv;
    if (plain < a->h_kv) plain = a->h_kv;
    // Fused: whole workgroups of consecutive ranges of one kv head, and no more
    // wavefronts than the counter reserve serves (levels x 2 counters per workgroup).
    const int64_t unit = static_cast<int64_t>(a->h_kv) * kWavesPerBlock;
    const int fanin = fold_fanin(R, a->d_head);
    auto counters = [&](int64_t n) { return fold_levels(n / unit, fanin) * 2 * (n / kWavesPerBlock); };
    int64_t fchunks = chunks / unit * unit;
    if (fchunks < unit) fchunks = unit;
    const bool capped = counters(fchunks) > kCounterWords;
    while (fchunks > unit && counters(fchunks) > kCounterWords) fchunks = (fchunks / 2) / unit * unit;
    if (fchunks < unit) fchunks = unit;
    const int levels = fold_levels(fchunks / unit, fanin);
    const bool fits = counters(fchunks) <= kCounterWords;
    bool fused;
    if (a->merge == GQA_MERGE_FUSED) {
        if (!fits)
            return fail(GQA_ERR_ARG, "the fused merge needs %lld counters for h_kv %d, above the %lld the reserve "
                        "holds", static_cast<long long>(counters(fchunks)), a->h_kv,
                        static_cast<long long>(kCounterWords));
        fused = true;
    } else if (a->merge == GQA_MERGE_KERNEL) {
        fused = false;
    } else {
        const int64_t min_chunk = a->min_chunk > 0 ? a->min_chunk : kAutoMinChunk;
        fused = fits && !capped && units <= kFusedMaxUnits && a->max_seq_len > 0 &&
                a->max_seq_len <= kWavesPerBlock * min_chunk;
    }
    out->chunks = fused ? fchunks : plain;
    out->fused = fused;
    out->fanin = fused ? fanin : 0;
    out->levels = fused ? levels : 0;
    return GQA_OK;
}

static int check_workspace(const gqa_decode_args *a, size_t need) {
    if (!a->workspace) return GQA_OK;
    if (!aligned(a->workspace, 256)) return fail(GQA_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (a->workspace_bytes < need)
        return fail(GQA_ERR_WORKSPACE, "workspace holds %zu bytes, the call needs %zu",
                    a->workspace_bytes, need);
    return GQA_OK;
}

int validate(const gqa_decode_args *a) {
    int st = check_basic(a);
    if (st != GQA_OK) return st;
    if (a->num_chunks > 0) {
        Shape sh;
        st = resolve_shape(a, a->num_chunks, &sh);
        if (st != GQA_OK) return st;
        const WorkspaceLayout L = workspace_layout(sh.chunks, rows_per_kv_head(a), a->d_head, sh.fused);
        st = check_workspace(a, L.bytes);
        if (st != GQA_OK) return st;
    }
    return GQA_OK;
}

PrefillWorkspace prefill_workspace(const gqa_prefill_args *a) {
    PrefillWorkspace W = {0, 0, 0, 0};
    if (a->split_pv != 0 || a->total_tokens <= 0) return W;
    W.nvb = (a->total_tokens + kPrefillStepKeys - 1) / kPrefillStepKeys + a->batch;
    const size_t blocks = static_cast<size_t>(W.nvb) * static_cast<size_t>(a->h_kv);
    W.flags_offset = round_up(blocks * static_cast<size_t>(a->d_head) * kPrefillStepKeys * 2, 256);
    W.queue_offset = round_up(W.flags_offset + blocks, 256);
    W.bytes = W.queue_offset + 256;
    return W;
}

int validate_prefill(const gqa_prefill_args *a, bool check_workspace) {
    if (!a) return fail(GQA_ERR_NULL, "args is NULL");
    if (!a->q || !a->k || !a->v || !a->o || !a->seq_lens)
        return fail(GQA_ERR_NULL, "q, k, v, o and seq_lens must be non-NULL");
    if (a->batch <= 0 || a->h_q <= 0 || a->h_kv <= 0)
        return fail(GQA_ERR_SHAPE, "batch (%d), h_q (%d) and h_kv (%d) must be positive", a->batch,
                    a->h_q, a->h_kv);
    if (a->h_q % a->h_kv != 0)
        return fail(GQA_ERR_SHAPE, "h_q (%d) is not a multiple of h_kv (%d)", a->h_q, a->h_kv);
    if (a->h_kv > kMaxHeadsKv)
        return fail(GQA_ERR_UNSUPPORTED, "h_kv %d exceeds %d", a->h_kv, kMaxHeadsKv);
    const int G = a->h_q / a->h_kv;
    if (G > kMaxRows) return fail(GQA_ERR_UNSUPPORTED, "G = h_q/h_kv = %d exceeds %d", G, kMaxRows);
    if (a->d_head != 64 && a->d_head != 128)
        return fail(GQA_ERR_UNSUPPORTED, "d_head %d not supported (64 or 128)", a->d_head);
    const bool pair_ok = (a->in_dtype == GQA_DTYPE_BF16 && a->out_dtype == GQA_DTYPE_BF16) ||
                         (a->in_dtype == GQA_DTYPE_BF16 && a->out_dtype == GQA_DTYPE_F32) ||
                         (a->in_dtype == GQA_DTYPE_F16 && a->out_dtype == GQA_DTYPE_F16) ||
                         (a->in_dtype == GQA_DTYPE_F16 && a->out_dtype == GQA_DTYPE_F32);
    if (!pair_ok)
        return fail(GQA_ERR_UNSUPPORTED, "prefill dtype pair (in %d, out %d) not supported", a->in_dtype,
                    a->out_dtype);
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->o, 16))
        return fail(GQA_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
    if (!aligned(a->seq_lens, 4)) return fail(GQA_ERR_ALIGN, "seq_lens must be 4-byte aligned");
    if (!std::isfinite(a->scale)) return fail(GQA_ERR_SCALE, "scale is not finite");
    if (a->num_blocks < 0 || a->num_blocks > kMaxPrefillBlocks)
        return fail(GQA_ERR_ARG, "num_blocks %d out of range [0, %d]", a->num_blocks, kMaxPrefillBlocks);
    if (a->split_pv != 0 && a->split_pv != 1) return fail(GQA_ERR_ARG, "split_pv %d is not 0 or 1", a->split_pv);
    if (a->total_tokens < 0 || (a->total_tokens > 0 && a->total_tokens > kMaxPrefillRowsHeads / a->h_kv))
        return fail(GQA_ERR_ARG, "total_tokens %lld out of range [0, 2^37 / h_kv]",
                    static_cast<long long>(a->total_tokens));
    {
        const PrefillWorkspace W = prefill_workspace(a);
        if (W.nvb > 0 && W.nvb > static_cast<int64_t>(0x7fffffff) / a->h_kv)
            return fail(GQA_ERR_ARG, "total_tokens %lld with batch %d and h_kv %d: the V copy needs more than 2^31 "
                        "workgroups", static_cast<long long>(a->total_tokens), a->batch, a->h_kv);
    }
    if (check_workspace && a->workspace) {
        const PrefillWorkspace W = prefill_workspace(a);
        if (W.bytes > 0) {
            if (!aligned(a->workspace, 256)) return fail(GQA_ERR_WORKSPACE, "workspace not 256-byte aligned");
            if (a->workspace_bytes < W.bytes)
                return fail(GQA_ERR_WORKSPACE, "workspace holds %zu bytes, the call needs %zu", a->workspace_bytes,
                            W.bytes);
        }
    }
    return GQA_OK;
}

int make_plan(const gqa_decode_args *a, int num_cus, int waves_per_cu, gqa_decode_plan *plan) {
    int st = check_basic(a);
    if (st != GQA_OK) return st;
    if (!plan) return fail(GQA_ERR_NULL, "plan is NULL");
    int64_t chunks = a->num_chunks;
    if (chunks == 0) {
        if (num_cus <= 0 || waves_per_cu <= 0)
            return fail(GQA_ERR_ARG, "automatic num_chunks needs num_cus (%d) and waves_per_cu (%d) > 0",
                        num_cus, waves_per_cu);
        chunks = static_cast<int64_t>(num_cus) * (waves_per_cu < kAutoWavesPerCu ? waves_per_cu : kAutoWavesPerCu);
        if (chunks > kMaxChunks) chunks = kMaxChunks;
    }
    Shape sh;
    st = resolve_shape(a, chunks, &sh);
    if (st != GQA_OK) return st;
    chunks = sh.chunks;
    if (chunks > kMaxChunks) return fail(GQA_ERR_ARG, "h_kv %d needs more than %d wavefronts", a->h_kv, kMaxChunks);
    const WorkspaceLayout L = workspace_layout(chunks, rows_per_kv_head(a), a->d_head, sh.fused);
    st = check_workspace(a, L.bytes);
    if (st != GQA_OK) return st;
    plan->num_chunks = static_cast<int32_t>(chunks);
    plan->min_chunk = a->min_chunk > 0 ? a->min_chunk : kAutoMinChunk;
    plan->split_blocks = static_cast<int32_t>((chunks + kWavesPerBlock - 1) / kWavesPerBlock);
    plan->fused = sh.fused ? 1 : 0;
    plan->fold_fanin = sh.fanin;
    plan->fold_levels = sh.levels;
    plan->workspace_bytes = L.bytes;
    if (sh.fused) {
        plan->merge_threads = plan->merge_slices = plan->merge_blocks = 0;
        return GQA_OK;
    }
    // Expected pieces per sequence: token ranges per sequence on average.
    const int64_t ranges = chunks / a->h_kv;
    const int R = rows_per_kv_head(a);
    const bool wide = ranges / a->batch > kWideMergePieces;
    const bool split = wide && static_cast<int64_t>(a->batch) * a->h_kv * R < kSplitMergeBelowBlocks;
    plan->merge_threads = wide ? kMergeThreadsWide : kMergeThreadsNarrow;
    plan->merge_slices = split ? a->d_head / (4 * kMergeSliceQuads) : 1;
    const int rows_per_block = wide ? 1 : kMergeThreadsNarrow / (a->d_head / 4);
    plan->merge_blocks = a->batch * a->h_kv * ((R + rows_per_block - 1) / rows_per_block) * plan->merge_slices;
    return GQA_OK;
}

}  // namespace gqa
