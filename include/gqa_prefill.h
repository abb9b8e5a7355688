/*
 * gqa_prefill.h -- C ABI of the causal grouped-query-attention prefill in
 * libgqa_decode.so (MI355X, gfx950).
 *
 * The operation (kernbench2 page "_gqa_attention_decode_long.py", commit
 * description: the long-context prefill panel with T_q = S_kv, d_head 128 and one
 * KV group, the query axis split across workers with disjoint output rows): the
 * decode operation of gqa_decode.h with every token of a sequence as a query.
 * For every sequence b < batch, token t < S = seq_lens[b] (negative counts as 0),
 * query head h < h_q, with G = h_q / h_kv, kv head j = h / G and
 * base = seq_lens[0] + ... + seq_lens[b-1]:
 *
 *   s_u              = scale * sum_i q[base+t, h, i] * k[base+u, j, i]     u <= t
 *   o[base+t, h, :]  = sum_{u <= t} softmax(s)_u * v[base+u, j, :]
 *
 * i.e. causal attention of each sequence over its own keys (the queries are the
 * sequence's own tokens, key u visible to token t iff u <= t).  The page says
 * nothing of the mask; this is the multi-token decode rule of gqa_decode.h with
 * t_q = S.  fp32 accumulation; a 16-bit output is the nearest-even rounding of the
 * fp32 result.
 *
 * Tensor layouts (row-major, contiguous, device memory of the current HIP device,
 * owned by the caller; the library never frees or keeps them):
 *   q, o      [sum(seq_lens), h_q, d_head]    in_dtype / out_dtype, sequences packed
 *   k, v      [sum(seq_lens), h_kv, d_head]   in_dtype, packed the same way
 *   seq_lens  int32[batch], device memory, read only by the kernel
 *
 * Supported: d_head in {64, 128}; G in 1..64 (a 256-row tile holds floor(256 / G)
 * tokens x G heads); (in, out) dtypes (bf16, bf16),
 * (bf16, f32), (f16, f16), (f16, f32).  q, k, v, o 16-byte aligned, seq_lens
 * 4-byte aligned.  Every output row is written by exactly one workgroup (no
 * cross-workgroup reduction).
 *
 * Cost of wide groups: a tile sweeps its keys in 64-key steps of 256 rows x 64
 * keys whatever G is, so K/V staging per step, and per flop, does not grow with G;
 * a G of 32 or 64 only makes more, shorter tiles (8 or 4 tokens), each staging
 * its own key prefix, and the work grows with h_q like the flops.  Measured on
 * one 32768-token sequence, one kv head, d_head 128: G 8, 16, 32 and 64 all run
 * at 1.23-1.25 PFLOP/s (1.79, 3.55, 7.08, 14.13 ms per call).  G not dividing 256
 * leaves 256 mod G rows of each tile idle.
 *
 * Workspace: the default precision mode (split_pv = 0) with total_tokens > 0
 * uses one -- V transposed and in fp16, 64 keys of one sequence at a time
 * (nvb = ceil(total_tokens / 64) + batch blocks of d_head x 64 values per kv
 * head), one flag byte per block and kv head, and the 8-byte counter of the
 * queue the workgroups take their tiles from, all rewritten by every call
 * (nothing needs initialising).  gqa_prefill_workspace_bytes() gives its size.
 * With workspace NULL the library uses its own, per (device, stream), grown
 * with hipMalloc (not capturable in a HIP graph; freed by gqa_release()); a
 * caller-provided workspace (256-byte aligned) makes the call capturable, after
 * one uncaptured call of the same dtypes and d_head on the device (as for
 * gqa_decode_ex).  Calls sharing one workspace must be ordered (one stream).
 *
 * Asynchrony and errors as in gqa_decode.h: work is enqueued on `stream`, host
 * errors return a gqa_status before anything is enqueued (o untouched), and
 * gqa_last_error_message() describes the last error of the calling thread.
 */
#ifndef GQA_PREFILL_H
#define GQA_PREFILL_H

#include "gqa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Full argument block.  Zero-initialise it, then set the fields.
 *
 * num_blocks  Workgroups of the persistent grid (each takes tiles of 256 / G
 *             tokens x G heads in a fixed order); 0 = one per resident slot
 *             (compute units x resident workgroups per compute unit).  Range
 *             0..2^20.  The result does not depend on it.
 * split_pv    Precision of the P V product.  0 (default): P is rounded to fp16
 *             (11 significant bits, times a common power of two that cancels) and
 *             V taken in fp16, one matrix-core product, V read from the call's
 *             transposed fp16 copy (bf16 converted); for bf16 input a tile's
 *             sweep switches to the split product from the first 64-key step
 *             whose V has a largest magnitude not in [2^-10, 2^16) (or a
 *             non-finite value), so the fp16 rounding of V never loses range or
 *             precision.  Typical error against the exact result: relative L2
 *             ~1e-4.  1: P split into a high and a low 16-bit part everywhere
 *             (about 16 significant bits, two products, ~1.5x the matrix-core
 *             work); error ~1e-6.  No workspace.
 * total_tokens  Rows held by q, k, v and o: at least sum(seq_lens).  Sizes the
 *             copy of V; 0 means unknown: no copy is made and every step uses
 *             the split product, as with split_pv = 1.  Unused with split_pv = 1.
 * workspace, workspace_bytes  See above; ignored where no workspace is used.
 */
typedef struct gqa_prefill_args {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    const int32_t *seq_lens;
    int32_t batch;
    int32_t h_q;
    int32_t h_kv;
    int32_t d_head;
    float scale;
    int32_t in_dtype;   /* GQA_DTYPE_BF16 or GQA_DTYPE_F16                  */
    int32_t out_dtype;  /* in_dtype or GQA_DTYPE_F32                        */
    int32_t num_blocks;
    void *stream;       /* hipStream_t; NULL = the null stream              */
    int32_t split_pv;   /* 0 or 1, see above                                */
    int64_t total_tokens;
    void *workspace;
    size_t workspace_bytes;
} gqa_prefill_args;

/* gqa_prefill -- bf16 q/k/v in, bf16 o out, total_tokens = sum(seq_lens) rows
 * (the copy of V lives in the library's workspace).  Returns a gqa_status. */
int gqa_prefill(const void *q, const void *k, const void *v, void *o, const int32_t *seq_lens,
                int32_t batch, int64_t total_tokens, int32_t h_q, int32_t h_kv, int32_t d_head, float scale,
                void *stream);

/* gqa_prefill_f16 -- IEEE fp16 q/k/v in, fp16 o out, total_tokens as above. */
int gqa_prefill_f16(const void *q, const void *k, const void *v, void *o, const int32_t *seq_lens,
                    int32_t batch, int64_t total_tokens, int32_t h_q, int32_t h_kv, int32_t d_head, float scale,
                    void *stream);

/* gqa_prefill_ex -- any supported dtype pair and grid size. */
int gqa_prefill_ex(const gqa_prefill_args *args);

/* Host-side checks only (no device access); returns the status gqa_prefill_ex
 * would return before enqueueing anything: GQA_ERR_NULL, GQA_ERR_SHAPE (batch,
 * h_q or h_kv <= 0, h_q not a multiple of h_kv), GQA_ERR_UNSUPPORTED (d_head, G,
 * h_kv above 65536 or the dtype pair), GQA_ERR_ALIGN, GQA_ERR_SCALE, GQA_ERR_ARG
 * (num_blocks out of range, split_pv not 0 or 1, total_tokens negative,
 * total_tokens * h_kv above 2^37, or a copy of V needing 2^31 or more
 * workgroups), GQA_ERR_WORKSPACE (a caller workspace that is not 256-byte
 * aligned or smaller than the call needs). */
int gqa_prefill_validate(const gqa_prefill_args *args);

/* Workspace bytes the call needs (0 where none is used), after the checks of
 * gqa_prefill_validate except the workspace's own.  Host only. */
int gqa_prefill_workspace_bytes(const gqa_prefill_args *args, size_t *bytes);

#ifdef __cplusplus
}
#endif

#endif /* GQA_PREFILL_H */
