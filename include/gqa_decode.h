/*
 * gqa_decode.h -- C ABI of the MI355X (gfx950) split-KV grouped-query-attention
 * decode library (libgqa_decode.so).
 *
 * The operation (kernbench2 page "_gqa_attention_decode_long.py": the kernel
 * docstring, the "Tile 0" block, the tile loop over 1024-key tiles with
 * `_merge_running`, and the final normalise-and-store block):
 *
 *   for every sequence b < batch and query head h < h_q, with G = h_q / h_kv,
 *   kv head j = h / G, S = seq_lens[b] (negative counts as 0) and
 *   base = seq_lens[0] + ... + seq_lens[b-1]:
 *
 *     s_t      = scale * sum_i q[b,h,i] * k[base+t, j, i]        t < S
 *     o[b,h,:] = sum_t softmax(s)_t * v[base+t, j, :]           (S = 0 gives 0)
 *
 * computed as a sweep over the key axis: the keys of every (sequence, kv head)
 * are cut into ranges, each range is reduced to a partial online-softmax triple
 * (m, l, O) for all G query heads of that kv head at once, and the triples are
 * combined with the log-sum-exp merge (m = max of both; each side rescaled by
 * exp(its m - m); l and O summed), then O / l is stored.  The page's reduction
 * across ranks of a device mesh becomes, on one GPU, the ranges of one kernel
 * grid plus a merge kernel.
 *
 * Readings where the page is silent: `scale` multiplies the raw dot product
 * (the page applies none; scale = 1 reproduces it); K is used truly transposed;
 * query head h reads kv head h / G; K/V of the sequences are packed back to
 * back; the accumulator, partials and merge are fp32; bf16 output is the
 * nearest-even rounding of the fp32 result.
 *
 * Tensor layouts (row-major, contiguous, all in device memory of the current
 * HIP device, owned by the caller; the library never frees or keeps them):
 *   q         [batch, h_q, d_head]            in_dtype
 *   k, v      [sum(seq_lens), h_kv, d_head]   in_dtype, sequences packed back to back
 *   o         [batch, h_q, d_head]            out_dtype (written)
 *   seq_lens  int32[batch]  (device memory; read by the kernels, never by the host,
 *             so a call needs no host synchronisation)
 *
 * Supported: d_head in {64, 128}; G = h_q / h_kv in 1..64 (G * t_q <= 64 rows per kv
 * head, swept as one to four 16-row tiles per wavefront over one read of the
 * keys); (in, out) dtypes
 * (bf16, bf16), (bf16, f32), (f16, f16), (f16, f32) and (f32, f32).  q, k, v, o must be 16-byte aligned,
 * seq_lens 4-byte aligned.
 *
 * Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns without synchronising.  Errors found on the host
 * return before anything is enqueued, and then `o` is untouched.
 *
 * Errors: every entry point returns GQA_OK (0) or a positive gqa_status code;
 * gqa_last_error_message() gives a thread-local description of the last error.
 * No C++ exception crosses this interface.
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
#define GQA_DTYPE_BF16 0
#define GQA_DTYPE_F32 1
#define GQA_DTYPE_F16 2 /* IEEE binary16 */

/* Merge forms (gqa_decode_args.merge). */
#define GQA_MERGE_AUTO 0   /* the plan chooses                                        */
#define GQA_MERGE_KERNEL 1 /* a second kernel merges the pieces of cut sequences       */
#define GQA_MERGE_FUSED 2  /* one kernel: the pieces are merged inside the sweep       */

/* Bytes at the start of every workspace (and of gqa_decode_noalloc's scratch)
 * that hold the fused merge's counters; see gqa_decode_args.workspace. */
#define GQA_DECODE_COUNTER_BYTES (64 * 1024)

/* Status codes. */
typedef enum gqa_status {
    GQA_OK = 0,
    GQA_ERR_NULL = 1,        /* a required pointer is NULL                              */
    GQA_ERR_SHAPE = 2,       /* batch, h_q or h_kv <= 0, h_q not a multiple of h_kv,    *
                              * t_q < 0, or batch * t_q * h_q above 2^31-1              */
    GQA_ERR_UNSUPPORTED = 3, /* d_head not 64/128, G * t_q > 64, or dtype pair          *
                              * not supported                                           */
    GQA_ERR_ALIGN = 4,       /* q/k/v/o not 16-byte aligned or seq_lens not 4-byte      */
    GQA_ERR_SCALE = 5,       /* scale is not finite                                     */
    GQA_ERR_WORKSPACE = 6,   /* caller workspace too small or not 256-byte aligned      */
    GQA_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed              */
    GQA_ERR_ARG = 8          /* a tuning field is out of range                          */
} gqa_status;

/*
 * gqa_decode -- bf16 q/k/v in, bf16 o out, fp32 accumulation.
 * Arguments as in the layouts above.  `scale` is usually 1/sqrt(d_head).
 * Uses a library-owned workspace (see gqa_decode_ex), so the first call on a
 * (device, stream) pair may allocate device memory.
 */
int gqa_decode(const void *q, const void *k, const void *v, void *o, const int32_t *seq_lens,
               int32_t batch, int32_t h_q, int32_t h_kv, int32_t d_head, float scale,
               void *stream);

/* gqa_decode_f32 -- the same operation with fp32 q/k/v in and fp32 o out. */
int gqa_decode_f32(const void *q, const void *k, const void *v, void *o,
                   const int32_t *seq_lens, int32_t batch, int32_t h_q, int32_t h_kv,
                   int32_t d_head, float scale, void *stream);

/* gqa_decode_f16 -- the same operation with IEEE fp16 q/k/v in and fp16 o out (the
 * page's element type); fp32 accumulation, o rounded to nearest even. */
int gqa_decode_f16(const void *q, const void *k, const void *v, void *o,
                   const int32_t *seq_lens, int32_t batch, int32_t h_q, int32_t h_kv,
                   int32_t d_head, float scale, void *stream);

/*
 * Full argument block.  Zero-initialise it, then set the fields.
 *
 * num_chunks  Wavefronts of the sweep.  The token axis -- the key rows of all
 *             sequences end to end, sum(seq_lens) rows -- is cut into
 *             num_chunks / h_kv equal ranges of `chunk` rows, where
 *               chunk = max(min_chunk, ceil(sum(seq_lens) / (num_chunks / h_kv)))
 *             is computed on the device from seq_lens, and each range is swept by
 *             h_kv wavefronts, one per kv head.  A range that holds a whole
 *             sequence writes its o rows directly; the pieces of a sequence that
 *             spans several ranges are merged by a second kernel, or inside the
 *             sweep kernel (see `merge`).  Rounded down to
 *             a multiple of h_kv (at least h_kv).  0 = automatic (compute units x
 *             min(resident wavefronts per compute unit, 4)).  Range: 0..2^24.
 * min_chunk   Smallest range in key rows; 0 = automatic (64).  Range: 0..2^30.
 *             min_chunk = 1024 with a large num_chunks reproduces the page's
 *             1024-key tiles as the split granularity.
 * workspace   Device scratch for the partial triples, at least
 *             gqa_decode_workspace_bytes() bytes, 256-byte aligned, owned by the
 *             caller and not used concurrently by another call.  Its first
 *             GQA_DECODE_COUNTER_BYTES bytes hold the fused merge's counters: they
 *             must read zero before the first call that uses the workspace (zero
 *             the buffer once after allocating it, or after using the memory for
 *             anything else, e.g. a prefill workspace), and every call leaves them
 *             zero; the rest needs no initialisation.  NULL = a library-owned
 *             buffer per (device, stream), grown with hipMalloc on demand (its
 *             counters cleared when it is allocated) and freed by gqa_release();
 *             callers that capture HIP graphs must pass their own, and make one
 *             uncaptured call of the same dtypes and d_head on the device first (it
 *             caches the device's compute-unit count and occupancy); the captured
 *             call then enqueues kernel launches only.
 * merge       GQA_MERGE_AUTO (0), GQA_MERGE_KERNEL or GQA_MERGE_FUSED: how the
 *             pieces of a sequence cut across ranges are merged.  KERNEL: a second
 *             kernel merges them after the sweep.  FUSED: one kernel; each
 *             workgroup sweeps 4 consecutive ranges of one kv head (num_chunks is
 *             then rounded down to a multiple of 4 * h_kv, at least 4 * h_kv),
 *             folds its wavefronts' pieces per sequence, and the workgroup-level
 *             pieces of a sequence are reduced by a tree of fixed fan-in whose
 *             nodes are folded by the last workgroup to arrive (device-scope
 *             atomic counters), in an order fixed by the tree, so results are the
 *             same from run to run.  AUTO chooses FUSED for calls of at most 16
 *             (sequence, kv head) units whose max_seq_len hint is at most 4 x
 *             min_chunk keys (every sequence then meets at most one other
 *             workgroup), where the second launch is a large part of the step,
 *             unless num_chunks needs more counters than the reserve holds.  The fused merge uses levels x num_chunks / 2
 *             counters (GQA_DECODE_COUNTER_BYTES / 4 at most): FUSED lowers
 *             num_chunks until they fit, and returns GQA_ERR_ARG only when even
 *             4 * h_kv wavefronts need more (h_kv above 8,192).
 * sweep_events  See the field's comment; leave NULL outside profiling.
 * t_q         See the field's comment; 0 for the single-token decode.
 */
typedef struct gqa_decode_args {
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
    int32_t in_dtype;  /* GQA_DTYPE_BF16, GQA_DTYPE_F16 or GQA_DTYPE_F32 */
    int32_t out_dtype; /* the input's type, or GQA_DTYPE_F32 */
    int32_t num_chunks;
    int32_t min_chunk;
    void *workspace;
    size_t workspace_bytes;
    void *stream; /* hipStream_t */
    /* Optional profiling hook: two hipEvent_t created by the caller.  When both
     * are non-NULL, the first is recorded on `stream` just before the partial
     * (sweep) kernel and the second just after it, so its duration can be read
     * with hipEventElapsedTime without a profiler.  NULL = not recorded. */
    void *sweep_events[2];
    /* Query tokens per sequence (multi-token decode, e.g. verifying draft tokens);
     * 0 or 1 = one.  With t_q > 1, q and o are [batch, t_q, h_q, d_head], the last
     * t_q key rows of every sequence belong to the new tokens, and query token t
     * attends to the keys at positions 0 .. seq_len - t_q + t (causal among the new
     * tokens; a token that sees no key gives 0).  G * t_q must not exceed 64. */
    int32_t t_q;
    int32_t merge;  /* GQA_MERGE_*, see above */
    /* Optional hint: no sequence is longer than max_seq_len keys (0 = unknown).
     * Used by the automatic merge choice, and with batch 1 by the merge kernel,
     * which reads the pieces for a length of exactly max_seq_len while it reads
     * seq_lens and checks the two before it stores (one memory round trip less
     * when they agree).  The kernels take the lengths from seq_lens: a wrong hint
     * changes the speed, never the result, and with the merge form fixed the
     * result is bit-identical with and without it. */
    int32_t max_seq_len;
} gqa_decode_args;

/* gqa_decode_ex -- the operation with every field of `args` (see above). */
int gqa_decode_ex(const gqa_decode_args *args);

/*
 * gqa_decode_noalloc -- gqa_decode_ex for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same operation, kernels and results as gqa_decode_ex with
 * the same plan; the partial triples go to a scratch array of
 * GQA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every device it
 * runs on until the process ends, instead of a workspace.  The call allocates
 * nothing (no hipMalloc, no allocating library routine).
 *
 * `workspace` must be NULL and `workspace_bytes` 0 (GQA_ERR_ARG otherwise).  A
 * call whose plan needs more scratch than the array holds -- the size
 * gqa_decode_workspace_bytes() reports for the same arguments: the counter
 * reserve plus num_chunks x 2 x (G * t_q) x (d_head + 2) x 4 bytes (and a
 * quarter of that again with the fused merge) -- returns GQA_ERR_WORKSPACE
 * before anything is enqueued; the automatic plan fits for up to 16 rows per kv
 * head (G * t_q) at d_head 128 and 32 at d_head 64 on a 256-compute-unit
 * device, and a smaller num_chunks fits larger shapes.  The array's first
 * GQA_DECODE_COUNTER_BYTES are the counter reserve: zero when the library is
 * loaded, and every call leaves them zero.
 *
 * Every call on a device shares that device's one scratch array, which keeps the
 * last call's contents: two calls that may overlap on one device (different
 * streams, or different threads without ordering) race on it and give
 * undefined results; calls ordered on one stream are safe.  The first call on a
 * device looks up the array's device address (and caches the device's compute-
 * unit count and occupancy, as gqa_decode_ex does): make that first call outside
 * graph capture.  Other arguments, layouts and errors as gqa_decode_ex.
 */
#define GQA_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
int gqa_decode_noalloc(const gqa_decode_args *args);

/*
 * gqa_decode_validate -- the host-side argument checks of gqa_decode_ex alone
 * (pointers, shapes, support, alignment, scale, tuning ranges; the workspace
 * size is checked only when num_chunks is given, since the automatic value needs
 * the device).  Touches no device and enqueues nothing.  Returns the status
 * gqa_decode_ex would return for these arguments before launching.
 */
int gqa_decode_validate(const gqa_decode_args *args);

/*
 * Resolved launch plan of a call (pure host arithmetic, no device access).
 * num_cus and waves_per_cu describe the device: the automatic num_chunks is
 * num_cus * min(waves_per_cu, 4) (at most one sweep wavefront per SIMD), rounded
 * down to a multiple of h_kv.  Returns GQA_OK or the validation status.
 */
typedef struct gqa_decode_plan {
    int32_t num_chunks;      /* wavefronts launched (h_kv per token range)         */
    int32_t min_chunk;       /* smallest token range in key rows                   */
    int32_t split_blocks;    /* workgroups of the sweep kernel (4 wavefronts each) */
    int32_t merge_blocks;    /* workgroups of the merge kernel                     */
    int32_t merge_threads;   /* threads per merge workgroup (256 or 1024)          */
    int32_t merge_slices;    /* d slices per output row in the merge (1 or d / 32) */
    size_t workspace_bytes;  /* partial-triple scratch the call needs              */
    int32_t fused;           /* 1: one kernel (GQA_MERGE_FUSED), merge_* are 0     */
    int32_t fold_fanin;      /* fused: children per node of the merge tree         */
    int32_t fold_levels;     /* fused: counter levels of the tree                  */
} gqa_decode_plan;

int gqa_decode_make_plan(const gqa_decode_args *args, int32_t num_cus, int32_t waves_per_cu,
                         gqa_decode_plan *plan);

/*
 * gqa_decode_workspace_bytes -- bytes of workspace a gqa_decode_ex call with these
 * arguments needs, in *bytes.  With num_chunks = 0 it queries the current
 * device's compute-unit count.  Returns a status: GQA_ERR_NULL when `bytes` is
 * NULL, the validation status of the arguments, or GQA_ERR_HIP when the device
 * query fails; *bytes is written only on GQA_OK.  The size comes back through a
 * pointer rather than as the return value because the query can fail in these
 * ways, and a size_t return would have to reserve a sentinel size for them, which
 * callers could mistake for a size.
 */
int gqa_decode_workspace_bytes(const gqa_decode_args *args, size_t *bytes);

/* Text of a status code (static storage). */
const char *gqa_status_str(int status);

/* Thread-local message of the last failing call on this thread ("" if none). */
const char *gqa_last_error_message(void);

/* Frees every library-owned workspace after synchronising its device. */
void gqa_release(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H */
