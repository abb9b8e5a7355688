// sweep_kernel.hip -- gfx950 (CDNA4) key-sweep kernel of split-KV GQA decode.
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
//   * The page's ranks become wavefronts.  The flattened token axis -- the key
//     rows of all sequences end to end -- is cut into equal ranges (stream-K
//     style), and each range is swept by h_kv consecutive wavefronts, one per kv
//     head, so ragged lengths cost no load imbalance and the wavefronts of one
//     range read the adjacent kv-head slices of the same rows at the same time
//     (contiguous DRAM traffic).  A range that covers a whole sequence stores o
//     itself; a sequence cut across ranges leaves one partial triple per piece
//     and kv head in a workspace, merged by merge_kernel -- or, in fused_kernel
//     (below), inside the sweep itself.
//   * A wavefront sweeps its piece in steps of 32 keys (bf16) or 16 keys (fp32).
//     Q K^T is v_mfma_f32_16x16x32_bf16 (16x16x4_f32 for fp32 input) with the 16
//     keys of a block as the M axis and 16 query rows (heads x query tokens) as
//     the N axis; up to four such 16-row tiles share each load of the keys;
//     K rows are loaded straight into the MFMA A-operand layout with 16-byte
//     buffer loads, so no LDS round trip is needed.  The d axis of the
//     contraction is permuted (the same permutation on Q and K) so each load
//     instruction reads 64 contiguous bytes of 16 key rows.
//   * P V runs on the matrix cores too, with V^T as the A operand and the keys
//     as the contraction: for bf16 input each lane loads 16 bytes of 8 key rows
//     (whole rows per load instruction) and repacks them in registers, and P is
//     split into bf16 high and low parts issued as two products (so P keeps about
//     16 significant bits); for fp32 input v_mfma_f32_16x16x4_f32 takes one key
//     per lane and stays in fp32.
//   * The softmax state of query head g lives in lanes with lane % 16 == g; the
//     block maximum is reduced across the 4 lane groups with two row-swap
//     exchanges, l is kept per lane and reduced once per piece.  Scores are kept
//     in the log2 domain (scale * log2 e folded in) and exponentiated with
//     v_exp_f32; the partial m is stored in that domain and merged with exp2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace gqa {
namespace {

using namespace dev;

#ifndef GQA_SWEEP_DEPTH
#define GQA_SWEEP_DEPTH 2
#endif
constexpr int kSweepDepth = GQA_SWEEP_DEPTH;   // register buffers of the fp32 sweep pipeline
// Cache policy of the K/V stream loads (buffer-instruction cache-policy bits).
// K and V are read exactly once, so they are loaded non-temporally (nt) and do
// not displace the partials, q and seq_lens from the caches.
#ifndef GQA_KV_CPOL
#define GQA_KV_CPOL 2
#endif
constexpr int kKvCachePolicy = GQA_KV_CPOL;

// ------------------------------------------------------------------ loads

// Buffer resource over `bytes` bytes at `base` (raw, stride 0): loads at offsets
// at or beyond `bytes` return zero without touching memory.  Both inputs are
// wave-uniform; readfirstlane makes that visible to the compiler so the resource
// lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const uint8_t *base, uint32_t bytes) {
    const int64_t a = uniform64(reinterpret_cast<int64_t>(base));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<uint8_t *>(a), 0,
                                             uniform32(static_cast<int>(bytes)), 0x00020000);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kKvCachePolicy);
    return make_uint4(x[0], x[1], x[2], x[3]);
}

template <int NW>
__device__ __forceinline__ void load_words(uint32_t (&dst)[NW], __amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (NW == 2) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kKvCachePolicy);
        dst[0] = x[0];
        dst[1] = x[1];
    } else {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const uint4 x = load16(r, off + 16 * i);
            dst[4 * i + 0] = x.x;
            dst[4 * i + 1] = x.y;
            dst[4 * i + 2] = x.z;
            dst[4 * i + 3] = x.w;
        }
    }
}

// Online-softmax update of one step's scores (the page's running merge of the
// step's (m, l, O) into the state): the scores of head lane%16 are reduced
// across the four lane groups, the state is rescaled by 2^(m_old - m_new) and
// p = 2^(s - m_new) is returned in place of s.
//
// kOffset shifts the exponent of p (not of the running max): p = 2^(s - m_new +
// kOffset), so l and O of the triple carry a constant factor 2^kOffset, which
// cancels in O / l and in the merge (every piece of a sequence carries it).
// fp16 P uses 15 so that small weights stay inside fp16's exponent range.
template <int N, int VEC, int kOffset>
__device__ __forceinline__ void softmax_step(float (&sv)[N], float &m_run, float &l_run,
                                             f32x4_t (&acc)[VEC]) {
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < N; ++i) mx = fmaxf(mx, sv[i]);
    mx = max_over_rows(mx);
    const float m_new = fmaxf(m_run, mx);
    // A row that has seen no key yet (all masked) keeps the identity (-inf, 0, 0):
    // exponentiate against 0 instead of -inf so that nothing becomes NaN.
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);   // 0 while the state is empty
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        sv[i] = __builtin_amdgcn_exp2f(sv[i] - m_ref + static_cast<float>(kOffset));
        sum += sv[i];
    }
    l_run = l_run * alpha + sum;
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] *= alpha;
    m_run = m_new;
}

// ------------------------------------------------------------------ bf16 / fp16 steps
//
// One step = 32 keys.  Q K^T: two v_mfma_f32_16x16x32_{bf16,f16} groups (16 keys
// each) with K rows as the A operand (M = keys) and Q^T as B (N = query heads);
// lane l of QK block b loads key row 8*(m/4) + 4b + m%4 (m = l%16), so that after
// the product lane l holds the scores of keys 8*kg + i (kg = l/16, i = 0..7) of
// its head -- exactly the eight keys it contributes to the P V product below.
//
// P V: O^T[d][g] += V^T[d][key] P^T[key][g] as the same MFMA with the 32 keys as
// the contraction.  Lane l loads 16 bytes (8 d) of key rows 8*kg + i, i = 0..7
// (each load instruction reads four whole rows), and repacks them in registers
// so its A operand for column c holds d = VEC*(l%16) + c of its eight keys.  P is
// split into a high part (round to nearest in the input's 16-bit format) and a
// low part (the rounded remainder) and the product is issued twice, so P keeps
// ~16 (bf16) or ~22 (fp16) significant bits; V, Q and K are exact.
template <int D, bool kHalf>
struct Packed16Step {
    // 16x16x32 product of eight 16-bit values per lane, in the input's format.
    __device__ __forceinline__ static f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
        if constexpr (kHalf)
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                          __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                           __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    static constexpr int kKeys = 32;
    static constexpr int ES = 2;
    static constexpr int ROWB = D * ES;
    static constexpr int NKP = ROWB / 64;   // 16-byte K pieces per lane per 16-key block
    static constexpr int VEC = D / 16;      // d elements per lane per key row
    static constexpr int VW = VEC / 2;      // 32-bit words per lane per V row
    struct Buf {
        uint4 k[2][NKP];
        uint32_t v[8][VW];
    };
    struct Lanes {
        uint32_t k[2];   // + 64p: K row of block b, bytes [16kg + 64p, +16)
        uint32_t v[8];   // V row 8kg + i, elements [VEC*m, VEC*m + VEC)
        __device__ __forceinline__ explicit Lanes(int rowstride) {
            const int lane = lane_id();
            const int m = lane & 15;
            const int kg = lane >> 4;
#pragma unroll
            for (int b = 0; b < 2; ++b)
                k[b] = static_cast<uint32_t>((8 * (m >> 2) + 4 * b + (m & 3)) * rowstride + 16 * kg);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = static_cast<uint32_t>((8 * kg + i) * rowstride + m * VEC * ES);
        }
    };
    // A step's K rows (two 16-key blocks) or V rows into the registers of B.
    __device__ __forceinline__ static void load_k(Buf &B, __amdgpu_buffer_rsrc_t rk, const Lanes &lo) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int p = 0; p < NKP; ++p) B.k[b][p] = load16(rk, lo.k[b] + 64 * p);
    }
    __device__ __forceinline__ static void load_v(Buf &B, __amdgpu_buffer_rsrc_t rv, const Lanes &lo) {
#pragma unroll
        for (int i = 0; i < 8; ++i) load_words<VW>(B.v[i], rv, lo.v[i]);
    }
    // A operand of P V column c: element i = V[key 8kg + i][d = VEC*m + c].
    __device__ __forceinline__ static uint4 v_operand(const Buf &B, int c) {
        uint32_t a[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t x = B.v[2 * w][c >> 1];
            const uint32_t y = B.v[2 * w + 1][c >> 1];
            // One byte permute per word: bytes (x0, x1, y0, y1) or (x2, x3, y2, y3).
            a[w] = __builtin_amdgcn_perm(y, x, (c & 1) ? 0x07060302u : 0x05040100u);
        }
        return make_uint4(a[0], a[1], a[2], a[3]);
    }
    // The step for kNT 16-row tiles on one load of the keys, in three phases:
    // every tile's scores (independent MFMA chains) and new row maxima; one
    // wave-wide test whether any reference moved (the accumulators are rescaled
    // only then: elsewhere the factor is exactly 1, or 0 on a still-empty state
    // whose accumulators are 0, so skipping the rescale changes no bit); then
    // every tile's weights, split P and products, with each V column's operand
    // repacked once for all tiles.  sl2 > 0 (a negative scale is moved into q).
    //   kMask   scores outside [lo, hi[nt]) are masked; the scores are scaled
    //           before the maxima and the exponent is (s sl2 - m) + offset.
    //           Otherwise every key is visible: maxima of the raw scores, then
    //           scaled, and the exponent one fused s sl2 + (offset - m).
    // after_qk() runs once every tile's Q K^T products are issued (the caller
    // loads the next step's keys there, into the registers B.k leaves free).
    template <int kNT, bool kMask, class AfterQK>
    __device__ __forceinline__ static void compute_tiles(const Buf &B, const uint4 (&qop)[kNT][NKP], int lo,
                                                         const int (&hi)[kNT], int kg, float sl2,
                                                         float (&m_run)[kNT], float (&l_run)[kNT],
                                                         f32x4_t (&acc)[kNT][VEC], AfterQK after_qk) {
        constexpr float kOff = kHalf ? 15.f : 0.f;
        float sv[kNT][8], m_ref[kNT], alpha[kNT];
        bool moved = false;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < NKP; ++p) sacc = mfma16(B.k[b][p], qop[nt][p], sacc);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int key = 8 * kg + 4 * b + q;
                    if constexpr (kMask)
                        sv[nt][4 * b + q] = (key >= lo && key < hi[nt]) ? sacc[q] * sl2 : -INFINITY;
                    else
                        sv[nt][4 * b + q] = sacc[q];
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        after_qk();
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            float mx = sv[nt][0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[nt][i]);
            // sl2 > 0: the scaled maximum is the maximum of the raw scores, scaled.
            // The reference (m_run) moves only when a row's maximum passes it by more
            // than kLag (log2 units), so after a piece's first steps the rescale is
            // rare; the weights are then below 2^kLag, which bf16 holds (fp16 P,
            // already offset by 2^15, keeps kLag = 0).
            constexpr float kLag = kHalf ? 0.f : 8.f;
            const float mxs = kMask ? max_over_rows(mx) : max_over_rows(mx) * sl2;
            const bool mv = mxs > m_run[nt] + kLag;
            const float m_new = mv ? fmaxf(m_run[nt], mxs) : m_run[nt];
            moved |= mv;
            // A row that has seen no key yet keeps the identity: exponentiate against 0.
            m_ref[nt] = m_new == -INFINITY ? 0.f : m_new;
            alpha[nt] = __builtin_amdgcn_exp2f(m_run[nt] - m_ref[nt]);   // 0 while the state is empty
            m_run[nt] = m_new;
        }
        if (__ballot(moved) != 0) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
                for (int c = 0; c < VEC; ++c) acc[nt][c] *= alpha[nt];
        }
        uint4 bhi[kNT], blo[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            float sum = 0.f;
            const float nmu = kOff - m_ref[nt];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if constexpr (kMask)
                    sv[nt][i] = __builtin_amdgcn_exp2f(sv[nt][i] - m_ref[nt] + kOff);
                else
                    sv[nt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[nt][i], sl2, nmu));
                sum += sv[nt][i];
            }
            l_run[nt] = l_run[nt] * alpha[nt] + sum;
            uint32_t ph[4], pl[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const f32x2_t pw = {sv[nt][2 * w], sv[nt][2 * w + 1]};
                if constexpr (kHalf) {
                    const f16x2_t h = __builtin_convertvector(pw, f16x2_t);
                    const f32x2_t hf = __builtin_convertvector(h, f32x2_t);
                    ph[w] = __builtin_bit_cast(uint32_t, h);
                    pl[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pw - hf, f16x2_t));
                } else {
                    const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(pw, bf16x2_t));
                    const f32x2_t r = {pw[0] - __uint_as_float(hb << 16), pw[1] - __uint_as_float(hb & 0xffff0000u)};
                    ph[w] = hb;
                    pl[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
                }
            }
            bhi[nt] = make_uint4(ph[0], ph[1], ph[2], ph[3]);
            blo[nt] = make_uint4(pl[0], pl[1], pl[2], pl[3]);
        }
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            const uint4 av = v_operand(B, c);
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                acc[nt][c] = mfma16(av, bhi[nt], acc[nt][c]);
                acc[nt][c] = mfma16(av, blo[nt], acc[nt][c]);
            }
        }
    }
};

// ------------------------------------------------------------------ fp32 steps
//
// One step = 16 keys.  Q K^T as v_mfma_f32_16x16x4_f32 (K rows as A, M = keys;
// lane l loads key m = l%16), P V as v_mfma_f32_16x16x4_f32 with V^T as A and
// P^T as B: lane l loads key rows 4*kg + r and contributes one key per product,
// so neither operand needs a transpose and everything stays in fp32.
template <int D>
struct F32Step {
    static constexpr int kKeys = 16;
    static constexpr int ES = 4;
    static constexpr int ROWB = D * ES;
    static constexpr int NKP = ROWB / 64;   // 16-byte K pieces per lane per step
    static constexpr int VEC = D / 16;
    static constexpr int VW = VEC;          // 32-bit words per lane per V row
    struct Buf {
        uint4 k[NKP];
        uint32_t v[4][VW];
    };
    struct Lanes {
        uint32_t k;
        uint32_t v[4];
        __device__ __forceinline__ explicit Lanes(int rowstride) {
            const int lane = lane_id();
            const int m = lane & 15;
            const int kg = lane >> 4;
            k = static_cast<uint32_t>(m * rowstride + 16 * kg);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = static_cast<uint32_t>((4 * kg + r) * rowstride + m * VEC * ES);
        }
    };
    __device__ __forceinline__ static void load(Buf &B, __amdgpu_buffer_rsrc_t rk,
                                                __amdgpu_buffer_rsrc_t rv, const Lanes &lo) {
#pragma unroll
        for (int p = 0; p < NKP; ++p) B.k[p] = load16(rk, lo.k + 64 * p);
#pragma unroll
        for (int r = 0; r < 4; ++r) load_words<VW>(B.v[r], rv, lo.v[r]);
    }
    __device__ __forceinline__ static void compute(const Buf &B, const uint4 (&qop)[NKP], int lo, int hi,
                                                   int kg, float sl2, float &m_run, float &l_run,
                                                   f32x4_t (&acc)[VEC]) {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NKP; ++p) {
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(B.k[p].x), __uint_as_float(qop[p].x), s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(B.k[p].y), __uint_as_float(qop[p].y), s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(B.k[p].z), __uint_as_float(qop[p].z), s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(B.k[p].w), __uint_as_float(qop[p].w), s, 0, 0, 0);
        }
        float sv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int key = 4 * kg + q;
            sv[q] = (key >= lo && key < hi) ? s[q] * sl2 : -INFINITY;
        }
        softmax_step<4, VEC, 0>(sv, m_run, l_run, acc);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < VEC; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(B.v[r][c]), sv[r], acc[c], 0, 0, 0);
    }
};

// Element types, numbered as the GQA_DTYPE_* codes of the C ABI.
constexpr int kBf16 = 0;
constexpr int kF32 = 1;
constexpr int kF16 = 2;

template <int kIn, int D>
using Step = typename std::conditional<kIn == kF32, F32Step<D>, Packed16Step<D, kIn == kF16>>::type;

// Stores n (a multiple of 8) consecutive outputs, rounded to the output type.
template <int kOut>
__device__ __forceinline__ void store_row(uint8_t *dst, const float *x, int n) {
    if constexpr (kOut == kF32) {
        for (int i = 0; i < n; i += 4)
            *reinterpret_cast<float4 *>(dst + 4 * i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
    } else {
        for (int i = 0; i < n; i += 8) {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = pack2<kOut == kF16>(x[i + 2 * k], x[i + 2 * k + 1]);
            *reinterpret_cast<uint4 *>(dst + 2 * i) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// One piece: keys [t0, t1) of (sequence b, kv head j); off = keys before b.  The
// wavefront takes the kv head's rows as kNT tiles of 16 (rows 16 nt .. 16 nt + 15)
// and computes each step once per tile on the same loaded keys; w = the
// wavefront, which indexes the workspace slots.  Returns -1 when the piece was
// the whole sequence (o written), else the slot its partial triple went to.
template <int kIn, int kOut, int D, int kDepth, int kNT, bool kLdsSlots = false>
__device__ __forceinline__ int process_piece(const DecodeParams &P, int b, int j, int64_t off,
                                             int t0, int t1, int len, int w, float *lds_o = nullptr,
                                             float2 *lds_ml = nullptr) {
    using S = Step<kIn, D>;
    constexpr int VEC = S::VEC;
    const int lane = lane_id();
    const int kg = lane >> 4;
    const int G = P.G;
    const int R = P.R;              // rows in use: G * t_q
    const int rowstride = P.h_kv * S::ROWB;

    // Steps cover key rows aligned to kKeys in the packed K/V (absolute row index),
    // so a step never straddles a kKeys-row boundary of the cache: the first step
    // of a piece starts at the aligned row at or below it (its leading rows, which
    // belong to the previous sequence and are in bounds, are masked), and the
    // buffer resources end at the piece's last row, so rows past it read as zero.
    const int64_t first = off + t0;                              // absolute key row
    const int64_t abase = first - (first % S::kKeys);
    const int lead = static_cast<int>(first - abase);            // masked rows of step 0
    const int span = lead + (t1 - t0);                           // keys from abase to the end
    const int nstep = (span + S::kKeys - 1) / S::kKeys;

    // The lane's row in each tile: query token t and head g, its q and o row, and
    // the causal limit of token t among the t_q new tokens -- it sees the keys at
    // sequence positions below len - t_q + t + 1, i.e. (key i of step st sits at
    // position abase - off + kKeys*st + i) below cap - kKeys*st in step coordinates.
    int r[kNT], cap[kNT];
    bool row_ok[kNT];
    int64_t qo_row[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        r[nt] = 16 * nt + (lane & 15);
        row_ok[nt] = r[nt] < R;
        const int t = (row_ok[nt] ? r[nt] : R - 1) / G;
        const int g = (row_ok[nt] ? r[nt] : R - 1) - t * G;
        qo_row[nt] = (static_cast<int64_t>(b) * P.t_q + t) * P.h_q + j * G + g;
        cap[nt] = len - P.t_q + t + 1 - static_cast<int>(abase - off);
    }

    // Q operand: query row (t, g), bytes [64p + 16kg, +16) of it: the same d
    // permutation as the K rows, so the contraction covers every d once.  Lanes of
    // unused rows (past R) hold a copy of row R - 1: their scores are finite and
    // never stored, and with no select on the loaded value the loads stay
    // unconditional and go out together.  A negative scale negates q instead
    // (exact), so that the steps scale by a positive factor and the largest scaled
    // score is the largest raw one.
    uint4 qop[kNT][S::NKP];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const uint8_t *qrow = P.q + qo_row[nt] * S::ROWB + 16 * kg;
#pragma unroll
        for (int p = 0; p < S::NKP; ++p) qop[nt][p] = *reinterpret_cast<const uint4 *>(qrow + 64 * p);
    }

    const int64_t row0 = abase * P.h_kv + j;
    const uint8_t *kbase = P.k + row0 * S::ROWB;
    const uint8_t *vbase = P.v + row0 * S::ROWB;
    const typename S::Lanes lo(rowstride);
    // Buffer resource over step st's rows of K (or V); a step at or past nstep
    // gets an empty range, so its loads return zeros without a memory access
    // (the prefetches past the piece cost no round trip).
    auto step_rsrc = [&](const uint8_t *base, int st) {
        const int hi = max(0, min(S::kKeys, span - st * S::kKeys));
        const int64_t boff = hi > 0 ? static_cast<int64_t>(st) * S::kKeys * rowstride : 0;
        return buffer_rsrc(base + boff, static_cast<uint32_t>(hi * rowstride));
    };
    // The first step's K and V (16-bit input: the refilled buffers below; fp32: the
    // first kDepth - 1 steps of its pipeline) go out with the Q loads, before any
    // of them is used: the scheduling barrier keeps the rest of the set-up (and
    // the register moves of Q) behind them, so a piece starts with one round trip.
    typename S::Buf bk[2], bv;
    typename S::Buf buf[kDepth];
    if constexpr (kIn != kF32) {
        S::load_k(bk[0], step_rsrc(kbase, 0), lo);
        S::load_v(bv, step_rsrc(vbase, 0), lo);
    } else {
#pragma unroll
        for (int ub = 0; ub + 1 < kDepth; ++ub)
            S::load(buf[ub], step_rsrc(kbase, ub), step_rsrc(vbase, ub), lo);
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t qflip = P.scale_log2 < 0.f ? (kIn == kF32 ? 0x80000000u : 0x80008000u) : 0u;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int p = 0; p < S::NKP; ++p) {
            qop[nt][p].x ^= qflip;
            qop[nt][p].y ^= qflip;
            qop[nt][p].z ^= qflip;
            qop[nt][p].w ^= qflip;
        }
    // Keys visible to every row of the wavefront: below the smallest causal limit.
    int capmin = cap[0];
#pragma unroll
    for (int nt = 1; nt < kNT; ++nt) capmin = min(capmin, cap[nt]);
#pragma unroll
    for (int sh = 1; sh < kWave; sh <<= 1) capmin = min(capmin, __shfl_xor(capmin, sh));
    capmin = uniform32(capmin);

    f32x4_t acc[kNT][VEC];
    float m_run[kNT], l_run[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[nt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_run[nt] = -INFINITY;
        l_run[nt] = 0.f;
    }

    // |scale| log2(e), kept above 0 so that a masked (-inf) score stays -inf.
    const float sl2 = fmaxf(fabsf(P.scale_log2), 1.17549435e-38f);
    if constexpr (kIn != kF32) {
        // 16-bit input: one K and one V register buffer, each refilled as soon as
        // its step has used it -- the next step's keys once the Q K^T products
        // are issued, its values once the P V products are -- so the loads of
        // step st+1 overlap the rest of step st with no second buffer (with
        // several tiles the registers go to the tiles instead; with one tile
        // this measured ~1% faster than two full buffers).
        // Unrolled twice with the K buffer named by parity: in a loop that is not
        // unrolled the compiler waits for every outstanding load (vmcnt(0)) at
        // the top of each step, V refill included.
        int st = 0;
        while (true) {
#pragma unroll
            for (int ub = 0; ub < 2; ++ub) {
                typename S::Buf cb;
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int p = 0; p < S::NKP; ++p) cb.k[b][p] = bk[ub].k[b][p];
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int w = 0; w < S::VW; ++w) cb.v[i][w] = bv.v[i][w];
                auto next_keys = [&]() { S::load_k(bk[ub ^ 1], step_rsrc(kbase, st + 1), lo); };
                const int hi = min(S::kKeys, span - st * S::kKeys);
                int his[kNT];
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) his[nt] = min(hi, cap[nt] - st * S::kKeys);
                // A step whose keys every row sees needs no mask (taken with four
                // tiles, where the masking is a measurable share of the vector work).
                if (kNT >= 4 && (st > 0 || lead == 0) && hi == S::kKeys && capmin - st * S::kKeys >= S::kKeys)
                    S::template compute_tiles<kNT, false>(cb, qop, 0, his, kg, sl2, m_run, l_run, acc, next_keys);
                else
                    S::template compute_tiles<kNT, true>(cb, qop, st == 0 ? lead : 0, his, kg, sl2, m_run, l_run,
                                                         acc, next_keys);
                __builtin_amdgcn_sched_barrier(0);   // the V refill after the products
                S::load_v(bv, step_rsrc(vbase, st + 1), lo);
                if (++st == nstep) goto swept;
            }
        }
    } else {
        // fp32 input: software pipeline over kDepth register buffers, the loads
        // of the next kDepth-1 steps in flight while a step is computed.  Every
        // load is unconditional.
        int st = 0;
        while (true) {
#pragma unroll
            for (int ub = 0; ub < kDepth; ++ub) {
                const int pf = st + kDepth - 1;
                S::load(buf[(ub + kDepth - 1) % kDepth], step_rsrc(kbase, pf), step_rsrc(vbase, pf), lo);
                __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the compute
                const int hi = min(S::kKeys, span - st * S::kKeys);
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt)
                    S::compute(buf[ub], qop[nt], st == 0 ? lead : 0, min(hi, cap[nt] - st * S::kKeys), kg, sl2,
                               m_run[nt], l_run[nt], acc[nt]);
                if (++st == nstep) goto swept;
            }
        }
    }
swept:

#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        float l_tot = l_run[nt] + __shfl_xor(l_run[nt], 16);
        l_tot += __shfl_xor(l_tot, 32);

        // The lane's outputs: O[row][d] for d in [4*VEC*kg, 4*VEC*kg + 4*VEC), index q*VEC + c.
        float out[4 * VEC];
        if (t0 == 0 && t1 == len) {
            // The whole sequence was in this range: normalise and store (a query
            // token that sees no key gives 0).
            const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int c = 0; c < VEC; ++c) out[q * VEC + c] = acc[nt][c][q] * inv;
            if (row_ok[nt]) {
                uint8_t *dst = P.o + (qo_row[nt] * D + 4 * VEC * kg) * (kOut == kF32 ? 4 : 2);
                store_row<kOut>(dst, out, 4 * VEC);
            }
        } else {
            // Slot 0: a piece of a sequence that began before this range; slot 1:
            // the first piece of a sequence that continues past it.
            const int slot = (t0 > 0) ? 0 : 1;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int c = 0; c < VEC; ++c) out[q * VEC + c] = acc[nt][c][q];
            if constexpr (kLdsSlots) {
                // The workgroup's own slots in LDS (16 rows each; w = the wavefront within
                // the workgroup): row r of slot 2w + slot.
                if (row_ok[nt]) {
                    const int lrow = (2 * w + slot) * 16 + r[nt];
                    float4 *dst = reinterpret_cast<float4 *>(lds_o + lrow * D + 4 * VEC * kg);
#pragma unroll
                    for (int i = 0; i < VEC; ++i)
                        dst[i] = make_float4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
                    if (kg == 0) lds_ml[lrow] = make_float2(m_run[nt], l_tot);
                }
            } else if (row_ok[nt]) {
                const int64_t srow = (static_cast<int64_t>(w) * 2 + slot) * R + r[nt];
                store_row<kF32>(reinterpret_cast<uint8_t *>(P.ws_o + srow * D + 4 * VEC * kg), out, 4 * VEC);
                if (kg == 0) P.ws_ml[srow] = make_float2(m_run[nt], l_tot);
            }
        }
    }
    return (t0 == 0 && t1 == len) ? -1 : (t0 > 0 ? 0 : 1);
}

template <int kIn, int kOut, int D, int kDepth, int kNT>
__global__ __launch_bounds__(kThreads) void split_kernel(DecodeParams P) {
    const int w = uniform32(static_cast<int>(blockIdx.x) * kWavesPerBlock +
                            static_cast<int>(threadIdx.x) / kWave);
    if (w >= P.num_chunks) return;
    // Wavefront w sweeps kv head j over token range c of the flattened token axis;
    // the h_kv wavefronts of one range are consecutive, so they stream the
    // adjacent kv-head slices of the same key rows at the same time.
    const int j = w % P.h_kv;
    const int c = w / P.h_kv;
    // Up to 64 sequences: their lengths stay in registers (one read of seq_lens).
    const bool few = P.batch <= kWave;
    FirstLens fl;
    if (few) fl.load(P.seq_lens, P.batch);
    const int64_t total = few ? fl.total() : total_len(P.seq_lens, P.batch);
    const int64_t chunk = chunk_keys(total, P.num_chunks / P.h_kv, P.min_chunk);
    int64_t pos = static_cast<int64_t>(c) * chunk;
    if (pos >= total) return;
    const int64_t end = pos + chunk < total ? pos + chunk : total;
    int b, len;
    int64_t off;
    if (few)
        fl.locate(P.batch, 1, pos, b, off, len);
    else
        locate(P.seq_lens, P.batch, 1, pos, b, off, len);
    while (true) {
        const int t0 = uniform32(static_cast<int>(pos - off));
        const int64_t lim = end - off;
        const int t1 = uniform32(static_cast<int>(lim < len ? lim : len));
        process_piece<kIn, kOut, D, kDepth, kNT>(P, b, j, off, t0, t1, len, w);
        pos = off + t1;
        if (pos >= end) break;
        off += len;   // next non-empty sequence (one exists: pos < total)
        do {
            ++b;
            len = few ? fl.len(b) : uniform32(seq_len_at(P.seq_lens, b));
        } while (len == 0);
    }
}

// ------------------------------------------------------------------ fused merge
//
// Single-kernel form of the decode for calls whose time is mostly latency (few
// (sequence, kv head) units): the merge of a sequence's pieces runs inside the
// sweep kernel, as the page's reduction runs inside its kernel (`_merge_running`
// applied as partial triples arrive), instead of in a second launch.
//
//   * A workgroup sweeps kWavesPerBlock consecutive token ranges of one kv head
//     (range group cg, head j: workgroup cg * h_kv + j).  Its wavefronts leave
//     their cut pieces in the workgroup's slots (LDS for up to 16 rows per kv
//     head, else the workspace); after a barrier the workgroup folds, in token
//     order, the pieces that belong to one sequence: a sequence that lies inside
//     the group's ranges gets its o here, and at most two sequences leave a
//     group-level piece in the workspace (slot 0: begun before the group's first
//     range; slot 1: continuing past its last), so the cross-workgroup reduction
//     sees one piece per workgroup and sequence.
//   * Group-level pieces are reduced by a tree of fixed fan-in K over the pieces
//     of a sequence in token order: a node's children are K consecutive nodes of
//     the level below.  Every workgroup that finishes a child increments the
//     node's counter (a relaxed vector atomic at device scope, issued after the
//     child's device-coherent stores have completed; the last arriver reads the
//     children with device-coherent loads after the increment returned), and the
//     one that completes the count -- the last arriver --
//     folds the children in ascending order, stores the node in its first
//     child's place and goes up one level; at the root it writes o.  The fold
//     order is fixed by the tree, not by arrival, so results are bit-identical
//     from run to run.  The last arriver also puts the counter back to zero, so
//     the counters read zero before and after every call.
//   * Empty sequences (no key) get zeros from the workgroups of range group
//     b mod (number of range groups).

// Running state of one fold over (m, l, O) triples: m in log2 units.
struct FoldState {
    float M, L;
    float4 acc;
};

__device__ __forceinline__ void fold_in(FoldState &r, float2 ml, float4 o) {
    const float Mn = fmaxf(r.M, ml.x);
    // Both sides empty (-inf): exponentiate against 0 so the identity stays NaN-free.
    const float Mr = Mn == -INFINITY ? 0.f : Mn;
    const float a = __builtin_amdgcn_exp2f(r.M - Mr);   // 0 while r is empty
    const float f = __builtin_amdgcn_exp2f(ml.x - Mr);  // 0 for an empty side
    r.L = r.L * a + ml.y * f;
    r.acc.x = r.acc.x * a + o.x * f;
    r.acc.y = r.acc.y * a + o.y * f;
    r.acc.z = r.acc.z * a + o.z * f;
    r.acc.w = r.acc.w * a + o.w * f;
    r.M = Mn;
}

// Stores four consecutive outputs (d = 4 dq .. 4 dq + 3) of one o row.
template <int kOut>
__device__ __forceinline__ void store_out_quad(uint8_t *row, int dq, float4 x) {
    if constexpr (kOut == kF32)
        reinterpret_cast<float4 *>(row)[dq] = x;
    else
        reinterpret_cast<uint2 *>(row)[dq] = make_uint2(pack2<kOut == kF16>(x.x, x.y), pack2<kOut == kF16>(x.z, x.w));
}

// The group-level triples travel between workgroups on different XCDs (each with
// its own L2) through device-coherent accesses: buffer loads and stores with the
// sc1 cache-policy bit, the form device-scope atomic loads and stores take on
// this architecture.  A store completes (vmcnt) only once it is visible device
// wide, and a load with sc1 reads the coherent copy, so no L2 writeback or
// invalidate is needed: each workgroup waits for its stores before it increments
// a node's counter, and the last arriver loads the children only after the
// counter's increment returned.
constexpr int kCoherent = 16;   // sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws2_rsrc(const void *base) {
    // Offsets stay below 2^32: the counter reserve limits a fused launch to
    // 8192 workgroups, so the group-level slots span at most 8192 x 2 x 64 rows
    // x 128 floats = 2^29 bytes.
    return make_rsrc(base, 0xffffffffu);
}

__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 x) {
    const uint4 u = make_uint4(__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z), __float_as_uint(x.w));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, u), r,
                                           off, 0, kCoherent);
}

__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float2 x) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 u = {__float_as_uint(x.x), __float_as_uint(x.y)};
    __builtin_amdgcn_raw_buffer_store_b64(u, r, off, 0, kCoherent);
}

__device__ __forceinline__ float4 load_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent);
    return make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]), __uint_as_float(u[3]));
}

__device__ __forceinline__ float2 load_coherent2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoherent);
    return make_float2(__uint_as_float(u[0]), __uint_as_float(u[1]));
}

// Stores a fold's result for quad (row, dq): into the o row of (sequence b, kv
// head j), normalised by L, or unnormalised into triple row srow0 + row of the
// workspace's group-level slots (with (M, L) from the row's dq == 0 thread).
template <int kOut, int D>
__device__ __forceinline__ void fold_store(const DecodeParams &P, const FoldState &r, int row, int dq, bool to_o,
                                           int b, int j, int64_t srow0) {
    if (to_o) {
        const int t = row / P.G;
        const int g = row - t * P.G;
        uint8_t *orow = P.o + ((static_cast<int64_t>(b) * P.t_q + t) * P.h_q + j * P.G + g) * D *
                                  (kOut == kF32 ? 4 : 2);
        const float inv = r.L > 0.f ? 1.0f / r.L : 0.f;   // a query token with no key gives 0
        store_out_quad<kOut>(orow, dq, make_float4(r.acc.x * inv, r.acc.y * inv, r.acc.z * inv, r.acc.w * inv));
    } else {
        const int64_t srow = srow0 + row;
        store_coherent(ws2_rsrc(P.ws2_o), static_cast<uint32_t>((srow * D + 4 * dq) * 4), r.acc);
        if (dq == 0) store_coherent(ws2_rsrc(P.ws2_ml), static_cast<uint32_t>(srow * 8), make_float2(r.M, r.L));
    }
}

// Folds children i = first, first + step, ... below n of quad (row, dq) into r,
// in ascending order, with every load of a batch of 16 issued before the folds.
constexpr int kFoldBatch = 16;
template <typename Load>
__device__ __forceinline__ void fold_span(FoldState &r, Load load, int first, int n, int step) {
    for (int i0 = first; i0 < n; i0 += kFoldBatch * step) {
        float2 ml[kFoldBatch];
        float4 ov[kFoldBatch];
#pragma unroll
        for (int i = 0; i < kFoldBatch; ++i)
            if (i0 + i * step < n) load(i0 + i * step, ml[i], ov[i]);
#pragma unroll
        for (int i = 0; i < kFoldBatch; ++i)
            if (i0 + i * step < n) fold_in(r, ml[i], ov[i]);
    }
}

// Folds n triples, child i at workspace group-level row index child(i) + row,
// and stores the result (o rows, or group-level rows srow0 ..).  The workgroup
// takes the R * D / 4 quads with PL = kThreads / quads threads ("piece lanes")
// per quad when there are fewer quads than threads: lane l folds children l, l +
// PL, ..., and the lanes are combined through LDS in ascending order, so the
// fold order is fixed.  Every load precedes a barrier that precedes every
// store, so the destination may be the first child's storage.  All threads of
// the workgroup must call it.
template <int kOut, int D, typename Child>
__device__ void fold_children(const DecodeParams &P, FoldState *s_comb, Child child, int n, bool to_o, int b, int j,
                              int64_t srow0) {
    constexpr int QD = D / 4;
    const int tid = static_cast<int>(threadIdx.x);
    const int quads = P.R * QD;
    const int PL = quads >= kThreads ? 1 : kThreads / quads;
    const int iters = (quads + kThreads - 1) / kThreads;
    for (int it = 0; it < iters; ++it) {
        const int qd = PL > 1 ? tid % quads : it * kThreads + tid;
        const int lane = PL > 1 ? tid / quads : 0;
        const bool active = qd < quads && lane < PL;
        const int row = qd / QD;
        const int dq = qd - row * QD;
        FoldState r = {-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
        if (active) {
            const auto ro = ws2_rsrc(P.ws2_o);
            const auto rml = ws2_rsrc(P.ws2_ml);
            auto load = [&](int i, float2 &ml, float4 &o) {
                const int64_t srow = child(i) + row;
                ml = load_coherent2(rml, static_cast<uint32_t>(srow * 8));
                o = load_coherent4(ro, static_cast<uint32_t>((srow * D + 4 * dq) * 4));
            };
            fold_span(r, load, lane, n, PL);
        }
        if (PL > 1) s_comb[tid] = r;
        __syncthreads();   // every child has been read
        if (active && lane == 0) {
            for (int l = 1; l < PL; ++l) {
                const FoldState x = s_comb[qd + l * quads];
                fold_in(r, make_float2(x.M, x.L), x.acc);
            }
            fold_store<kOut, D>(P, r, row, dq, to_o, b, j, srow0);
        }
        if (PL > 1) __syncthreads();   // s_comb is free again
    }
}

// One wavefront slot's record for the workgroup fold.
struct SlotMeta {
    int b, t0, t1, len;
    int64_t off;
};

template <int kIn, int kOut, int D, int kDepth, int kNT>
__global__ __launch_bounds__(kThreads) void fused_kernel(DecodeParams P) {
    // Up to 16 rows per kv head, the wavefronts' slots live in LDS: slot e =
    // 2 * wavefront + slot, 16 rows each.
    constexpr bool kLds = kNT == 1;
    constexpr int kSlots = 2 * kWavesPerBlock;
    __shared__ float s_slot_o[kLds ? kSlots * 16 * D : 4];
    __shared__ float2 s_slot_ml[kLds ? kSlots * 16 : 1];
    __shared__ FoldState s_comb[kThreads];
    __shared__ SlotMeta s_meta[kSlots];
    __shared__ int s_last;
    const int tid = static_cast<int>(threadIdx.x);
    const int wave = uniform32(tid / kWave);
    const int lane = lane_id();
    const int wg = static_cast<int>(blockIdx.x);
    const int j = wg % P.h_kv;
    const int cg = wg / P.h_kv;                          // range group
    const int n_groups = P.num_chunks / (P.h_kv * kWavesPerBlock);
    const int w = wg * kWavesPerBlock + wave;            // the wavefront's workspace slots
    const int c = cg * kWavesPerBlock + wave;            // the wavefront's token range
    if (lane == 0) {
        s_meta[2 * wave].b = -1;
        s_meta[2 * wave + 1].b = -1;
    }
    const bool few = P.batch <= kWave;
    FirstLens fl;
    if (few) fl.load(P.seq_lens, P.batch);
    const int64_t total = few ? fl.total() : total_len(P.seq_lens, P.batch);
    const int64_t chunk = chunk_keys(total, P.num_chunks / P.h_kv, P.min_chunk);

    // ---- zeros for empty sequences b with b mod n_groups == cg (head j's rows); the
    // workgroup's wavefronts take them in turn.
    {
        const int64_t rowq = static_cast<int64_t>(P.R) * (D / 4);   // quads of one (sequence, head)
        auto zero = [&](int eb) {
            for (int64_t qd = lane; qd < rowq; qd += kWave) {
                const int row = static_cast<int>(qd / (D / 4));
                const int dq = static_cast<int>(qd - static_cast<int64_t>(row) * (D / 4));
                const FoldState z = {-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
                fold_store<kOut, D>(P, z, row, dq, true, eb, j, 0);
            }
        };
        if (few) {
            unsigned long long m = __ballot(lane < P.batch && fl.li == 0 && lane % n_groups == cg);
            for (int idx = 0; m; ++idx) {
                const int eb = __ffsll(static_cast<long long>(m)) - 1;
                m &= m - 1;
                if (idx % kWavesPerBlock == wave) zero(eb);
            }
        } else {
            for (int64_t k0 = 0; cg + k0 * n_groups < P.batch; k0 += kWave) {
                const int64_t bb = cg + (k0 + lane) * n_groups;
                unsigned long long m = __ballot(bb < P.batch && P.seq_lens[bb] <= 0);
                for (int idx = 0; m; ++idx) {
                    const int src = __ffsll(static_cast<long long>(m)) - 1;
                    m &= m - 1;
                    if (idx % kWavesPerBlock == wave) zero(static_cast<int>(cg + (k0 + src) * n_groups));
                }
            }
        }
    }

    // ---- the wavefront's own range, as in split_kernel
    int64_t pos = static_cast<int64_t>(c) * chunk;
    if (pos < total) {
        const int64_t end = pos + chunk < total ? pos + chunk : total;
        int b, len;
        int64_t off;
        if (few)
            fl.locate(P.batch, 1, pos, b, off, len);
        else
            locate(P.seq_lens, P.batch, 1, pos, b, off, len);
        while (true) {
            const int t0 = uniform32(static_cast<int>(pos - off));
            const int64_t lim = end - off;
            const int t1 = uniform32(static_cast<int>(lim < len ? lim : len));
            const int slot = process_piece<kIn, kOut, D, kDepth, kNT, kLds>(
                P, b, j, off, t0, t1, len, kLds ? wave : w, s_slot_o, s_slot_ml);
            if (slot >= 0 && lane == 0) s_meta[2 * wave + slot] = SlotMeta{b, t0, t1, len, off};
            pos = off + t1;
            if (pos >= end) break;
            off += len;
            do {
                ++b;
                len = few ? fl.len(b) : uniform32(seq_len_at(P.seq_lens, b));
            } while (len == 0);
        }
    }
    __syncthreads();

    // ---- workgroup fold of the wavefronts' pieces, sequence by sequence in token order
    // (slots e = 2 * wavefront + slot are in token order; a sequence's slots are
    // consecutive among the filled ones).  The slot records are read once into
    // registers and each thread reads all slots of its quad before folding, so the
    // fold costs one round of LDS reads; every loop over the slots is unrolled.
    SlotMeta meta[kSlots];
#pragma unroll
    for (int e = 0; e < kSlots; ++e) meta[e] = s_meta[e];
    // group-level pieces left for the cross-workgroup reduction: (sequence, off, len)
    int gp_b0 = 0, gp_len0 = 0, gp_b1 = 0, gp_len1 = 0, ngp = 0;
    int64_t gp_off0 = 0, gp_off1 = 0;
    {
        int cur = -1, first_t0 = 0;
        SlotMeta last = meta[0];
        auto close = [&]() {
            if (cur >= 0 && !(first_t0 == 0 && last.t1 == last.len)) {
                if (ngp == 0) {
                    gp_b0 = cur;
                    gp_len0 = last.len;
                    gp_off0 = last.off;
                } else {
                    gp_b1 = cur;
                    gp_len1 = last.len;
                    gp_off1 = last.off;
                }
                ++ngp;
            }
        };
#pragma unroll
        for (int e = 0; e < kSlots; ++e) {
            if (meta[e].b >= 0) {
                if (meta[e].b != cur) {
                    close();
                    cur = meta[e].b;
                    first_t0 = meta[e].t0;
                }
                last = meta[e];
            }
        }
        close();
    }
    constexpr int QD = D / 4;
    const int quads = P.R * QD;
    for (int qd = tid; qd < quads; qd += kThreads) {
        const int row = qd / QD;
        const int dq = qd - row * QD;
        float2 sml[kSlots];
        float4 so[kSlots];
#pragma unroll
        for (int e = 0; e < kSlots; ++e) {
            sml[e] = make_float2(-INFINITY, 0.f);
            so[e] = make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (kLds) {
                const int lrow = e * 16 + row;
                sml[e] = s_slot_ml[lrow];
                so[e] = reinterpret_cast<const float4 *>(s_slot_o + lrow * D)[dq];
            } else if (meta[e].b >= 0) {
                const int64_t srow = (static_cast<int64_t>(wg * kWavesPerBlock + e / 2) * 2 + (e & 1)) * P.R + row;
                sml[e] = P.ws_ml[srow];
                so[e] = reinterpret_cast<const float4 *>(P.ws_o + srow * D)[dq];
            }
        }
        FoldState r = {-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
        int cur = -1, first_t0 = 0;
        SlotMeta last = meta[0];
        auto close = [&]() {
            if (cur < 0) return;
            const bool whole = first_t0 == 0 && last.t1 == last.len;
            fold_store<kOut, D>(P, r, row, dq, whole, cur, j,
                                (static_cast<int64_t>(wg) * 2 + (first_t0 > 0 ? 0 : 1)) * P.R);
        };
#pragma unroll
        for (int e = 0; e < kSlots; ++e) {
            if (meta[e].b >= 0) {
                if (meta[e].b != cur) {
                    close();
                    cur = meta[e].b;
                    first_t0 = meta[e].t0;
                    r = FoldState{-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
                }
                fold_in(r, sml[e], so[e]);
                last = meta[e];
            }
        }
        close();
    }

    // ---- tree reduction of the group-level pieces across workgroups (32-bit
    // indices: range groups and workgroups number below 2^22)
    const int kl = P.fold_k_log2;
    const int64_t chunk_g = chunk * kWavesPerBlock;
    const int level_stride = 2 * (P.num_chunks / kWavesPerBlock);   // counters per level
    for (int q = 0; q < ngp; ++q) {
        const int gpb = q == 0 ? gp_b0 : gp_b1;
        const int64_t gpoff = q == 0 ? gp_off0 : gp_off1;
        const int gplen = q == 0 ? gp_len0 : gp_len1;
        const int ca = static_cast<int>(div_nonneg(gpoff, chunk_g));
        const int cb = static_cast<int>(div_nonneg(gpoff + gplen - 1, chunk_g));
        int nprev = cb - ca + 1;              // nodes at the level below (pieces at first)
        int idx = cg - ca;                    // this workgroup's node at that level
        int sl = 0;                           // log2 of the pieces per node at that level
        for (int level = 0;; ++level) {
            const int gidx = idx >> kl;
            const int first = gidx << kl;
            const int nchild = min(nprev - first, 1 << kl);
            const int ncur = (nprev + (1 << kl) - 1) >> kl;
            const int p0 = first << sl;                      // the node's first piece
            // storage of piece p: workgroup (ca + p) * h_kv + j, slot 1 for the first piece
            const int st0 = ((ca + p0) * P.h_kv + j) * 2 + (p0 == 0 ? 1 : 0);
            if (nchild > 1) {
                // Every thread's coherent stores of the child are complete (visible device
                // wide) before the workgroup counts it.
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (tid == 0) {
                    uint32_t *ctr = P.counters + level * level_stride + st0;
                    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const int last = old == static_cast<uint32_t>(nchild - 1);
                    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    s_last = last;
                }
                __syncthreads();
                if (!s_last) break;
                // child i (node first + i of the level below) is stored with its first piece
                auto child = [&](int i) {
                    const int p = (first + i) << sl;
                    return static_cast<int64_t>((((ca + p) * P.h_kv + j) * 2 + (p == 0 ? 1 : 0)) * P.R);
                };
                fold_children<kOut, D>(P, s_comb, child, nchild, ncur == 1, gpb, j,
                                       static_cast<int64_t>(st0) * P.R);
            }
            if (ncur == 1) break;
            idx = gidx;
            nprev = ncur;
            sl += kl;
        }
    }
}

template <int kIn, int kOut, int kNT>
void launch_iot(const DecodeParams &P, int D, int blocks, bool fused, hipStream_t stream) {
    if (fused) {
        if (D == 128)
            hipLaunchKernelGGL((fused_kernel<kIn, kOut, 128, kSweepDepth, kNT>), dim3(blocks), dim3(kThreads), 0,
                               stream, P);
        else
            hipLaunchKernelGGL((fused_kernel<kIn, kOut, 64, kSweepDepth, kNT>), dim3(blocks), dim3(kThreads), 0,
                               stream, P);
        return;
    }
    if (D == 128)
        hipLaunchKernelGGL((split_kernel<kIn, kOut, 128, kSweepDepth, kNT>), dim3(blocks), dim3(kThreads), 0, stream,
                           P);
    else
        hipLaunchKernelGGL((split_kernel<kIn, kOut, 64, kSweepDepth, kNT>), dim3(blocks), dim3(kThreads), 0, stream, P);
}

// 16-row tiles per wavefront: 1 up to 16 rows per kv head (G * t_q), 2 up to 32,
// 3 up to 48, 4 up to 64 (the keys of a step are loaded once for all of them).
template <int kIn, int kOut>
hipError_t launch_io(const DecodeParams &P, int D, int blocks, bool fused, hipStream_t stream) {
    if (P.R <= 16)
        launch_iot<kIn, kOut, 1>(P, D, blocks, fused, stream);
    else if (P.R <= 32)
        launch_iot<kIn, kOut, 2>(P, D, blocks, fused, stream);
    else if (P.R <= 48)
        launch_iot<kIn, kOut, 3>(P, D, blocks, fused, stream);
    else
        launch_iot<kIn, kOut, 4>(P, D, blocks, fused, stream);
    return hipGetLastError();
}

template <int kIn, int kOut>
hipError_t occupancy_io(int D, int *blocks_per_cu) {
    return D == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                          blocks_per_cu, split_kernel<kIn, kOut, 128, kSweepDepth, 1>, kThreads, 0)
                    : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                          blocks_per_cu, split_kernel<kIn, kOut, 64, kSweepDepth, 1>, kThreads, 0);
}

}  // namespace

// (in, out) pairs the validation admits: (bf16, bf16), (bf16, f32), (f32, f32),
// (f16, f16), (f16, f32).
hipError_t launch_sweep(const DecodeParams &P, int in_dtype, int out_dtype, int D, int blocks, bool fused,
                        hipStream_t stream) {
    if (in_dtype == kBf16) return out_dtype == kBf16 ? launch_io<kBf16, kBf16>(P, D, blocks, fused, stream)
                                                     : launch_io<kBf16, kF32>(P, D, blocks, fused, stream);
    if (in_dtype == kF16) return out_dtype == kF16 ? launch_io<kF16, kF16>(P, D, blocks, fused, stream)
                                                   : launch_io<kF16, kF32>(P, D, blocks, fused, stream);
    return launch_io<kF32, kF32>(P, D, blocks, fused, stream);
}

hipError_t sweep_occupancy(int in_dtype, int out_dtype, int D, int *blocks_per_cu) {
    if (in_dtype == kBf16) return out_dtype == kBf16 ? occupancy_io<kBf16, kBf16>(D, blocks_per_cu)
                                                     : occupancy_io<kBf16, kF32>(D, blocks_per_cu);
    if (in_dtype == kF16) return out_dtype == kF16 ? occupancy_io<kF16, kF16>(D, blocks_per_cu)
                                                   : occupancy_io<kF16, kF32>(D, blocks_per_cu);
    return occupancy_io<kF32, kF32>(D, blocks_per_cu);
}

}  // namespace gqa
