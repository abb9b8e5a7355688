// prefill_kernel.hip -- gfx950 (CDNA4) causal GQA prefill.
//
// Every token t of a sequence attends to the keys at positions 0 .. t of that
// sequence: o = softmax(scale * q_t K[0..t]^T) V[0..t] for each query head, the
// head reading kv head h / G.  This is the multi-token decode definition with
// the query tokens being the whole sequence (the long-context prefill panel of
// the kernbench2 page "_gqa_attention_decode_long.py", commit description:
// T_q = S_kv, d_head 128, one KV group, the query axis split across workers
// with disjoint output rows, so no cross-worker reduction is needed).
//
// Mapping to one MI355X:
//   * A workgroup (8 wavefronts) owns one tile of 256 rows = 256 / G tokens x G
//     query heads of one (sequence, kv head), and sweeps the keys 0 .. its last
//     token with the page's online-softmax fold; the rows are disjoint, so every
//     tile normalises and stores its own outputs.
//   * The keys are swept in 64-key steps.  K and V go HBM/L2 -> LDS into four
//     slots (K and V of two steps) that all 256 rows share, so the K/V bytes per
//     output row fall with the tile height.  The loads write LDS directly (buffer
//     loads with the LDS as destination: no registers, no LDS store
//     instructions) and run a step ahead of their use; one barrier per step.
//     LDS rows are XOR-swizzled in 16-byte chunks so the operand reads hit
//     distinct banks; a direct load writes lane i's 16 bytes at base + 16 i, so
//     the swizzle is applied by choosing which global chunk each lane fetches.
//   * The fast loop is software pipelined: while the vector units turn the
//     scores of step x into P, the matrix cores compute the scores of step x+1;
//     then O += V P for step x.
//   * Each wavefront owns 32 rows as two 16-row N tiles of
//     v_mfma_f32_16x16x32_{bf16,f16}: S^T = K Q^T with the keys on the M axis
//     (the K rows are read from LDS in the key order that leaves lane l holding
//     keys 8*(l/16) .. +7 of its row), then O^T += V^T P^T and l += 1^T P^T (the
//     row sums come out of the matrix core, from the same rounded P).  The V^T
//     operand comes out of LDS with 16-byte loads from the transposed copy (fast
//     loop) or through transpose loads from V as given (masked loop).  Two
//     wavefronts share a SIMD (at most 256 VGPRs each, no AGPR traffic).
//   * P V precision: by default P is rounded to fp16 and V read as fp16, one
//     product per step.  A pre-pass (vprep_kernel) writes every sequence's V, 64
//     keys at a time, transposed and in fp16 into the workspace (bf16 is
//     converted -- exactly for magnitudes in fp16's normal range -- and a block
//     whose largest |v| is not in [2^-10, 2^16) is flagged), so that the fast
//     loop reads the V^T operand with plain 16-byte LDS loads.  From the first
//     flagged step on, a tile's sweep uses the split product (P as a high and a
//     low part in the input format, V as given, two products), which the
//     diagonal band always uses and which the caller can ask for everywhere.
//   * The running maximum is allowed to lag the true one: the accumulators are
//     rescaled only when some row's scores pass its reference by more than 8
//     (log2 units; the masked loop computes the row maxima every step) or make
//     an fp16 weight overflow (the fast loop computes the maxima only for a
//     tile's first step and then watches each step's row sums for infinity,
//     recomputing that step with moved references when one appears).  Weights
//     are then below 2^16 (the exponent offset 2^7 keeps small weights inside
//     fp16's range), and the common factor cancels in O / l.
//   * Tiles are handed out over a persistent grid: the tiles of a (sequence, kv
//     head) are enumerated last token first (longest first), and workgroup w
//     takes tiles w, 2g-1-w, 2g+w, ... (g = grid size, a snake that evens out
//     the causal triangle's work), except that the last round's tiles come
//     from a counter in the workspace (zeroed by the V copy kernel), so that
//     compute units that ran faster take more of them.  Without a workspace
//     (split_pv = 1) the whole order is fixed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace gqa {
namespace {

using namespace dev;

constexpr int kBf16 = 0;
constexpr int kF32 = 1;
constexpr int kF16 = 2;

constexpr int kWavesP = kPrefillThreads / kWave;   // 8
constexpr int kNT = kPrefillRows / kWavesP / 16;   // 16-row N tiles per wavefront (2)
constexpr int kRowsPerWave = 16 * kNT;             // 32
#ifndef GQA_PREFILL_STEP_KEYS
#define GQA_PREFILL_STEP_KEYS 64
#endif
constexpr int kStepKeys = GQA_PREFILL_STEP_KEYS;   // keys per compute step (a multiple of 32)
constexpr float kLagLog2 = 8.f;                    // allowed lag of the running maximum
static_assert(kWavesP * kRowsPerWave == kPrefillRows, "tile rows");

template <bool kHalf>
__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
    if constexpr (kHalf)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Tiles of `len` tokens with `tt` tokens per tile.
__device__ __forceinline__ int64_t tiles_of(int64_t len, int tt) { return (len + tt - 1) / tt; }

// Work items (tiles x kv heads) of the whole batch; the same value in every lane.
__device__ int64_t count_items(const int32_t *seq_lens, int batch, int tt, int h_kv) {
    const int lane = lane_id();
    int64_t acc = 0;
    for (int base = 0; base < batch; base += kWave) {
        const int i = base + lane;
        const int64_t n = (i < batch) ? tiles_of(seq_len_at(seq_lens, i), tt) : 0;
        acc += shfl64(inclusive_scan64(n), kWave - 1);
    }
    return uniform64(acc * h_kv);
}

// The sequence b holding work item `it`, with off = tokens before b, len = its
// length, local = the item's index among b's items and steps = the 64-key steps
// of the sequences before b (sum of ceil(len / 64)).  b = batch if there is none.
__device__ void locate_item(const int32_t *seq_lens, int batch, int tt, int h_kv, int64_t it, int &b,
                            int64_t &off, int &len, int64_t &local, int64_t &steps) {
    const int lane = lane_id();
    int64_t run_items = 0, run_len = 0, run_steps = 0;
    for (int base = 0; base < batch; base += kWave) {
        const int i = base + lane;
        const int64_t li = (i < batch) ? seq_len_at(seq_lens, i) : 0;
        const int64_t ni = tiles_of(li, tt) * h_kv;
        const int64_t si = tiles_of(li, kPrefillStepKeys);
        const int64_t inc_n = inclusive_scan64(ni);
        const int64_t inc_l = inclusive_scan64(li);
        const int64_t inc_s = inclusive_scan64(si);
        const bool hit = (i < batch) && (run_items + inc_n > it);
        const unsigned long long mask = __ballot(hit);
        if (mask) {
            const int src = __ffsll(static_cast<long long>(mask)) - 1;
            b = base + src;
            len = uniform32(static_cast<int>(shfl64(li, src)));
            off = uniform64(run_len + shfl64(inc_l, src) - len);
            local = uniform64(it - (run_items + shfl64(inc_n, src) - shfl64(ni, src)));
            steps = uniform64(run_steps + shfl64(inc_s, src) - shfl64(si, src));
            return;
        }
        run_items += shfl64(inc_n, kWave - 1);
        run_len += shfl64(inc_l, kWave - 1);
        run_steps += shfl64(inc_s, kWave - 1);
    }
    b = batch;
    off = run_len;
    len = 0;
    local = 0;
    steps = run_steps;
}

// Stores 4 consecutive outputs, rounded to the output type.
template <int kOut>
__device__ __forceinline__ void store4(uint8_t *dst, const float (&x)[4]) {
    if constexpr (kOut == kF32)
        *reinterpret_cast<float4 *>(dst) = make_float4(x[0], x[1], x[2], x[3]);
    else
        *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2<kOut == kF16>(x[0], x[1]), pack2<kOut == kF16>(x[2], x[3]));
}

template <int kIn, int kOut, int D>
struct PrefillTile {
    static constexpr bool kHalf = kIn == kF16;
    static constexpr int ROWB = D * 2;              // bytes of one key row of one kv head
    static constexpr int LROW = ROWB;               // LDS row pitch (chunks swizzled, see swz)
    static constexpr int NKP = ROWB / 64;           // 16-byte K pieces per lane per 16-key block
    static constexpr int VEC = D / 16;              // d elements per lane per V row
    static constexpr int CH = ROWB / 16;            // 16-byte chunks per key row
    static constexpr int kChunks = kStepKeys * CH;  // 16-byte chunks of one step's K (or V) rows
    static constexpr int kPer = kChunks / kPrefillThreads;   // direct loads per wavefront per step and tensor
    static constexpr int kOff = 7;                  // exponent offset of P: p <= 2^(8 + 7)
    static constexpr int kSlotBytes = kStepKeys * LROW;   // one step's K (or V) rows in LDS
    static constexpr int kVtRow = kStepKeys * 2;          // bytes of one d row of a transposed V step
    static_assert(kStepKeys == kPrefillStepKeys, "the V copy's blocks are the kernel's steps");
    static_assert(D * kVtRow == kSlotBytes, "a transposed V step fills one slot");
    static_assert(kChunks % kPrefillThreads == 0, "whole direct loads per wavefront");
    static constexpr uint32_t kOnesF16 = 0x3c003c00u;
    static constexpr uint32_t kOnesIn = kHalf ? 0x3c003c00u : 0x3f803f80u;

    // 16 bytes per lane from buffer `r` at byte `off` straight into LDS: lane i
    // writes dst + 16 i (dst is the same for the whole wavefront); a lane whose
    // bytes lie beyond the buffer's range writes zeros.
    __device__ __forceinline__ static void lds_load16(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t off) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, off, 0, 0, 0);
    }
    // Waits for this wavefront's outstanding vector-memory loads (the direct LDS
    // loads among them: their data is in LDS once the counter drops).
    __device__ __forceinline__ static void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0f70); }   // vmcnt(0)

    // LDS layout of a K slot, or of a V slot holding V as given: key row r at
    // r * LROW, its 16-byte chunk c at chunk position c ^ swz(r) (K) or c ^ swzv(r)
    // (V).  One K operand read hits rows {0-3, 8-11, 16-19, 24-27} (+4 for the
    // second block) at one chunk; one transposed V read (pv() with V as given)
    // hits 4 consecutive rows at 2 chunks.  The swizzles spread both over
    // distinct banks.  (A slot holding the transposed copy has its own layout:
    // see pv().)
    __device__ __forceinline__ static int swz(int r) { return ((r & 3) | ((r >> 1) & 12)) & (CH - 1); }
    __device__ __forceinline__ static int swzv(int r) { return (2 * (r & 3)) & (CH - 1); }

    // ds_read_b64_tr_b16: within each group of 16 lanes, lane l receives element
    // l % 4 of the 8-byte blocks addressed by lanes 4e + (l % 16) / 4, e = 0..3
    // (its elements e).  With lane 4e + q of group kg addressing V[key 8kg + 4t +
    // e][d = 16c + 4q .. +3], lane (m, kg) receives V[8kg + 4t + e][16c + m]: two
    // reads (t = 0, 1) give it the eight keys 8kg .. 8kg + 7 at d = 16c + m, the A
    // operand of V^T P^T for the d block c, with no register shuffling.
    __device__ __forceinline__ static uint2 lds_read_tr16(const uint8_t *p) {
        typedef short v4s __attribute__((ext_vector_type(4)));
        const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s *)(const_cast<uint8_t *>(p)));
        return __builtin_bit_cast(uint2, r);
    }

    static constexpr int kH = kStepKeys / 32;   // 32-key halves of a step

    // S^T = K Q^T of one step for the N tiles: the lane holds keys k0 + 32h + 8kg +
    // i of its rows in sv[nt][h][i].  The contraction over d runs in the outer
    // loop, so the 2 kNT kH accumulators -- the score registers themselves -- form
    // independent chains that the matrix core interleaves (a chain of dependent
    // products issues at a fraction of the rate).  Every K operand read is issued
    // before the first product (kept there by a scheduling barrier), so the
    // products wait for one LDS round trip instead of one per d piece.
    __device__ __forceinline__ static void qk(const uint8_t *Kt, const uint32_t (&koff)[2][NKP],
                                              const uint4 (&qop)[kNT][NKP], float (&sv)[kNT][kH][8]) {
        f32x4_t sacc[kNT][kH][2];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
            for (int h = 0; h < kH; ++h)
#pragma unroll
                for (int b = 0; b < 2; ++b) sacc[nt][h][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        uint4 kop[NKP][kH][2];
#pragma unroll
        for (int p = 0; p < NKP; ++p)
#pragma unroll
            for (int h = 0; h < kH; ++h)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    kop[p][h][b] = *reinterpret_cast<const uint4 *>(Kt + h * 32 * LROW + koff[b][p]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < NKP; ++p)
#pragma unroll
            for (int h = 0; h < kH; ++h)
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        sacc[nt][h][b] = mfma16<kHalf>(kop[p][h][b], qop[nt][p], sacc[nt][h][b]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
            for (int h = 0; h < kH; ++h)
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int q = 0; q < 4; ++q) sv[nt][h][4 * b + q] = sacc[nt][h][b][q];
    }

    // Row maxima of a step and the (rare) move of the references, for both N tiles
    // before any exponential.  Moves the references only when some row's maximum
    // passes its reference by more than the allowed lag (wave-uniform branch; rows
    // that did not ask follow along, with alpha = 1 where nothing changes).
    // Returns in nmu the exponent offsets of p = 2^(s*sl2 - m_ref + kOff) (a row
    // with no visible key yet keeps the reference -inf and takes 0 in its place:
    // its weights are masked to 0).  lim[nt]: key 32h + i of the lane is visible
    // iff 32h + i < lim[nt] (used with kDiag only).
    template <bool kDiag>
    __device__ __forceinline__ static void references(const float (&sv)[kNT][kH][8], const int (&lim)[kNT], float sl2,
                                                      float (&m_ref)[kNT], f32x4_t (&accl)[kNT],
                                                      f32x4_t (&acc)[kNT][VEC], float (&nmu)[kNT]) {
        float mxs[kNT];
        bool move = false;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            float mx = -INFINITY;
#pragma unroll
            for (int h = 0; h < kH; ++h)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if constexpr (kDiag)
                        mx = 32 * h + i < lim[nt] ? fmaxf(mx, sv[nt][h][i]) : mx;
                    else
                        mx = fmaxf(mx, sv[nt][h][i]);
                }
            mx = max_over_rows(mx);
            mxs[nt] = mx == -INFINITY ? -INFINITY : mx * sl2;   // scaled, log2 units
            move |= mxs[nt] > m_ref[nt] + kLagLog2;
        }
        if (__ballot(move)) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const float m_new = fmaxf(m_ref[nt], mxs[nt]);
                const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref[nt] - m_new);
                accl[nt] *= alpha;
#pragma unroll
                for (int c = 0; c < VEC; ++c) acc[nt][c] *= alpha;
                m_ref[nt] = m_new;
            }
        }
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
            nmu[nt] = static_cast<float>(kOff) - (m_ref[nt] == -INFINITY ? 0.f : m_ref[nt]);
    }

    // P = 2^(s*sl2 + nmu) of a step in the P V product's format (the row sums come
    // from the same rounded P as the product).
    //   kDiag   mask keys at or beyond each row's causal limit lim.
    //   kSplit  P in the input's 16-bit format as a high and a low part (two
    //           products, V as given); otherwise P in fp16 (one product) against
    //           V in fp16.
    template <bool kDiag, bool kSplit>
    __device__ __forceinline__ static void exp_p(const float (&sv)[kNT][kH][8], const int (&lim)[kNT], float sl2,
                                                 const float (&nmu)[kNT], uint4 (&bhi)[kNT][kH],
                                                 uint4 (&blo)[kNT][kH]) {
        constexpr bool kPvHalf = kSplit ? kHalf : true;   // element type of the P V product
#pragma unroll
        for (int h = 0; h < kH; ++h) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                float pv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[nt][h][i], sl2, nmu[nt]));
                    if constexpr (kDiag) pv[i] = 32 * h + i < lim[nt] ? pv[i] : 0.f;
                }
                uint32_t phi[4], plo[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const f32x2_t pw = {pv[2 * w], pv[2 * w + 1]};
                    if constexpr (kPvHalf) {
                        const f16x2_t hv = __builtin_convertvector(pw, f16x2_t);
                        phi[w] = __builtin_bit_cast(uint32_t, hv);
                        if constexpr (kSplit) {
                            const f32x2_t hf = __builtin_convertvector(hv, f32x2_t);
                            plo[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pw - hf, f16x2_t));
                        }
                    } else {
                        const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(pw, bf16x2_t));
                        const f32x2_t r = {pw[0] - __uint_as_float(hb << 16), pw[1] - __uint_as_float(hb & 0xffff0000u)};
                        phi[w] = hb;
                        plo[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
                    }
                }
                bhi[nt][h] = make_uint4(phi[0], phi[1], phi[2], phi[3]);
                if constexpr (kSplit) blo[nt][h] = make_uint4(plo[0], plo[1], plo[2], plo[3]);
            }
        }
    }

    // O^T += V^T P^T and l += 1^T P^T for a step, half by half (d block c: d =
    // 16c + M; the A operand holds keys 32h + 8kg + i, d = 16c + m).
    //   kVT     V is in the slot transposed (the fast loop's copy: row d holds the
    //           step's 64 keys, 16-byte chunk k at position k ^ (d & 7)), read with
    //           one 16-byte load per operand at voff[h]; otherwise V rows as
    //           given, read with transpose loads at voff[c & 3].
    //   kRowSum also accumulate the row sums into accl (otherwise row_sums() does).
    // The fast loop's form (kVT, fp16 P, no row sums) issues every operand read
    // before the first product, as qk() does.
    template <bool kSplit, bool kVT, bool kRowSum = true>
    __device__ __forceinline__ static void pv(const uint4 (&bhi)[kNT][kH], const uint4 (&blo)[kNT][kH],
                                              const uint8_t *Vt, const uint32_t *voff, f32x4_t (&accl)[kNT],
                                              f32x4_t (&acc)[kNT][VEC]) {
        constexpr bool kPvHalf = kSplit ? kHalf : true;
        if constexpr (kVT && !kSplit && !kRowSum) {
            uint4 av[kH][VEC];
#pragma unroll
            for (int h = 0; h < kH; ++h)
#pragma unroll
                for (int c = 0; c < VEC; ++c) av[h][c] = *reinterpret_cast<const uint4 *>(Vt + c * 16 * kVtRow + voff[h]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < kH; ++h)
#pragma unroll
                for (int c = 0; c < VEC; ++c)
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt) acc[nt][c] = mfma16<true>(av[h][c], bhi[nt][h], acc[nt][c]);
            return;
        }
#pragma unroll
        for (int h = 0; h < kH; ++h) {
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                uint4 av;
                if constexpr (kVT) {
                    av = *reinterpret_cast<const uint4 *>(Vt + c * 16 * kVtRow + voff[h]);
                } else {
                    const uint8_t *base = Vt + h * 32 * LROW + (c >> 2) * 128 + voff[c & 3];
                    const uint2 lo = lds_read_tr16(base);
                    const uint2 hi = lds_read_tr16(base + 4 * LROW);
                    av = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) acc[nt][c] = mfma16<kPvHalf>(av, bhi[nt][h], acc[nt][c]);
                if constexpr (kSplit) {
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt) acc[nt][c] = mfma16<kPvHalf>(av, blo[nt][h], acc[nt][c]);
                }
            }
            // Row sums of this half (after the half's products, so the two
            // updates of accl[nt] are far apart).
            if constexpr (kRowSum) {
                const uint32_t one = kPvHalf ? kOnesF16 : kOnesIn;
                const uint4 ones = make_uint4(one, one, one, one);
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) {
                    accl[nt] = mfma16<kPvHalf>(ones, bhi[nt][h], accl[nt]);
                    if constexpr (kSplit) accl[nt] = mfma16<kPvHalf>(ones, blo[nt][h], accl[nt]);
                }
            }
        }
    }

    // Row sums of one step's fp16 P (every element of rs[nt] is the sum of the
    // lane's row).
    __device__ __forceinline__ static void row_sums(const uint4 (&bhi)[kNT][kH], f32x4_t (&rs)[kNT]) {
        const uint4 ones = make_uint4(kOnesF16, kOnesF16, kOnesF16, kOnesF16);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) rs[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < kH; ++h)
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) rs[nt] = mfma16<true>(ones, bhi[nt][h], rs[nt]);
    }

    // Key limits of the lane's rows for a step at key k0 (see references()).
    __device__ __forceinline__ static void limits(const int (&cap)[kNT], int k0, int (&lim)[kNT]) {
        const int kg = lane_id() >> 4;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) lim[nt] = cap[nt] - (k0 + 8 * kg);
    }

    // One unpipelined step (the masked / split loop): S, references, P V.
    template <bool kDiag, bool kSplit>
    __device__ __forceinline__ static void step(const uint8_t *Kt, const uint8_t *Vt, int k0,
                                                const uint32_t (&koff)[2][NKP], const uint32_t (&voff)[4],
                                                const uint4 (&qop)[kNT][NKP], const int (&cap)[kNT],
                                                float sl2, float (&m_ref)[kNT], f32x4_t (&accl)[kNT],
                                                f32x4_t (&acc)[kNT][VEC]) {
        float sv[kNT][kH][8];
        qk(Kt, koff, qop, sv);
        int lim[kNT];
        limits(cap, k0, lim);
        float nmu[kNT];
        references<kDiag>(sv, lim, sl2, m_ref, accl, acc, nmu);
        uint4 bhi[kNT][kH], blo[kNT][kH];
        exp_p<kDiag, kSplit>(sv, lim, sl2, nmu, bhi, blo);
        pv<kSplit, false>(bhi, blo, Vt, voff, accl, acc);
    }

    // Tile `tile` of (sequence b at token offset off, length len; kv head j).
    __device__ __forceinline__ static void run(const PrefillParams &P, uint8_t *K0, uint8_t *K1, uint8_t *V0,
                                               uint8_t *V1, int64_t off, int len, int j, int tile, int64_t vblk) {
        const int tid = static_cast<int>(threadIdx.x);
        const int wave = uniform32(tid / kWave);
        const int lane = lane_id();
        const int m = lane & 15;
        const int kg = lane >> 4;
        const int G = P.G;
        const int tt = kPrefillRows / G;                 // tokens per tile
        const int tstart = tile * tt;
        const int tcount = min(tt, len - tstart);         // > 0
        const int rowstride = P.h_kv * ROWB;

        const uint32_t qflip = P.scale_log2 < 0.f ? 0x80008000u : 0u;
        // |scale| * log2 e, kept above 0 so that masked (-inf) scores stay -inf.
        const float sl2 = fmaxf(fabsf(P.scale_log2), 1.17549435e-38f);

        // The lane's rows: row = 32 wave + 16 nt + m -> (token, head) = (row / G, row % G).
        int cap[kNT];
        uint4 qop[kNT][NKP];
        int64_t orow[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const int row = wave * kRowsPerWave + 16 * nt + m;
            const int tok = row / G;
            const int gh = row - tok * G;
            const bool active = tok < tcount;
            cap[nt] = active ? tstart + tok + 1 : 0;   // keys visible: positions < cap
            orow[nt] = ((off + tstart + (active ? tok : 0)) * P.h_q + j * G + gh);
            const uint8_t *qrow = P.q + orow[nt] * ROWB + 16 * kg;
#pragma unroll
            for (int p = 0; p < NKP; ++p) {
                uint4 x = *reinterpret_cast<const uint4 *>(qrow + 64 * p);
                // A negative scale: negate q (exact) so the kernel scales by |scale|.
                x.x ^= qflip;
                x.y ^= qflip;
                x.z ^= qflip;
                x.w ^= qflip;
                qop[nt][p] = active ? x : make_uint4(0, 0, 0, 0);
            }
        }
        const int wtok_lo = (wave * kRowsPerWave) / G;
        const int wtok_hi = min((wave * kRowsPerWave + kRowsPerWave - 1) / G, tcount - 1);
        const int wkeys = wtok_lo < tcount ? tstart + wtok_hi + 1 : 0;   // keys this wavefront needs
        const int nkeys = tstart + tcount;                                 // keys the tile needs
        const int nsteps = (nkeys + kStepKeys - 1) / kStepKeys;             // 64-key steps
        const uint8_t *kbase = P.k + (off * P.h_kv + j) * ROWB;
        const uint8_t *vbase = P.v + (off * P.h_kv + j) * ROWB;

        // Direct load i of this wavefront fills LDS chunks p = 64 (kPer wave + i) +
        // lane of a step's K (or V) region: row r = p / CH at position p % CH,
        // which holds the row's global chunk (p % CH) ^ swz(r) (swzv(r) for V).
        auto raw_offset = [&](int i, bool is_v) -> uint32_t {
            const int p = (wave * kPer + i) * kWave + lane;
            const int r = p / CH;
            const int pos = p - r * CH;
            return static_cast<uint32_t>(r * rowstride + (pos ^ (is_v ? swzv(r) : swz(r))) * 16);
        };
        uint32_t gk[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) gk[i] = raw_offset(i, false);
        // The same for a transposed V step (row d of 8 chunks, chunk k at position
        // k ^ (d & 7)), and the lane's operand offsets in it: keys 32h + 8kg ..
        // +7 of d row m (+ 16 c).
        uint32_t gt[kPer], vto[kH];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int p = (wave * kPer + i) * kWave + lane;
            const int r = p / 8;
            const int pos = p - r * 8;
            gt[i] = static_cast<uint32_t>(r * kVtRow + ((pos ^ (r & 7)) * 16));
        }
#pragma unroll
        for (int h = 0; h < kH; ++h)
            vto[h] = static_cast<uint32_t>(m * kVtRow + (((4 * h + kg) ^ (m & 7)) & 7) * 16);
        // Per-lane LDS offsets of the step's operands (fixed for the whole tile):
        // K operand of block b, piece p: row 8(m/4) + 4b + m%4, chunk 4p + kg.
        // V (transposed read, t = 0, d block c = 4 ch + cl): lane 4e + q of group kg
        // addresses row 8kg + e (+ 4t), d = 16c + 4q, i.e. chunk 2c + q/2, bytes
        // 8 (q % 2); with the swizzle (2c + q/2) ^ 2e = 8ch + 2(cl ^ e) + q/2.
        uint32_t koff[2][NKP];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int r = 8 * (m >> 2) + 4 * b + (m & 3);
#pragma unroll
            for (int p = 0; p < NKP; ++p) koff[b][p] = static_cast<uint32_t>(r * LROW + ((4 * p + kg) ^ swz(r)) * 16);
        }
        // Steps that run the fast (fp16 P V, pipelined) loop: every step below the
        // tile's first token, up to the first one whose V the copy flagged; none
        // without a copy.  Step x holds the sequence's keys 64 x .. + 63, block
        // vblk + x of the copy.
        const int nfull = min(nsteps, (tstart + 1) / kStepKeys);
        int nfast = 0;
        if (nfull > 0 && vblk + nfull <= P.nvb) {   // (a copy exists and covers these steps)
            // First step whose V the copy flagged (bf16 input only sets flags).
            const uint8_t *fl = P.vflags + j * P.nvb + vblk;
            nfast = nfull;
            for (int x0 = 0; x0 < nfull; x0 += kWave) {
                const int x = x0 + lane;
                const unsigned long long mask = __ballot(x < nfull && fl[x] != 0);
                if (mask) {
                    nfast = x0 + (__ffsll(static_cast<long long>(mask)) - 1);
                    break;
                }
            }
            nfast = uniform32(nfast);
        }
        const uint8_t *vtb = nfast > 0 ? P.vt + (j * P.nvb + vblk) * kSlotBytes : vbase;
        // Loads the K (or V) rows of step x into a slot; rows at or beyond the
        // sequence's end read as zero.  V comes from the fp16 copy for the fast
        // loop's steps.
        auto issue_k = [&](uint8_t *dst, int x) {
            const int k0 = x * kStepKeys;
            const uint32_t bytes = k0 < len ? static_cast<uint32_t>(min(kStepKeys, len - k0) * rowstride) : 0u;
            const auto rs = make_rsrc(kbase + static_cast<int64_t>(k0) * rowstride, bytes);
#pragma unroll
            for (int i = 0; i < kPer; ++i) lds_load16(rs, dst + (wave * kPer + i) * kWave * 16, gk[i]);
        };
        auto issue_v = [&](uint8_t *dst, int x) {
            if (x < nfast) {   // the transposed fp16 copy of step x (a full step)
                const auto rs = make_rsrc(vtb + static_cast<int64_t>(x) * kSlotBytes, kSlotBytes);
#pragma unroll
                for (int i = 0; i < kPer; ++i) lds_load16(rs, dst + (wave * kPer + i) * kWave * 16, gt[i]);
            } else {
                const int k0 = x * kStepKeys;
                const uint32_t bytes = k0 < len ? static_cast<uint32_t>(min(kStepKeys, len - k0) * rowstride) : 0u;
                const auto rs = make_rsrc(vbase + static_cast<int64_t>(k0) * rowstride, bytes);
#pragma unroll
                for (int i = 0; i < kPer; ++i) lds_load16(rs, dst + (wave * kPer + i) * kWave * 16, raw_offset(i, true));
            }
        };
        float m_ref[kNT];
        f32x4_t accl[kNT];
        f32x4_t acc[kNT][VEC];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            m_ref[nt] = -INFINITY;
            accl[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[nt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        // LDS slots: K of step x in K[x & 1], V of step x in V[x & 1]; the four
        // slots are separate arrays named at every use, so the compiler can tell
        // that operand reads never touch the loads in flight to another slot.
        //
        // Fast loop, software pipelined: iteration x holds S(x) from the previous
        // one, and computes S(x+1) = K(x+1) Q^T on the matrix cores while the
        // vector units turn S(x) into P(x) (the two are independent, so they
        // interleave), then O += V(x) P(x).  At its start K(x+1) and V(x) are in
        // LDS and the slot of K(x) is free; it loads K(x+2) and V(x+1) and ends
        // with one barrier.  The S of the step after the fast loop is computed and
        // dropped (the masked loop recomputes it).
        //
        // Masked / split loop: steps the diagonal band crosses, and every step from
        // the first whose V range does not suit fp16 on; each wavefront skips the
        // steps beyond its own last token.  Step x reads K(x), V(x), loads the
        // next step's (K(x+1) may be there already) and ends with one barrier.
        issue_k(K0, 0);
        issue_v(V0, 0);
        if (nsteps > 1) issue_k(K1, 1);
        wait_loads();
        __syncthreads();
        float sa[kNT][kH][8], sb[kNT][kH][8];
        int lim0[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) lim0[nt] = 0;   // unused by the unmasked references
        float nmu[kNT];
        if (nfast > 0) {
            qk(K0, koff, qop, sa);
            references<false>(sa, lim0, sl2, m_ref, accl, acc, nmu);   // references from step 0's maxima
            __syncthreads();   // every wavefront is done with K(0)
        }
        // After step 0 the fast loop does not compute row maxima: a score more than
        // ~9 (log2 units) above its row's reference makes its fp16 weight, and so
        // the step's row sum, infinite, and only then are the maxima computed, the
        // references moved and P recomputed (rare; the accumulators still hold
        // the previous steps only).  Otherwise the weights stay below 2^16.
        auto fast_iter = [&](uint8_t *Kfree, const uint8_t *Knext, const uint8_t *Vcur, uint8_t *Vnext, int x,
                             float (&scur)[kNT][kH][8], float (&snext)[kNT][kH][8]) {
            if (x + 2 < nsteps) issue_k(Kfree, x + 2);
            if (x + 1 < nsteps) issue_v(Vnext, x + 1);
            uint4 ph[kNT][kH], pl[kNT][kH];
            qk(Knext, koff, qop, snext);
            exp_p<false, false>(scur, lim0, sl2, nmu, ph, pl);
            f32x4_t rs[kNT];
            row_sums(ph, rs);
            bool bad = false;
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) bad |= !(fabsf(rs[nt][0]) < INFINITY);   // inf or NaN
            if (__ballot(bad)) {
                references<false>(scur, lim0, sl2, m_ref, accl, acc, nmu);
                exp_p<false, false>(scur, lim0, sl2, nmu, ph, pl);
                row_sums(ph, rs);
            }
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) accl[nt][0] += rs[nt][0];   // element 0 is the one read at the end
            pv<false, true, false>(ph, pl, Vcur, vto, accl, acc);
            wait_loads();
            __syncthreads();
        };
        {
            int x = 0;
            for (; x + 1 < nfast; x += 2) {
                fast_iter(K0, K1, V0, V1, x, sa, sb);
                fast_iter(K1, K0, V1, V0, x + 1, sb, sa);
            }
            if (x < nfast) fast_iter(K0, K1, V0, V1, x, sa, sb);
        }
        int x = nfast;
        const int kloaded = nfast + 1;   // K(0 .. kloaded) are loaded or being loaded
        uint32_t voff[4];
        {
            const int e = m >> 2;
            const int q = m & 3;
#pragma unroll
            for (int cl = 0; cl < 4; ++cl)
                voff[cl] = static_cast<uint32_t>((8 * kg + e) * LROW + 32 * (cl ^ e) + 16 * (q >> 1) + 8 * (q & 1));
        }
        auto slow_iter = [&](const uint8_t *Kcur, uint8_t *Knext, const uint8_t *Vcur, uint8_t *Vnext, int x) {
            if (x + 1 < nsteps) {
                if (x + 1 > kloaded) issue_k(Knext, x + 1);
                issue_v(Vnext, x + 1);
            }
            const int k0 = x * kStepKeys;
            // A step below the tile's first token is visible to every row: no mask.
            if (k0 < wkeys) {
                if (x < nfull)
                    step<false, true>(Kcur, Vcur, k0, koff, voff, qop, cap, sl2, m_ref, accl, acc);
                else
                    step<true, true>(Kcur, Vcur, k0, koff, voff, qop, cap, sl2, m_ref, accl, acc);
            }
            wait_loads();
            __syncthreads();
        };
        if (x < nsteps && (x & 1)) {
            slow_iter(K1, K0, V1, V0, x);
            ++x;
        }
        for (; x + 1 < nsteps; x += 2) {
            slow_iter(K0, K1, V0, V1, x);
            slow_iter(K1, K0, V1, V0, x + 1);
        }
        if (x < nsteps) slow_iter(K0, K1, V0, V1, x);

#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const float l_tot = accl[nt][0];   // the row sum (the fast loop adds to element 0 only)
            const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
            // acc[nt][c][q] is O[row][d = 16c + 4kg + q].
            if (cap[nt] > 0) {
#pragma unroll
                for (int c = 0; c < VEC; ++c) {
                    const float x[4] = {acc[nt][c][0] * inv, acc[nt][c][1] * inv, acc[nt][c][2] * inv,
                                        acc[nt][c][3] * inv};
                    store4<kOut>(P.o + (orow[nt] * D + 16 * c + 4 * kg) * (kOut == kF32 ? 4 : 2), x);
                }
            }
        }
    }
};

template <int kIn, int kOut, int D>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillParams P) {
    using T = PrefillTile<kIn, kOut, D>;
    // The K and V slots of two steps, four separate arrays; see run().
    __shared__ __align__(16) uint8_t k0s[T::kSlotBytes];
    __shared__ __align__(16) uint8_t k1s[T::kSlotBytes];
    __shared__ __align__(16) uint8_t v0s[T::kSlotBytes];
    __shared__ __align__(16) uint8_t v1s[T::kSlotBytes];
    __shared__ int64_t s_item;
    const int tt = kPrefillRows / P.G;
    const int64_t items = count_items(P.seq_lens, P.batch, tt, P.h_kv);
    const int64_t g = gridDim.x;
    const int64_t w = blockIdx.x;
    // Every round but the last in the fixed snake order (the workgroups of a round
    // sweep neighbouring tiles of a sequence at about the same pace, so their K/V
    // reads meet in the cache); the last round's items -- the shortest tiles --
    // from the workspace's counter, longest first, so that workgroups on compute
    // units that ran faster take more of them.  One loop with one call of run():
    // a second inlined copy of the tile sweep costs registers in its inner loops.
    const int64_t rounds = (items + g - 1) / g;
    const int64_t first_dyn = P.queue && rounds > 1 ? (rounds - 1) * g : items;
    for (int64_t r = 0;; ++r) {
        int64_t it;
        if (r * g < first_dyn) {
            it = r * g + ((r & 1) ? g - 1 - w : w);   // snake order
            if (it >= first_dyn) continue;
        } else {
            if (first_dyn >= items) break;
            if (threadIdx.x == 0)
                s_item = first_dyn + static_cast<int64_t>(atomicAdd(P.queue, 1ull));   // relaxed; selects work only
            __syncthreads();
            it = s_item;
            __syncthreads();   // every thread has read it before thread 0 takes the next
            if (it >= items) break;   // each workgroup's last take is past the end
        }
        int b, len;
        int64_t off, local, steps;
        locate_item(P.seq_lens, P.batch, tt, P.h_kv, it, b, off, len, local, steps);
        const int ntile = static_cast<int>(tiles_of(len, tt));
        const int j = static_cast<int>(local / ntile);
        const int tile = ntile - 1 - static_cast<int>(local - static_cast<int64_t>(j) * ntile);   // longest first
        T::run(P, k0s, k1s, v0s, v1s, off, len, j, tile, steps);
    }
}

// Transposed fp16 copy of V for the fast loop: workgroup j * nvb + blk takes
// block blk of kv head j -- step x of sequence b, the keys 64 x .. + 63 (zeros
// beyond the sequence's end) -- and writes it as D rows of 64 keys (row d holds
// v[key, j, d] for the 64 keys, in fp16: bf16 input is converted, exactly for
// magnitudes in fp16's normal range).  flags[j * nvb + blk] = 1 for bf16 input
// whose block holds a largest |v| not in [2^-10, 2^16) (or a non-finite value):
// that step must not take the fp16 product.  Blocks past the last step of the
// last sequence are left alone.
template <int kIn, int D>
__global__ __launch_bounds__(kVprepThreads) void vprep_kernel(VprepParams p) {
    constexpr int ROWB = D * 2;                    // bytes of one key row (one kv head)
    constexpr int CH = ROWB / 16;                  // 16-byte chunks per key row
    constexpr int K = kPrefillStepKeys;            // keys per block
    constexpr int kPitch = ROWB + 16;              // LDS row pitch (keys x d tile)
    typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
    __shared__ __align__(16) uint8_t tile[K * kPitch];
    __shared__ unsigned wmax[kVprepThreads / kWave];
    const int64_t idx = blockIdx.x;
    if (idx == 0 && threadIdx.x == 0) *p.queue = 0;   // the prefill kernel's tile queue starts at item 0
    const int j = static_cast<int>(idx / p.nvb);
    const int64_t blk = idx - static_cast<int64_t>(j) * p.nvb;
    int b, len;
    int64_t off, x, steps;
    locate_item(p.seq_lens, p.batch, K, 1, blk, b, off, len, x, steps);
    if (b >= p.batch) return;   // the same for the whole workgroup
    const int tid = static_cast<int>(threadIdx.x);
    // Load the block's key rows (16 bytes a thread at a time) into LDS as fp16.
    u16x2_t mag = {0, 0};
    for (int c = tid; c < K * CH; c += kVprepThreads) {
        const int key = c / CH;
        const int dc = c - key * CH;
        const int64_t row = x * K + key;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (row < len) w = *reinterpret_cast<const uint4 *>(p.v + ((off + row) * p.h_kv + j) * ROWB + dc * 16);
        if constexpr (kIn == kBf16) {
            const uint32_t a[4] = {w.x, w.y, w.z, w.w};
            uint32_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mag = __builtin_elementwise_max(mag, __builtin_bit_cast(u16x2_t, a[i] & 0x7fff7fffu));
                const f32x2_t f = {__uint_as_float(a[i] << 16), __uint_as_float(a[i] & 0xffff0000u)};
                h[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
            }
            w = make_uint4(h[0], h[1], h[2], h[3]);
        }
        *reinterpret_cast<uint4 *>(tile + key * kPitch + dc * 16) = w;
    }
    __syncthreads();
    // Write row d, keys 8 kc .. + 7, as one 16-byte chunk.
    uint8_t *dst = p.vt + idx * (D * K * 2);
    for (int c = tid; c < D * (K / 8); c += kVprepThreads) {
        const int d = c / (K / 8);
        const int kc = c - d * (K / 8);
        uint32_t o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t lo = *reinterpret_cast<const uint16_t *>(tile + (8 * kc + 2 * t) * kPitch + d * 2);
            const uint32_t hi = *reinterpret_cast<const uint16_t *>(tile + (8 * kc + 2 * t + 1) * kPitch + d * 2);
            o[t] = lo | (hi << 16);
        }
        *reinterpret_cast<uint4 *>(dst + d * (K * 2) + kc * 16) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    if constexpr (kIn == kBf16) {
        // Largest magnitude bits of the block (bf16 magnitude bits order like the
        // magnitudes; NaN and inf sort above every finite value).
        unsigned mm = mag.x > mag.y ? mag.x : mag.y;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const unsigned y = static_cast<unsigned>(__shfl_xor(static_cast<int>(mm), d));
            mm = mm > y ? mm : y;
        }
        if (lane_id() == 0) wmax[tid / kWave] = mm;
        __syncthreads();
        if (tid == 0) {
#pragma unroll
            for (int i = 1; i < kVprepThreads / kWave; ++i) mm = mm > wmax[i] ? mm : wmax[i];
            p.flags[idx] = (mm >= 0x4780u || mm < 0x3a80u) ? 1 : 0;
        }
    } else {
        if (tid == 0) p.flags[idx] = 0;
    }
}

template <int kIn>
hipError_t launch_vprep_in(const VprepParams &p, int D, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.nvb * p.h_kv));   // < 2^31 by the argument checks
    if (D == 128)
        hipLaunchKernelGGL((vprep_kernel<kIn, 128>), grid, dim3(kVprepThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((vprep_kernel<kIn, 64>), grid, dim3(kVprepThreads), 0, stream, p);
    return hipGetLastError();
}

template <int kIn, int kOut>
hipError_t launch_pio(const PrefillParams &P, int D, int blocks, hipStream_t stream) {
    if (D == 128)
        hipLaunchKernelGGL((prefill_kernel<kIn, kOut, 128>), dim3(blocks), dim3(kPrefillThreads), 0, stream, P);
    else
        hipLaunchKernelGGL((prefill_kernel<kIn, kOut, 64>), dim3(blocks), dim3(kPrefillThreads), 0, stream, P);
    return hipGetLastError();
}

template <int kIn, int kOut>
hipError_t occupancy_pio(int D, int *blocks_per_cu) {
    return D == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, prefill_kernel<kIn, kOut, 128>,
                                                                   kPrefillThreads, 0)
                    : hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, prefill_kernel<kIn, kOut, 64>,
                                                                   kPrefillThreads, 0);
}

}  // namespace

// (in, out) pairs the prefill validation admits: (bf16, bf16), (bf16, f32),
// (f16, f16), (f16, f32).
hipError_t launch_prefill(const PrefillParams &P, int in_dtype, int out_dtype, int D, int blocks,
                          hipStream_t stream) {
    if (in_dtype == kBf16) return out_dtype == kBf16 ? launch_pio<kBf16, kBf16>(P, D, blocks, stream)
                                                     : launch_pio<kBf16, kF32>(P, D, blocks, stream);
    return out_dtype == kF16 ? launch_pio<kF16, kF16>(P, D, blocks, stream)
                             : launch_pio<kF16, kF32>(P, D, blocks, stream);
}

hipError_t launch_vprep(const VprepParams &p, int in_dtype, int D, hipStream_t stream) {
    return in_dtype == kBf16 ? launch_vprep_in<kBf16>(p, D, stream) : launch_vprep_in<kF16>(p, D, stream);
}

hipError_t prefill_occupancy(int in_dtype, int out_dtype, int D, int *blocks_per_cu) {
    if (in_dtype == kBf16) return out_dtype == kBf16 ? occupancy_pio<kBf16, kBf16>(D, blocks_per_cu)
                                                     : occupancy_pio<kBf16, kF32>(D, blocks_per_cu);
    return out_dtype == kF16 ? occupancy_pio<kF16, kF16>(D, blocks_per_cu)
                             : occupancy_pio<kF16, kF32>(D, blocks_per_cu);
}

}  // namespace gqa
