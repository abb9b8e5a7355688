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
//   * K and V go HBM/L2 -> LDS in 128-key stages (double buffered, one barrier
//     per stage) that all 256 rows share, so the K/V bytes per output row fall
//     with the tile height.  The loads write LDS directly (buffer loads with the
//     LDS as destination: no registers, no LDS store instructions), the next
//     stage's loads in flight during the whole current stage.  A stage is
//     computed as two 64-key steps.  LDS rows are XOR-swizzled in 16-byte chunks
//     (one pattern for K, one for V) so the operand reads hit distinct banks; a
//     direct load writes lane i's 16 bytes at base + 16 i, so the swizzle is
//     applied by choosing which global chunk each lane fetches.
//   * Each wavefront owns 32 rows as two 16-row N tiles of
//     v_mfma_f32_16x16x32_{bf16,f16}: S^T = K Q^T with the keys on the M axis
//     (the K rows are read from LDS in the key order that leaves lane l holding
//     keys 8*(l/16) .. +7 of its row), then O^T += V^T P^T and l += 1^T P^T (the
//     row sums come out of the matrix core, from the same rounded P).  The V^T
//     operand comes straight out of LDS through transpose reads.  Two wavefronts
//     share a SIMD (at most 256 VGPRs each, no AGPR traffic).
//   * P V precision: by default P is rounded to fp16 and V read as fp16, one
//     product per step.  For bf16 input a pre-pass (vconv_kernel) writes an fp16
//     copy of V into the workspace -- exact for magnitudes in fp16's normal range
//     -- and flags every 128-token block whose largest |v| is not in
//     [2^-10, 2^16); from the first stage that touches a flagged block on, a
//     tile's sweep uses the split product (P as a high and a low part in the
//     input format, V as given, two products), which the diagonal band always
//     uses and which the caller can ask for everywhere.
//   * The running maximum is allowed to lag the true one by up to 8 (log2
//     units): the accumulators are rescaled only when some row of an N tile
//     exceeds its reference by more, which removes almost every rescale of the
//     accumulators.  Weights are then at most 2^(8+7) (the 2^7 keeps small
//     weights inside fp16's exponent range), and the common factor cancels in
//     O / l.
//   * Tiles are handed out in a fixed snake order over a persistent grid: the
//     tiles of a (sequence, kv head) are enumerated last token first (longest
//     first), and workgroup w takes tiles w, 2g-1-w, 2g+w, ... (g = grid size),
//     which evens out the causal triangle's work.
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
#ifndef GQA_PREFILL_STAGE_STEPS
#define GQA_PREFILL_STAGE_STEPS 2
#endif
constexpr int kStageSteps = GQA_PREFILL_STAGE_STEPS;   // compute steps per LDS stage (per barrier)
constexpr int kStageKeys = kStepKeys * kStageSteps;
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
// length and local = the item's index among b's items.
__device__ void locate_item(const int32_t *seq_lens, int batch, int tt, int h_kv, int64_t it, int &b,
                            int64_t &off, int &len, int64_t &local) {
    const int lane = lane_id();
    int64_t run_items = 0, run_len = 0;
    for (int base = 0; base < batch; base += kWave) {
        const int i = base + lane;
        const int64_t li = (i < batch) ? seq_len_at(seq_lens, i) : 0;
        const int64_t ni = tiles_of(li, tt) * h_kv;
        const int64_t inc_n = inclusive_scan64(ni);
        const int64_t inc_l = inclusive_scan64(li);
        const bool hit = (i < batch) && (run_items + inc_n > it);
        const unsigned long long mask = __ballot(hit);
        if (mask) {
            const int src = __ffsll(static_cast<long long>(mask)) - 1;
            b = base + src;
            len = uniform32(static_cast<int>(shfl64(li, src)));
            off = uniform64(run_len + shfl64(inc_l, src) - len);
            local = uniform64(it - (run_items + shfl64(inc_n, src) - shfl64(ni, src)));
            return;
        }
        run_items += shfl64(inc_n, kWave - 1);
        run_len += shfl64(inc_l, kWave - 1);
    }
    b = batch;
    off = run_len;
    len = 0;
    local = 0;
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
    static constexpr int kTileBytes = kStageKeys * LROW;
    // LDS regions of a stage buffer: K, and V (fp16 in the fast loop, as given
    // in the masked / split loop).
    static constexpr int kRegions = 2;
    static constexpr int kK = 0, kV = 1;
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

    // LDS layout of a K or V tile: key row r at r * LROW, its 16-byte chunk c at
    // chunk position c ^ swz(r) (K) or c ^ swzv(r) (V).  One K operand read hits
    // rows {0-3, 8-11, 16-19, 24-27} (+4 for the second block) at one chunk; one
    // transposed V read (see v_operand) hits 4 consecutive rows at 2 chunks.  The
    // swizzles spread both over distinct banks.
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

    // One step: S^T = K Q^T for the N tiles, online softmax with the lagging
    // maximum, then O^T += V^T P^T and l += 1^T P^T (the row sums from the same
    // rounded P as the product).
    //   kDiag   some key of the step lies beyond some row's causal limit: mask
    //           (chosen per wavefront and step; off the diagonal no row needs it).
    //   kSplit  P in the input's 16-bit format as a high and a low part (two
    //           products, V as given); otherwise P in fp16 (one product) against
    //           V converted to fp16.
    // sl2 > 0 (a negative scale is folded into Q).
    template <bool kDiag, bool kSplit>
    __device__ __forceinline__ static void step(const uint8_t *Kt, const uint8_t *Vt, int k0,
                                                const uint32_t (&koff)[2][NKP], const uint32_t (&voff)[4],
                                                const uint4 (&qop)[kNT][NKP], const int (&cap)[kNT],
                                                float sl2, float (&m_ref)[kNT], f32x4_t (&accl)[kNT],
                                                f32x4_t (&acc)[kNT][VEC]) {
        constexpr bool kPvHalf = kSplit ? kHalf : true;   // element type of the P V product
        constexpr int kH = kStepKeys / 32;                 // 32-key halves of the step
        const int lane = lane_id();
        const int kg = lane >> 4;
        // S^T = K Q^T, half by half: lane holds keys k0 + 32h + 8kg + i of its rows.
        float sv[kNT][kH][8];
#pragma unroll
        for (int h = 0; h < kH; ++h) {
            uint4 kop[2][NKP];
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int p = 0; p < NKP; ++p)
                    kop[b][p] = *reinterpret_cast<const uint4 *>(Kt + h * 32 * LROW + koff[b][p]);
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int p = 0; p < NKP; ++p) s = mfma16<kHalf>(kop[b][p], qop[nt][p], s);
#pragma unroll
                    for (int q = 0; q < 4; ++q) sv[nt][h][4 * b + q] = s[q];
                }
        }
        // Row maxima of the step and the (rare) move of the references, for both N
        // tiles before any exponential, so that everything after it -- P for
        // each half, the P V products, the row sums -- is one branch-free stretch
        // the scheduler can interleave (the exponentials of half 1 with the
        // products of half 0).
        int lim[kNT];
        float mxs[kNT];
        bool move = false;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            lim[nt] = cap[nt] - (k0 + 8 * kg);   // key 32h + i is visible iff 32h + i < lim
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
        // Move the references only when some row's maximum passes its reference by
        // more than the allowed lag (wave-uniform branch; rows that did not ask
        // follow along, with alpha = 1 where nothing changes).
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
        // p = 2^(s*sl2 - m_ref + kOff); a row with no visible key yet keeps the
        // reference -inf and takes 0 in its place (its weights are masked to 0).
        float nmu[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
            nmu[nt] = static_cast<float>(kOff) - (m_ref[nt] == -INFINITY ? 0.f : m_ref[nt]);
        uint4 bhi[kNT][kH], blo[kNT][kH];
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
            // O^T += V^T P^T for this half, d block c (d = 16c + M): the A operand is
            // read transposed from LDS (keys 32h + 8kg + i, d = 16c + m).
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                const uint8_t *base = Vt + h * 32 * LROW + (c >> 2) * 128 + voff[c & 3];
                const uint2 lo = lds_read_tr16(base);
                const uint2 hi = lds_read_tr16(base + 4 * LROW);
                const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) {
                    acc[nt][c] = mfma16<kPvHalf>(av, bhi[nt][h], acc[nt][c]);
                    if constexpr (kSplit) acc[nt][c] = mfma16<kPvHalf>(av, blo[nt][h], acc[nt][c]);
                }
            }
        }
        const uint32_t one = kPvHalf ? kOnesF16 : kOnesIn;
        const uint4 ones = make_uint4(one, one, one, one);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
            for (int h = 0; h < kH; ++h) {
                accl[nt] = mfma16<kPvHalf>(ones, bhi[nt][h], accl[nt]);
                if constexpr (kSplit) accl[nt] = mfma16<kPvHalf>(ones, blo[nt][h], accl[nt]);
            }
    }

    // Tile `tile` of (sequence b at token offset off, length len; kv head j).
    __device__ __forceinline__ static void run(const PrefillParams &P, uint8_t (*buf0)[kTileBytes],
                                               uint8_t (*buf1)[kTileBytes], int64_t off, int len, int j, int tile) {
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
        const int nstages = (nkeys + kStageKeys - 1) / kStageKeys;
        const uint8_t *kbase = P.k + (off * P.h_kv + j) * ROWB;
        const uint8_t *vbase = P.v + (off * P.h_kv + j) * ROWB;

        // Direct load i of this wavefront fills LDS chunks p = 64 (kPer wave + i) +
        // lane of a step's K (or V) region: row r = p / CH at position p % CH,
        // which holds the row's global chunk (p % CH) ^ swz(r) (swzv(r) for V).
        uint32_t gk[kPer], gv[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int p = (wave * kPer + i) * kWave + lane;
            const int r = p / CH;
            const int pos = p - r * CH;
            gk[i] = static_cast<uint32_t>(r * rowstride + (pos ^ swz(r)) * 16);
            gv[i] = static_cast<uint32_t>(r * rowstride + (pos ^ swzv(r)) * 16);
        }
        // Per-lane LDS offsets of the step's operands (fixed for the whole tile):
        // K operand of block b, piece p: row 8(m/4) + 4b + m%4, chunk 4p + kg.
        // V (transposed read, t = 0, d block c = 4 ch + cl): lane 4e + q of group kg
        // addresses row 8kg + e (+ 4t), d = 16c + 4q, i.e. chunk 2c + q/2, bytes
        // 8 (q % 2); with the swizzle (2c + q/2) ^ 2e = 8ch + 2(cl ^ e) + q/2.
        uint32_t koff[2][NKP], voff[4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int r = 8 * (m >> 2) + 4 * b + (m & 3);
#pragma unroll
            for (int p = 0; p < NKP; ++p) koff[b][p] = static_cast<uint32_t>(r * LROW + ((4 * p + kg) ^ swz(r)) * 16);
        }
        {
            const int e = m >> 2;
            const int q = m & 3;
#pragma unroll
            for (int cl = 0; cl < 4; ++cl)
                voff[cl] = static_cast<uint32_t>((8 * kg + e) * LROW + 32 * (cl ^ e) + 16 * (q >> 1) + 8 * (q & 1));
        }
        // Stages that run the fast (fp16 P V) loop: every stage below the tile's
        // first token, up to the first stage touching a 128-token block of V that
        // the pre-pass flagged (blocks at or beyond the copy's end count as
        // flagged).  Stage s holds tokens off + 128 s .. + 127 of the packed axis.
        const int nfull = min(nstages, (tstart + 1) / kStageKeys);
        int nfast = 0;
        if (!P.split_pv) {
            if constexpr (kHalf) {
                nfast = nfull;
            } else if (nfull > 0) {
                constexpr int VB = kPrefillVBlock;
                const int64_t g_lo = off / VB;
                const int64_t g_hi = (off + static_cast<int64_t>(nfull) * kStageKeys - 1) / VB;
                int64_t g_bad = -1;
                for (int64_t g = g_lo; g <= g_hi; g += kWave) {
                    const int64_t gl = g + lane;
                    const bool bad = gl <= g_hi && (gl >= P.nblk || P.vflags[j * P.nblk + gl] != 0);
                    const unsigned long long mask = __ballot(bad);
                    if (mask) {
                        g_bad = g + (__ffsll(static_cast<long long>(mask)) - 1);
                        break;
                    }
                }
                nfast = nfull;
                if (g_bad >= 0) {
                    const int64_t t = g_bad * VB - off - kStageKeys + 1;   // first stage reaching block g_bad
                    const int64_t s_bad = t <= 0 ? 0 : (t + kStageKeys - 1) / kStageKeys;
                    nfast = static_cast<int>(min(static_cast<int64_t>(nfull), s_bad));
                }
                nfast = uniform32(nfast);
            }
        }
        const uint8_t *vfast = nfast > 0 ? P.v16 + (off * P.h_kv + j) * ROWB : vbase;
        // Loads stage sg into buffer B (both 64-key parts, K and V); rows at or
        // beyond the sequence's end read as zero.  V comes from the fp16 copy for
        // stages of the fast loop.
        auto issue = [&](uint8_t (*B)[kTileBytes], int sg) {
            const uint8_t *vsrc = sg < nfast ? vfast : vbase;
#pragma unroll
            for (int pt = 0; pt < kStageSteps; ++pt) {
                const int k0 = sg * kStageKeys + pt * kStepKeys;
                const uint32_t bytes = k0 < len ? static_cast<uint32_t>(min(kStepKeys, len - k0) * rowstride) : 0u;
                const int64_t boff = static_cast<int64_t>(k0) * rowstride;
                const auto rsk = make_rsrc(kbase + boff, bytes);
                const auto rsv = make_rsrc(vsrc + boff, bytes);
#pragma unroll
                for (int i = 0; i < kPer; ++i) {
                    const uint32_t lo = static_cast<uint32_t>(pt * kStepKeys * LROW + (wave * kPer + i) * kWave * 16);
                    lds_load16(rsk, B[kK] + lo, gk[i]);
                    lds_load16(rsv, B[kV] + lo, gv[i]);
                }
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
        issue(buf0, 0);
        wait_loads();
        __syncthreads();
        // Steps whose keys every row of the tile sees (below the tile's first
        // token) run unmasked with fp16 P V; the rest -- the tile's diagonal band,
        // and everything from the first stage whose V range does not suit fp16 on
        // -- masked with the exact split product, each wavefront skipping the steps
        // beyond its own last token.  Two loops, so the fast one carries no masking
        // or fallback code at all.  Each stage starts the loads of the next one
        // into the other buffer and ends with one barrier.  The buffers are two
        // separate LDS arrays named at every use, so the compiler can tell that
        // the operand reads of one never touch the loads in flight to the other.
        auto stage_fast = [&](uint8_t (*cur)[kTileBytes], uint8_t (*nxt)[kTileBytes], int st) {
            if (st + 1 < nstages) issue(nxt, st + 1);
#pragma unroll
            for (int pt = 0; pt < kStageSteps; ++pt) {
                // Each step is scheduled on its own: interleaving two steps would
                // need more than the 256 registers of two wavefronts per SIMD.
                __builtin_amdgcn_sched_barrier(0);
                step<false, false>(cur[kK] + pt * kStepKeys * LROW, cur[kV] + pt * kStepKeys * LROW,
                                   st * kStageKeys + pt * kStepKeys, koff, voff, qop, cap, sl2, m_ref, accl, acc);
            }
            __builtin_amdgcn_sched_barrier(0);
            wait_loads();
            __syncthreads();
        };
        auto stage_slow = [&](uint8_t (*cur)[kTileBytes], uint8_t (*nxt)[kTileBytes], int st) {
            if (st + 1 < nstages) issue(nxt, st + 1);
#pragma unroll
            for (int pt = 0; pt < kStageSteps; ++pt) {
                __builtin_amdgcn_sched_barrier(0);
                const int k0 = st * kStageKeys + pt * kStepKeys;
                if (k0 < wkeys)
                    step<true, true>(cur[kK] + pt * kStepKeys * LROW, cur[kV] + pt * kStepKeys * LROW, k0, koff,
                                     voff, qop, cap, sl2, m_ref, accl, acc);
            }
            wait_loads();
            __syncthreads();
        };
        // Stage st computes from buffer st & 1; the loops go two stages at a time
        // so that every call names its buffers statically.
        int st = 0;
        for (; st + 1 < nfast; st += 2) {
            stage_fast(buf0, buf1, st);
            stage_fast(buf1, buf0, st + 1);
        }
        if (st < nfast) {
            stage_fast(buf0, buf1, st);
            ++st;
        }
        if (st < nstages && (st & 1)) {
            stage_slow(buf1, buf0, st);
            ++st;
        }
        for (; st + 1 < nstages; st += 2) {
            stage_slow(buf0, buf1, st);
            stage_slow(buf1, buf0, st + 1);
        }
        if (st < nstages) stage_slow(buf0, buf1, st);

#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const float l_tot = accl[nt][0];   // every element of the ones product is the row sum
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
    // The two stage buffers (K and V regions each) are separate arrays; see run().
    __shared__ __align__(16) uint8_t buf0[T::kRegions][T::kTileBytes];
    __shared__ __align__(16) uint8_t buf1[T::kRegions][T::kTileBytes];
    const int tt = kPrefillRows / P.G;
    const int64_t items = count_items(P.seq_lens, P.batch, tt, P.h_kv);
    const int64_t g = gridDim.x;
    const int64_t w = blockIdx.x;
    for (int64_t r = 0; r * g < items; ++r) {
        const int64_t it = r * g + ((r & 1) ? g - 1 - w : w);   // snake order
        if (it >= items) continue;
        int b, len;
        int64_t off, local;
        locate_item(P.seq_lens, P.batch, tt, P.h_kv, it, b, off, len, local);
        const int ntile = static_cast<int>(tiles_of(len, tt));
        const int j = static_cast<int>(local / ntile);
        const int tile = ntile - 1 - static_cast<int>(local - static_cast<int64_t>(j) * ntile);   // longest first
        T::run(P, buf0, buf1, off, len, j, tile);
    }
}

// fp16 copy of bf16 V and the range flags of its 128-token blocks: workgroup
// j * nblk + g converts rows g * 128 .. + 127 (those below `total`) of kv head j
// and sets flags[j * nblk + g] to 1 if the block's largest |v| is not in
// [2^-10, 2^16) (or is not finite), else 0.  The conversion is exact for values
// in fp16's normal range; flagged blocks are never read from the copy.
template <int D>
__global__ __launch_bounds__(kVconvThreads) void vconv_kernel(VconvParams p) {
    constexpr int ROWB = D * 2;
    constexpr int CH = ROWB / 16;
    constexpr int kChunks = kPrefillVBlock * CH;
    typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
    const int64_t idx = blockIdx.x;
    const int j = static_cast<int>(idx / p.nblk);
    const int64_t g = idx - static_cast<int64_t>(j) * p.nblk;
    const int tid = static_cast<int>(threadIdx.x);
    u16x2_t mag = {0, 0};
    for (int c = tid; c < kChunks; c += kVconvThreads) {
        const int64_t row = g * kPrefillVBlock + c / CH;
        if (row >= p.total) break;   // rows grow with c
        const int64_t o = (row * p.h_kv + j) * ROWB + (c % CH) * 16;
        const uint4 x = *reinterpret_cast<const uint4 *>(p.v + o);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        uint32_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mag = __builtin_elementwise_max(mag, __builtin_bit_cast(u16x2_t, w[i] & 0x7fff7fffu));
            const f32x2_t f = {__uint_as_float(w[i] << 16), __uint_as_float(w[i] & 0xffff0000u)};
            h[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
        }
        *reinterpret_cast<uint4 *>(p.v16 + o) = make_uint4(h[0], h[1], h[2], h[3]);
    }
    // Largest magnitude bits of the block (bf16 magnitude bits order like the
    // magnitudes; NaN and inf sort above every finite value).
    unsigned m = mag.x > mag.y ? mag.x : mag.y;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const unsigned y = static_cast<unsigned>(__shfl_xor(static_cast<int>(m), d));
        m = m > y ? m : y;
    }
    __shared__ unsigned wmax[kVconvThreads / kWave];
    if (lane_id() == 0) wmax[tid / kWave] = m;
    __syncthreads();
    if (tid == 0) {
#pragma unroll
        for (int i = 1; i < kVconvThreads / kWave; ++i) m = m > wmax[i] ? m : wmax[i];
        p.flags[idx] = (m >= 0x4780u || m < 0x3a80u) ? 1 : 0;
    }
}

hipError_t launch_vconv_impl(const VconvParams &p, int D, int h_kv, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.nblk * h_kv));   // <= 2^30 by the total_tokens * h_kv limit
    if (D == 128)
        hipLaunchKernelGGL(vconv_kernel<128>, grid, dim3(kVconvThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(vconv_kernel<64>, grid, dim3(kVconvThreads), 0, stream, p);
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

hipError_t launch_vconv(const VconvParams &p, int D, int h_kv, hipStream_t stream) {
    return launch_vconv_impl(p, D, h_kv, stream);
}

hipError_t prefill_occupancy(int in_dtype, int out_dtype, int D, int *blocks_per_cu) {
    if (in_dtype == kBf16) return out_dtype == kBf16 ? occupancy_pio<kBf16, kBf16>(D, blocks_per_cu)
                                                     : occupancy_pio<kBf16, kF32>(D, blocks_per_cu);
    return out_dtype == kF16 ? occupancy_pio<kF16, kF16>(D, blocks_per_cu)
                             : occupancy_pio<kF16, kF32>(D, blocks_per_cu);
}

}  // namespace gqa
