// driver.cpp -- host-only driver for an AddressSanitizer / UndefinedBehavior-
// Sanitizer build of the library's host C++ (argument validation and launch
// planning, plan.cpp) and of the fp64 CPU oracle (oracle.c, test
// infrastructure).  No HIP, no Python: tests/test_host_sanitize.py compiles this
// file with g++ and the sanitizers and runs it.
//
// It walks the validation rules over a grid of bad and edge-case arguments
// (null pointers, shapes, unsupported sizes, alignment, scale, tuning ranges,
// workspace sizes, t_q limits, h_kv at its 65,536 limit), checks the invariants
// of every plan it makes, and runs the oracle on empty, negative and shorter-
// than-t_q sequences, checking their defined results (zeros for a query that
// sees no key, finite values elsewhere).  Exit status 0 means every check held.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "host.h"

extern "C" {
int oracle_gqa_decode_tq_f64(const void *q, const void *k, const void *v, const int32_t *seq_lens,
                             int32_t batch, int32_t t_q, int32_t h_q, int32_t h_kv, int32_t d, double scale,
                             int32_t dtype, double *out);
int oracle_partial_f64(const void *q, const void *k, const void *v, const int32_t *seq_lens, int32_t batch,
                       int32_t h_q, int32_t h_kv, int32_t d, double scale, int32_t dtype, int32_t b, int32_t h,
                       int32_t t0, int32_t t1, double *m_out, double *l_out, double *O);
int oracle_softmax_weights_f64(const void *q, const void *k, const int32_t *seq_lens, int32_t batch,
                               int32_t h_q, int32_t h_kv, int32_t d, double scale, int32_t dtype, int32_t b,
                               int32_t h, double *w);
}

static int g_checks = 0, g_failures = 0;

#define CHECK(cond, ...)                                              \
    do {                                                              \
        ++g_checks;                                                   \
        if (!(cond)) {                                                \
            ++g_failures;                                             \
            std::fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);                        \
            std::fprintf(stderr, "\n");                               \
        }                                                             \
    } while (0)

static gqa_decode_args base_args() {
    gqa_decode_args a;
    std::memset(&a, 0, sizeof a);
    a.q = reinterpret_cast<const void *>(0x10000);
    a.k = reinterpret_cast<const void *>(0x20000);
    a.v = reinterpret_cast<const void *>(0x30000);
    a.o = reinterpret_cast<void *>(0x40000);
    a.seq_lens = reinterpret_cast<const int32_t *>(0x50000);
    a.batch = 4;
    a.h_q = 32;
    a.h_kv = 8;
    a.d_head = 128;
    a.scale = 0.088f;
    a.in_dtype = GQA_DTYPE_BF16;
    a.out_dtype = GQA_DTYPE_BF16;
    return a;
}

static void validation_grid() {
    gqa_decode_args a = base_args();
    CHECK(gqa::validate(&a) == GQA_OK, "base arguments");
    CHECK(gqa::validate(nullptr) == GQA_ERR_NULL, "null args");
    const char *fields[] = {"q", "k", "v", "o", "seq_lens"};
    for (int f = 0; f < 5; ++f) {
        a = base_args();
        const void **slot[] = {&a.q, &a.k, &a.v, const_cast<const void **>(reinterpret_cast<void **>(&a.o)),
                               reinterpret_cast<const void **>(&a.seq_lens)};
        *slot[f] = nullptr;
        CHECK(gqa::validate(&a) == GQA_ERR_NULL, "null %s", fields[f]);
    }
    struct Case {
        int32_t batch, h_q, h_kv, d, t_q, in, out;
        int expect;
    } cases[] = {
        {0, 32, 8, 128, 0, 0, 0, GQA_ERR_SHAPE},
        {-1, 32, 8, 128, 0, 0, 0, GQA_ERR_SHAPE},
        {4, 0, 8, 128, 0, 0, 0, GQA_ERR_SHAPE},
        {4, 32, 0, 128, 0, 0, 0, GQA_ERR_SHAPE},
        {4, 30, 8, 128, 0, 0, 0, GQA_ERR_SHAPE},
        {4, 32, 8, 128, -1, 0, 0, GQA_ERR_SHAPE},
        {1 << 20, 1 << 12, 1 << 12, 128, 0, 0, 0, GQA_ERR_SHAPE},      // batch * h_q > 2^31 - 1
        {1 << 18, 1 << 10, 1 << 10, 128, 8, 0, 0, GQA_ERR_SHAPE},      // batch * t_q * h_q = 2^31
        {4, 32, 8, 96, 0, 0, 0, GQA_ERR_UNSUPPORTED},
        {4, 32, 8, 256, 0, 0, 0, GQA_ERR_UNSUPPORTED},
        {4, 65, 1, 128, 0, 0, 0, GQA_ERR_UNSUPPORTED},
        {4, 64, 8, 128, 9, 0, 0, GQA_ERR_UNSUPPORTED},
        {4, 64, 8, 128, 8, 0, 0, GQA_OK},
        {4, 8, 8, 128, 64, 0, 0, GQA_OK},
        {4, 8, 8, 128, 65, 0, 0, GQA_ERR_UNSUPPORTED},
        {4, 65537, 65537, 128, 0, 0, 0, GQA_ERR_UNSUPPORTED},
        {4, 65536, 65536, 128, 0, 0, 0, GQA_OK},
        {4, 32, 8, 128, 0, GQA_DTYPE_F32, GQA_DTYPE_BF16, GQA_ERR_UNSUPPORTED},
        {4, 32, 8, 128, 0, GQA_DTYPE_F16, GQA_DTYPE_BF16, GQA_ERR_UNSUPPORTED},
        {4, 32, 8, 128, 0, GQA_DTYPE_BF16, GQA_DTYPE_F16, GQA_ERR_UNSUPPORTED},
        {4, 32, 8, 128, 0, 7, 7, GQA_ERR_UNSUPPORTED},
        {4, 32, 8, 64, 0, GQA_DTYPE_F32, GQA_DTYPE_F32, GQA_OK},
        {4, 32, 8, 128, 0, GQA_DTYPE_F16, GQA_DTYPE_F32, GQA_OK},
    };
    for (const Case &c : cases) {
        a = base_args();
        a.batch = c.batch;
        a.h_q = c.h_q;
        a.h_kv = c.h_kv;
        a.d_head = c.d;
        a.t_q = c.t_q;
        a.in_dtype = c.in;
        a.out_dtype = c.out;
        CHECK(gqa::validate(&a) == c.expect, "shape case b%d hq%d hkv%d d%d tq%d in%d out%d: got %d want %d", c.batch,
              c.h_q, c.h_kv, c.d, c.t_q, c.in, c.out, gqa::validate(&a), c.expect);
    }
    for (int f = 0; f < 4; ++f) {
        a = base_args();
        const void **slot[] = {&a.q, &a.k, &a.v, const_cast<const void **>(reinterpret_cast<void **>(&a.o))};
        *slot[f] = reinterpret_cast<const void *>(0x10008);
        CHECK(gqa::validate(&a) == GQA_ERR_ALIGN, "misaligned pointer %d", f);
    }
    a = base_args();
    a.seq_lens = reinterpret_cast<const int32_t *>(0x50002);
    CHECK(gqa::validate(&a) == GQA_ERR_ALIGN, "misaligned seq_lens");
    const float bad_scales[] = {INFINITY, -INFINITY, NAN};
    for (float s : bad_scales) {
        a = base_args();
        a.scale = s;
        CHECK(gqa::validate(&a) == GQA_ERR_SCALE, "scale %g", static_cast<double>(s));
    }
    const int32_t bad_chunks[] = {-1, (1 << 24) + 1, INT32_MIN, INT32_MAX};
    for (int32_t n : bad_chunks) {
        a = base_args();
        a.num_chunks = n;
        CHECK(gqa::validate(&a) == GQA_ERR_ARG, "num_chunks %d", n);
    }
    const int32_t bad_min[] = {-5, (1 << 30) + 1, INT32_MIN, INT32_MAX};
    for (int32_t n : bad_min) {
        a = base_args();
        a.min_chunk = n;
        CHECK(gqa::validate(&a) == GQA_ERR_ARG, "min_chunk %d", n);
    }
    // Workspace: size and alignment checked once num_chunks is explicit.
    a = base_args();
    a.num_chunks = 100;
    gqa_decode_plan plan;
    CHECK(gqa::make_plan(&a, 256, 4, &plan) == GQA_OK, "plan for the workspace case");
    a.workspace = reinterpret_cast<void *>(0x100000);
    a.workspace_bytes = plan.workspace_bytes;
    CHECK(gqa::validate(&a) == GQA_OK, "workspace of the exact size");
    a.workspace_bytes = plan.workspace_bytes - 1;
    CHECK(gqa::validate(&a) == GQA_ERR_WORKSPACE, "workspace one byte short");
    a.workspace_bytes = plan.workspace_bytes;
    a.workspace = reinterpret_cast<void *>(0x100010);
    CHECK(gqa::validate(&a) == GQA_ERR_WORKSPACE, "misaligned workspace");
    a.workspace = reinterpret_cast<void *>(0x100000);
    a.workspace_bytes = 0;
    CHECK(gqa::validate(&a) == GQA_ERR_WORKSPACE, "zero-byte workspace");
    CHECK(gqa::make_plan(&a, 256, 4, nullptr) == GQA_ERR_WORKSPACE || gqa::make_plan(&a, 256, 4, nullptr) == GQA_ERR_NULL,
          "null plan");
    a = base_args();
    CHECK(gqa::make_plan(&a, 256, 4, nullptr) == GQA_ERR_NULL, "null plan pointer");
    CHECK(gqa::make_plan(&a, 0, 4, &plan) == GQA_ERR_ARG, "automatic plan without compute units");
    CHECK(gqa::make_plan(&a, 256, 0, &plan) == GQA_ERR_ARG, "automatic plan without occupancy");
}

static void plan_grid() {
    const int cus[] = {1, 7, 80, 256, 304};
    const int waves[] = {1, 2, 4, 8, 16};
    const int32_t batches[] = {1, 3, 64, 4096, 1 << 20};
    const int32_t hkvs[] = {1, 3, 8, 64, 65536};
    const int32_t Gs[] = {1, 4, 8, 16, 33, 64};
    const int32_t tqs[] = {0, 1, 2, 5, 8, 64};
    const int32_t chunks[] = {0, 1, 9, 1000, 1 << 24};
    const int32_t merges[] = {GQA_MERGE_AUTO, GQA_MERGE_KERNEL, GQA_MERGE_FUSED};
    int made = 0, fused = 0;
    for (int nc : cus)
        for (int wv : waves)
            for (int32_t batch : batches)
                for (int32_t hkv : hkvs)
                    for (int32_t G : Gs)
                        for (int32_t tq : tqs)
                            for (int32_t ch : chunks)
                            for (int32_t mg : merges) {
                                gqa_decode_args a = base_args();
                                a.merge = mg;
                                a.batch = batch;
                                a.h_kv = hkv;
                                a.h_q = static_cast<int32_t>(static_cast<int64_t>(G) * hkv > INT32_MAX ? 0 : G * hkv);
                                a.t_q = tq;
                                a.num_chunks = ch;
                                a.d_head = (G & 1) ? 64 : 128;
                                gqa_decode_plan p;
                                std::memset(&p, 0xab, sizeof p);
                                const int st = gqa::make_plan(&a, nc, wv, &p);
                                const int vst = gqa::validate(&a);
                                if (st != GQA_OK) {
                                    CHECK(st == vst || st == GQA_ERR_ARG, "plan status %d vs validate %d", st, vst);
                                    continue;
                                }
                                ++made;
                                const int64_t R = static_cast<int64_t>(G) * (tq > 0 ? tq : 1);
                                CHECK(p.num_chunks >= hkv && p.num_chunks % hkv == 0, "num_chunks %d h_kv %d",
                                      p.num_chunks, hkv);
                                CHECK(p.fused == 0 || p.fused == 1, "fused %d", p.fused);
                                CHECK(mg != GQA_MERGE_KERNEL || p.fused == 0, "kernel merge planned fused");
                                CHECK(mg != GQA_MERGE_FUSED || p.fused == 1, "fused merge planned as two kernels");
                                if (p.fused) {
                                    ++fused;
                                    const int64_t wgs = p.num_chunks / gqa::kWavesPerBlock;
                                    CHECK(p.num_chunks % (static_cast<int64_t>(hkv) * gqa::kWavesPerBlock) == 0,
                                          "fused num_chunks %d not a multiple of 4 h_kv %d", p.num_chunks, hkv);
                                    CHECK(p.fold_fanin >= 2 && p.fold_fanin <= gqa::kMaxFanIn &&
                                              (p.fold_fanin & (p.fold_fanin - 1)) == 0,
                                          "fan-in %d", p.fold_fanin);
                                    CHECK(static_cast<int64_t>(p.fold_fanin) * R * a.d_head * 4 <= gqa::kFoldBytes ||
                                              p.fold_fanin == 2, "fold volume of fan-in %d", p.fold_fanin);
                                    double span = 1;
                                    for (int l = 0; l < p.fold_levels; ++l) span *= p.fold_fanin;
                                    CHECK(span >= static_cast<double>(wgs / hkv), "levels %d of fan-in %d cover %g < %lld",
                                          p.fold_levels, p.fold_fanin, span, static_cast<long long>(wgs / hkv));
                                    CHECK(static_cast<int64_t>(p.fold_levels) * 2 * wgs <= gqa::kCounterWords,
                                          "counters %lld", static_cast<long long>(p.fold_levels * 2 * wgs));
                                    CHECK(p.merge_blocks == 0 && p.merge_threads == 0, "fused plan with a merge kernel");
                                    const double need = static_cast<double>(gqa::kCounterBytes) +
                                                        1.25 * p.num_chunks * 2 * R * (a.d_head + 2) * 4;
                                    CHECK(static_cast<double>(p.workspace_bytes) >= need && p.workspace_bytes % 256 == 0,
                                          "fused workspace %zu for %g", p.workspace_bytes, need);
                                    continue;
                                }
                                CHECK(p.num_chunks <= (1 << 24), "num_chunks %d above 2^24", p.num_chunks);
                                if (ch == 0)
                                    CHECK(p.num_chunks <= std::max<int64_t>(hkv, static_cast<int64_t>(nc) * std::min(wv, 4)),
                                          "automatic num_chunks %d above %d x min(%d, 4)", p.num_chunks, nc, wv);
                                CHECK(static_cast<int64_t>(p.split_blocks) * gqa::kWavesPerBlock >= p.num_chunks,
                                      "split blocks %d for %d wavefronts", p.split_blocks, p.num_chunks);
                                CHECK(p.merge_blocks > 0 && (p.merge_threads == 256 || p.merge_threads == 1024),
                                      "merge blocks %d threads %d", p.merge_blocks, p.merge_threads);
                                const double need = static_cast<double>(p.num_chunks) * 2 * R * (a.d_head + 2) * 4;
                                CHECK(static_cast<double>(p.workspace_bytes) >= need && p.workspace_bytes % 256 == 0,
                                      "workspace %zu for %g", p.workspace_bytes, need);
                                CHECK(p.min_chunk > 0, "min_chunk %d", p.min_chunk);
                            }
    CHECK(made > 1000 && fused > 100, "only %d plans (%d fused) were made", made, fused);
}

static void prefill_grid() {
    gqa_prefill_args a;
    std::memset(&a, 0, sizeof a);
    a.q = reinterpret_cast<const void *>(0x10000);
    a.k = reinterpret_cast<const void *>(0x20000);
    a.v = reinterpret_cast<const void *>(0x30000);
    a.o = reinterpret_cast<void *>(0x40000);
    a.seq_lens = reinterpret_cast<const int32_t *>(0x50000);
    a.batch = 2;
    a.h_q = 8;
    a.h_kv = 1;
    a.d_head = 128;
    a.scale = 0.088f;
    a.total_tokens = 32768;
    CHECK(gqa::validate_prefill(&a) == GQA_OK, "prefill base");
    const int64_t totals[] = {-1, 0, 1, 63, 64, 65, 1 << 20, int64_t(1) << 37, (int64_t(1) << 37) + 1, INT64_MAX};
    const int32_t hkvs[] = {1, 2, 8, 65536};
    const int32_t batches[] = {1, 2, 1 << 20, INT32_MAX};
    for (int64_t t : totals)
        for (int32_t hkv : hkvs)
            for (int32_t b : batches)
                for (int split = 0; split < 3; ++split) {
                    a.total_tokens = t;
                    a.h_kv = hkv;
                    a.h_q = hkv;
                    a.batch = b;
                    a.split_pv = split;
                    a.workspace = nullptr;
                    const int st = gqa::validate_prefill(&a);
                    if (split == 2) {
                        CHECK(st == GQA_ERR_ARG, "split_pv 2 accepted");
                        continue;
                    }
                    if (t < 0) CHECK(st == GQA_ERR_ARG, "negative total_tokens accepted");
                    if (st != GQA_OK) continue;
                    const gqa::PrefillWorkspace W = gqa::prefill_workspace(&a);
                    if (split == 1 || t == 0) {
                        CHECK(W.bytes == 0, "a call without a V copy needs %zu bytes", W.bytes);
                    } else {
                        CHECK(W.nvb >= (t + 63) / 64 + b && W.bytes > W.flags_offset, "nvb %lld bytes %zu",
                              static_cast<long long>(W.nvb), W.bytes);
                        a.workspace = reinterpret_cast<void *>(0x100000);
                        a.workspace_bytes = W.bytes - 1;
                        CHECK(gqa::validate_prefill(&a) == GQA_ERR_WORKSPACE, "short prefill workspace");
                        a.workspace_bytes = W.bytes;
                        CHECK(gqa::validate_prefill(&a) == GQA_OK, "exact prefill workspace");
                        a.workspace = reinterpret_cast<void *>(0x100080);
                        CHECK(gqa::validate_prefill(&a) == GQA_ERR_WORKSPACE, "misaligned prefill workspace");
                    }
                }
}

// Deterministic values in [-2, 2) for the oracle's inputs.
static float value(uint32_t i) {
    i ^= i >> 16;
    i *= 0x7feb352dU;
    i ^= i >> 15;
    i *= 0x846ca68bU;
    i ^= i >> 16;
    return static_cast<float>(i >> 8) / 4194304.0f - 2.0f;
}

static void oracle_edges() {
    const int32_t h_q = 4, h_kv = 2, d = 8;
    const int32_t G = h_q / h_kv;
    // Sequences: empty, negative (counts as empty), one key, three keys, six keys.
    const int32_t lens[] = {0, -7, 1, 3, 6};
    const int32_t batch = 5;
    int64_t rows = 0;
    for (int32_t L : lens) rows += L > 0 ? L : 0;
    for (int32_t t_q = 1; t_q <= 8; ++t_q) {
        std::vector<float> q(static_cast<size_t>(batch) * t_q * h_q * d), k(rows * h_kv * d), v(rows * h_kv * d);
        for (size_t i = 0; i < q.size(); ++i) q[i] = value(static_cast<uint32_t>(i) * 3 + 1);
        for (size_t i = 0; i < k.size(); ++i) k[i] = value(static_cast<uint32_t>(i) * 3 + 2);
        for (size_t i = 0; i < v.size(); ++i) v[i] = value(static_cast<uint32_t>(i) * 3 + 3);
        std::vector<double> out(q.size(), NAN);
        const int rc = oracle_gqa_decode_tq_f64(q.data(), k.data(), v.data(), lens, batch, t_q, h_q, h_kv, d, 0.35,
                                                GQA_DTYPE_F32, out.data());
        CHECK(rc == 0, "oracle rc %d at t_q %d", rc, t_q);
        for (int32_t b = 0; b < batch; ++b) {
            const int32_t S = lens[b] > 0 ? lens[b] : 0;
            for (int32_t t = 0; t < t_q; ++t) {
                const int32_t seen = std::min(S, std::max(0, S - t_q + t + 1));
                for (int32_t h = 0; h < h_q; ++h)
                    for (int32_t i = 0; i < d; ++i) {
                        const double x = out[((static_cast<size_t>(b) * t_q + t) * h_q + h) * d + i];
                        if (seen == 0)
                            CHECK(x == 0.0, "b %d t %d of t_q %d sees no key but gives %g", b, t, t_q, x);
                        else
                            CHECK(std::isfinite(x) && std::fabs(x) <= 2.0, "b %d t %d: %g", b, t, x);
                    }
            }
        }
    }
    // Partial triples over every range of every sequence, including empty ones.
    std::vector<float> q(static_cast<size_t>(batch) * h_q * d), k(rows * h_kv * d), v(rows * h_kv * d);
    for (size_t i = 0; i < q.size(); ++i) q[i] = value(static_cast<uint32_t>(i) + 7);
    for (size_t i = 0; i < k.size(); ++i) k[i] = value(static_cast<uint32_t>(i) + 99);
    for (size_t i = 0; i < v.size(); ++i) v[i] = value(static_cast<uint32_t>(i) + 1234);
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t S = lens[b] > 0 ? lens[b] : 0;
        for (int32_t h = 0; h < h_q; ++h) {
            std::vector<double> w(S > 0 ? S : 1);
            CHECK(oracle_softmax_weights_f64(q.data(), k.data(), lens, batch, h_q, h_kv, d, 0.35, GQA_DTYPE_F32, b,
                                             h, w.data()) == 0, "weights b %d h %d", b, h);
            for (int32_t t0 = 0; t0 <= S; ++t0)
                for (int32_t t1 = t0; t1 <= S; ++t1) {
                    double m = 0, l = -1, O[d];
                    CHECK(oracle_partial_f64(q.data(), k.data(), v.data(), lens, batch, h_q, h_kv, d, 0.35,
                                             GQA_DTYPE_F32, b, h, t0, t1, &m, &l, O) == 0, "partial");
                    if (t0 == t1) CHECK(m == -INFINITY && l == 0.0, "empty partial (%g, %g)", m, l);
                    else CHECK(std::isfinite(m) && l >= 1.0 && l <= (t1 - t0), "partial (%g, %g)", m, l);
                }
            double m, l, O[d];
            CHECK(oracle_partial_f64(q.data(), k.data(), v.data(), lens, batch, h_q, h_kv, d, 0.35, GQA_DTYPE_F32, b,
                                     h, 0, S + 1, &m, &l, O) == -1, "range past the sequence accepted");
            CHECK(oracle_partial_f64(q.data(), k.data(), v.data(), lens, batch, h_q, h_kv, d, 0.35, GQA_DTYPE_F32, b,
                                     h, -1, 0, &m, &l, O) == -1, "negative range accepted");
        }
    }
    (void)G;
    double m, l, O[d];
    CHECK(oracle_partial_f64(q.data(), k.data(), v.data(), lens, batch, h_q, h_kv, d, 0.35, GQA_DTYPE_F32, batch, 0, 0,
                             0, &m, &l, O) == -1, "sequence past the batch accepted");
    std::vector<double> out(8, 0.0);
    CHECK(oracle_gqa_decode_tq_f64(q.data(), k.data(), v.data(), lens, batch, 0, h_q, h_kv, d, 0.35, GQA_DTYPE_F32,
                                   out.data()) == -1, "t_q 0 accepted");
    CHECK(oracle_gqa_decode_tq_f64(q.data(), k.data(), v.data(), lens, batch, 1, 3, h_kv, d, 0.35, GQA_DTYPE_F32,
                                   out.data()) == -1, "h_q not a multiple of h_kv accepted");
    // batch 0: nothing to compute.
    CHECK(oracle_gqa_decode_tq_f64(q.data(), k.data(), v.data(), lens, 0, 1, h_q, h_kv, d, 0.35, GQA_DTYPE_F32,
                                   out.data()) == 0, "batch 0");
}

int main() {
    validation_grid();
    plan_grid();
    prefill_grid();
    oracle_edges();
    std::printf("host sanitize driver: %d checks, %d failed\n", g_checks, g_failures);
    return g_failures == 0 ? 0 : 1;
}
