/*
 * oracle.c -- plain fp64 CPU oracle for grouped-query-attention decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under gqa_split_kv_amd/) never links, loads or calls it, and it
 * shares no code, header or table with that path.
 *
 * What it computes (plain definition, no tiling, no online rescaling):
 *
 *   for each sequence b and query head h, with j = floor(h / G), G = h_q / h_kv,
 *   S = seq_lens[b] (negative counts as 0) and base = sum of the earlier lengths:
 *     s_t = scale * sum_i q[b,h,i] * k[base+t, j, i]          t < S
 *     m   = max_t s_t,  w_t = exp(s_t - m),  l = sum_t w_t
 *     o[b,h,:] = (sum_t w_t * v[base+t, j, :]) / l            (S = 0 gives o = 0)
 *
 * Source: kernbench2 page "_gqa_attention_decode_long.py" -- the "Tile 0" block
 * (scores = Q.K^T, row max, exp of the centred scores, row sum, exp.V) taken over
 * the whole key range as one tile, followed by the "Final normalise + store"
 * block (O / l).  Readings of that page used here:
 *   - scale multiplies the raw dot product before the softmax (the page's GEMMs
 *     carry no softmax_scale; scale = 1 reproduces the page);
 *   - the score uses the true transpose of K (the page's reshape of K is flagged
 *     there as correct only for zero or symmetric inputs);
 *   - query head h reads kv head floor(h/G) (consecutive grouping, G = h_q // h_kv
 *     as in the page's rank decomposition);
 *   - K and V are packed [sum(seq_lens), h_kv, d] (the page has no batch axis).
 *
 * Every input element is widened exactly to double (bf16 is read as its raw
 * 16 bits and shifted into a float; IEEE fp16 is decoded from its bits; float
 * widens exactly).  Sums run in index
 * order.  OpenMP spreads (sequence, kv head) pairs over the host cores; that
 * changes nothing in the arithmetic of any single output.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_F32 1
#define ORACLE_F16 2

/* IEEE binary16 bits -> double, exactly: (1024 + m) * 2^(e - 25) for a normal
 * number, m * 2^-24 for a subnormal, infinities and NaN kept. */
static double half_bits_to_double(uint16_t h) {
    const int sign = h >> 15;
    const int e = (h >> 10) & 0x1f;
    const int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);
    return sign ? -v : v;
}

static double widen(const void *base, int64_t idx, int dtype) {
    if (dtype == ORACLE_F32) return (double)((const float *)base)[idx];
    if (dtype == ORACLE_F16) return half_bits_to_double(((const uint16_t *)base)[idx]);
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* The widening the oracle applies to its inputs, exposed for testing. */
void oracle_widen_f64(const void *src, int64_t n, int32_t dtype, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = widen(src, i, dtype);
}

static int32_t clamp_len(int32_t n) { return n > 0 ? n : 0; }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Start row of sequence b in the packed K/V (sum of the earlier lengths). */
static int64_t seq_base(const int32_t *seq_lens, int32_t b) {
    int64_t base = 0;
    for (int32_t i = 0; i < b; ++i) base += clamp_len(seq_lens[i]);
    return base;
}

/* s_t for query row qrow (element offset into q) against kv head j over keys
 * [t0, t1) of the sequence starting at row `base`, into s[0 .. t1-t0). */
static void scores_row(const void *q, const void *k, int64_t qrow, int32_t j, int32_t h_kv,
                       int32_t d, double scale, int dtype, int64_t base, int32_t t0, int32_t t1,
                       double *s) {
    for (int32_t t = t0; t < t1; ++t) {
        const int64_t krow = ((base + t) * h_kv + j) * (int64_t)d;
        double dot = 0.0;
        for (int32_t i = 0; i < d; ++i) dot += widen(q, qrow + i, dtype) * widen(k, krow + i, dtype);
        s[t - t0] = scale * dot;
    }
}

/* s_t for one (b, h) of a single-query decode (q is [batch, h_q, d]). */
static void scores(const void *q, const void *k, int32_t h_q, int32_t h_kv, int32_t d,
                   double scale, int dtype, int32_t b, int32_t h, int64_t base, int32_t t0,
                   int32_t t1, double *s) {
    const int32_t G = h_q / h_kv;
    scores_row(q, k, ((int64_t)b * h_q + h) * d, h / G, h_kv, d, scale, dtype, base, t0, t1, s);
}

/*
 * Full decode with t_q query tokens per sequence: q and out are
 * [batch, t_q, h_q, d]; the last t_q key rows of a sequence of S keys belong to
 * the new tokens, and query token t sees keys 0 .. S - t_q + t (causal among the
 * new tokens): S_t = min(S, max(0, S - t_q + t + 1)) keys.  S_t = 0 gives 0.
 * t_q = 1 is the single-token decode of the page.  Returns 0, or -1 on bad shape.
 */
int oracle_gqa_decode_tq_f64(const void *q, const void *k, const void *v, const int32_t *seq_lens,
                             int32_t batch, int32_t t_q, int32_t h_q, int32_t h_kv, int32_t d,
                             double scale, int32_t dtype, double *out) {
    if (batch < 0 || t_q <= 0 || h_q <= 0 || h_kv <= 0 || d <= 0 || h_q % h_kv != 0) return -1;
    const int32_t G = h_q / h_kv;
    int64_t *bases = (int64_t *)malloc(sizeof(int64_t) * (size_t)(batch > 0 ? batch : 1));
    int32_t max_len = 0;
    for (int32_t b = 0; b < batch; ++b) {
        bases[b] = seq_base(seq_lens, b);
        if (clamp_len(seq_lens[b]) > max_len) max_len = clamp_len(seq_lens[b]);
    }
    const int64_t units = (int64_t)batch * h_kv;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !acc) failed = 1;
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!s || !acc) continue;
            const int32_t b = (int32_t)(u / h_kv);
            const int32_t j = (int32_t)(u % h_kv);
            const int32_t S = clamp_len(seq_lens[b]);
            for (int32_t t = 0; t < t_q; ++t) {
                int32_t St = S - t_q + t + 1;
                if (St < 0) St = 0;
                if (St > S) St = S;
                for (int32_t g = 0; g < G; ++g) {
                    const int32_t h = j * G + g;
                    const int64_t row = ((int64_t)b * t_q + t) * h_q + h;
                    double *o = out + row * d;
                    if (St == 0) {
                        for (int32_t i = 0; i < d; ++i) o[i] = 0.0;
                        continue;
                    }
                    /* pass 1: scores and their maximum */
                    scores_row(q, k, row * d, j, h_kv, d, scale, dtype, bases[b], 0, St, s);
                    double m = -INFINITY;
                    for (int32_t x = 0; x < St; ++x)
                        if (s[x] > m) m = s[x];
                    /* pass 2: weights, their sum, and the weighted sum of V rows */
                    double l = 0.0;
                    for (int32_t i = 0; i < d; ++i) acc[i] = 0.0;
                    for (int32_t x = 0; x < St; ++x) {
                        const double w = exp(s[x] - m);
                        l += w;
                        const int64_t vrow = ((bases[b] + x) * h_kv + j) * (int64_t)d;
                        for (int32_t i = 0; i < d; ++i) acc[i] += w * widen(v, vrow + i, dtype);
                    }
                    for (int32_t i = 0; i < d; ++i) o[i] = acc[i] / l;
                }
            }
        }
        free(s);
        free(acc);
    }
    free(bases);
    return failed ? -2 : 0;
}

/* Single-token decode: out is double[batch, h_q, d]. */
int oracle_gqa_decode_f64(const void *q, const void *k, const void *v, const int32_t *seq_lens,
                          int32_t batch, int32_t h_q, int32_t h_kv, int32_t d, double scale,
                          int32_t dtype, double *out) {
    return oracle_gqa_decode_tq_f64(q, k, v, seq_lens, batch, 1, h_q, h_kv, d, scale, dtype, out);
}

/*
 * Softmax weights w_t / l of one (b, h): w is double[seq_lens[b]].
 * Same definition as above; exposed so tests can check the weights themselves.
 */
int oracle_softmax_weights_f64(const void *q, const void *k, const int32_t *seq_lens,
                               int32_t batch, int32_t h_q, int32_t h_kv, int32_t d,
                               double scale, int32_t dtype, int32_t b, int32_t h, double *w) {
    if (b < 0 || b >= batch || h < 0 || h >= h_q || h_q % h_kv != 0) return -1;
    const int32_t S = clamp_len(seq_lens[b]);
    if (S == 0) return 0;
    scores(q, k, h_q, h_kv, d, scale, dtype, b, h, seq_base(seq_lens, b), 0, S, w);
    double m = -INFINITY;
    for (int32_t t = 0; t < S; ++t)
        if (w[t] > m) m = w[t];
    double l = 0.0;
    for (int32_t t = 0; t < S; ++t) {
        w[t] = exp(w[t] - m);
        l += w[t];
    }
    for (int32_t t = 0; t < S; ++t) w[t] /= l;
    return 0;
}

/*
 * The partial triple of one (b, h) over keys [t0, t1), natural-exp domain:
 *   m = max s_t,  l = sum exp(s_t - m),  O = sum exp(s_t - m) v_t  (not divided by l).
 * This is the page's per-tile (m, l, O) ("Tile 0" block) for an arbitrary key
 * range.  An empty range returns the identity (-inf, 0, 0).
 * Outputs: m[1], l[1], O[d].
 */
int oracle_partial_f64(const void *q, const void *k, const void *v, const int32_t *seq_lens,
                       int32_t batch, int32_t h_q, int32_t h_kv, int32_t d, double scale,
                       int32_t dtype, int32_t b, int32_t h, int32_t t0, int32_t t1, double *m_out,
                       double *l_out, double *O) {
    if (b < 0 || b >= batch || h < 0 || h >= h_q || h_q % h_kv != 0) return -1;
    const int32_t S = clamp_len(seq_lens[b]);
    if (t0 < 0 || t1 > S || t0 > t1) return -1;
    for (int32_t i = 0; i < d; ++i) O[i] = 0.0;
    if (t0 == t1) {
        *m_out = -INFINITY;
        *l_out = 0.0;
        return 0;
    }
    const int32_t G = h_q / h_kv;
    const int32_t j = h / G;
    const int64_t base = seq_base(seq_lens, b);
    double *s = (double *)malloc(sizeof(double) * (size_t)(t1 - t0));
    if (!s) return -2;
    scores(q, k, h_q, h_kv, d, scale, dtype, b, h, base, t0, t1, s);
    double m = -INFINITY;
    for (int32_t t = 0; t < t1 - t0; ++t)
        if (s[t] > m) m = s[t];
    double l = 0.0;
    for (int32_t t = t0; t < t1; ++t) {
        const double w = exp(s[t - t0] - m);
        l += w;
        const int64_t vrow = ((base + t) * h_kv + j) * (int64_t)d;
        for (int32_t i = 0; i < d; ++i) O[i] += w * widen(v, vrow + i, dtype);
    }
    free(s);
    *m_out = m;
    *l_out = l;
    return 0;
}
