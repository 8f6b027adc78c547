/*
 * CPU fp64 oracle for single-token GQA flash-decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the package smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes (sparkinfer PR #874, "Why it is bit-identical": an online
 * softmax over the keys of one kv head; sparkinfer PR #877, "Mechanism": the
 * (m, l, acc) partials folded by the log-sum-exp rescale; AstrAI csrc commit
 * log, the split-KV bullets: unnormalised (O, m, l) partials reduced by a
 * combine step), written as its plain definition:
 *
 *     G   = Hq / Hkv,  kvh = h / G                  (query heads grouped
 *                                                    consecutively per kv head)
 *     s_t = scale * sum_d q[b,h,d] * K[b,kvh,t,d]    for t < seq_lens[b]
 *     out[b,h,:] = sum_t softmax(s)_t * V[b,kvh,t,:]
 *
 * Inputs are bf16 bit patterns, widened exactly to double; scale arrives as
 * a float and is widened exactly.  All arithmetic is IEEE double in a fixed,
 * documented order (d ascending, t ascending).  The softmax is the exact
 * two-pass form (max, then exp(s - max) and the sums): the method's online
 * rescale reaches the same value up to rounding, so the oracle does not copy
 * it.  A sequence of length 0 yields a zero output row.
 *
 * The split entry points compute fp64 partials over consecutive token chunks
 * [i*chunk, min((i+1)*chunk, n)) and fold them with the log-sum-exp rescale
 * in ascending chunk order.  They exist only so the tests can pin the split
 * algebra (invariance to the split count) against the plain definition.
 *
 * Quantized cache (the int8/fp8 pools of sparkinfer PR #874, "Cost and
 * fallbacks", dequantised before use; the pages fix no format, the reading
 * taken here is the plainest one): K and V hold OCP FP8 E4M3 bytes, one
 * fp32 scale per tensor, and the value of an element is its scale times the
 * E4M3 value of the byte (sign bit, 4-bit exponent with bias 7, 3-bit
 * mantissa; exponent 0 is subnormal, m/8 * 2^-6; byte 0x7F / 0xFF is NaN).
 *
 * Multi-query decode (speculative verification of M drafted tokens, the
 * block of the sparkinfer PR #874 speculative-decode report, section
 * "ok"; causal masking as in the prefill kernel of the AstrAI csrc commit
 * log): each sequence carries M query tokens, the last M positions of the
 * sequence, whose keys and values are already in the cache.  Query i
 * (0-based) attends to the keys 0 .. len - M + i, so row (b, i, h) is the
 * single-query definition over the first n_i = len - M + i + 1 keys (a row
 * with n_i <= 0 is zero).  q and out are [B][M][Hq][D].
 *
 * Cache layouts (the pages fix only the index order K[b, h/G, t]):
 *   contiguous: K, V are [B][Hkv][S_max][D]
 *   paged:      K, V pools are [num_pages][Hkv][page_size][D]; token t of
 *               sequence b lives in page page_table[b*max_pages + t/page_size]
 *               at row t % page_size (AstrAI csrc/tests commit log, the paged
 *               decode bullets: one page-table entry covers page_size tokens).
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -shared -fPIC
 * (no fast-math, no intrinsics).  OpenMP only distributes independent
 * (b, h) rows; it does not change any row's arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    const void *k, *v;
    const int32_t *page_table; /* NULL for the contiguous layout */
    int Hkv, D;
    int S_max;                 /* contiguous capacity per (b, kv head) */
    int page_size, max_pages;  /* paged only */
    int fp8;                   /* 0: bf16 bit patterns; 1: E4M3 bytes times k_scale / v_scale */
    double k_scale, v_scale;
} kv_layout;

/* bf16 -> double: the bf16 pattern is the upper half of an IEEE float. */
static double widen_bf16(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 byte -> double, from the format's definition. */
static double decode_e4m3(uint8_t byte) {
    const double sign = (byte & 0x80) ? -1.0 : 1.0;
    const int e = (byte >> 3) & 0xF, m = byte & 7;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) return sign * ldexp((double)m / 8.0, -6);
    return sign * ldexp(1.0 + (double)m / 8.0, e - 7);
}

/* Element i of the K / V storage, dequantised. */
static double k_elem(const kv_layout *L, size_t i) {
    if (L->fp8) return L->k_scale * decode_e4m3(((const uint8_t *)L->k)[i]);
    return widen_bf16(((const uint16_t *)L->k)[i]);
}
static double v_elem(const kv_layout *L, size_t i) {
    if (L->fp8) return L->v_scale * decode_e4m3(((const uint8_t *)L->v)[i]);
    return widen_bf16(((const uint16_t *)L->v)[i]);
}

/* Element offset of row (b, kvh, t) in the K or V storage. */
static size_t row_offset(const kv_layout *L, int b, int kvh, int t) {
    if (L->page_table == NULL)
        return (((size_t)b * L->Hkv + kvh) * (size_t)L->S_max + (size_t)t) * (size_t)L->D;
    int page = L->page_table[(size_t)b * L->max_pages + (size_t)(t / L->page_size)];
    return (((size_t)page * L->Hkv + kvh) * (size_t)L->page_size + (size_t)(t % L->page_size)) *
           (size_t)L->D;
}

/* score of token t for the query row q (D bf16 values) */
static double score(const kv_layout *L, const uint16_t *q, int b, int kvh, int t, double scale) {
    const size_t kbase = row_offset(L, b, kvh, t);
    double dot = 0.0;
    for (int d = 0; d < L->D; ++d) dot += widen_bf16(q[d]) * k_elem(L, kbase + d);
    return scale * dot;
}

/*
 * Softmax statistics of one query row over tokens [t0, t1):
 *   m = max_t s_t,  l = sum_t exp(s_t - m),  acc[d] = sum_t exp(s_t - m) V[t][d].
 * An empty range gives m = -inf, l = 0, acc = 0.  `s` is scratch of length
 * at least t1 - t0.
 */
static void range_stats(const kv_layout *L, const uint16_t *q, int b, int kvh, int t0, int t1,
                        double scale, double *s, double *m_out, double *l_out, double *acc) {
    const int D = L->D;
    for (int d = 0; d < D; ++d) acc[d] = 0.0;
    double m = -INFINITY, l = 0.0;
    for (int t = t0; t < t1; ++t) {
        s[t - t0] = score(L, q, b, kvh, t, scale);
        if (s[t - t0] > m) m = s[t - t0];
    }
    for (int t = t0; t < t1; ++t) {
        double w = exp(s[t - t0] - m);
        const size_t vbase = row_offset(L, b, kvh, t);
        l += w;
        for (int d = 0; d < D; ++d) acc[d] += w * v_elem(L, vbase + d);
    }
    *m_out = m;
    *l_out = l;
}

/*
 * out[b,h,:] for every (b, h).  chunk <= 0: one pass over the whole
 * sequence.  chunk > 0: consecutive chunks folded by the log-sum-exp rescale
 *     M = max_i m_i,  w_i = exp(m_i - M) (0 for an empty chunk),
 *     out = (sum_i w_i acc_i) / (sum_i w_i l_i),   i ascending.
 */
static int decode_all(const kv_layout *L, const uint16_t *q, const int32_t *seq_lens, int B,
                      int M, int Hq, double scale, int chunk, double *out) {
    const int Hkv = L->Hkv, D = L->D;
    if (B < 0 || M <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return 1;
    const int G = Hq / Hkv;
    int maxlen = 0;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < 0) return 2;
        if (seq_lens[b] > maxlen) maxlen = seq_lens[b];
    }
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        double *sum = (double *)malloc(sizeof(double) * (size_t)D);
        if (s == NULL || acc == NULL || sum == NULL) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long long row = 0; row < (long long)B * M * Hq; ++row) {
                const int b = (int)(row / ((long long)M * Hq));
                const int i = (int)(row / Hq % M), h = (int)(row % Hq);
                const int kvh = h / G;
                const int n = seq_lens[b] - M + i + 1;     /* keys this query row attends to */
                const uint16_t *qrow = q + (((size_t)b * M + i) * Hq + h) * (size_t)D;
                double *o = out + (((size_t)b * M + i) * Hq + h) * (size_t)D;
                if (n <= 0) {
                    for (int d = 0; d < D; ++d) o[d] = 0.0;
                    continue;
                }
                if (chunk <= 0) {
                    double m, l;
                    range_stats(L, qrow, b, kvh, 0, n, scale, s, &m, &l, acc);
                    for (int d = 0; d < D; ++d) o[d] = acc[d] / l;
                    continue;
                }
                const int nchunks = (n + chunk - 1) / chunk;
                double M = -INFINITY;
                for (int i = 0; i < nchunks; ++i) { /* pass 1: the global max of the chunk maxima */
                    int t0 = i * chunk, t1 = t0 + chunk < n ? t0 + chunk : n;
                    double m, l;
                    range_stats(L, qrow, b, kvh, t0, t1, scale, s, &m, &l, acc);
                    if (m > M) M = m;
                }
                double Lsum = 0.0;
                for (int d = 0; d < D; ++d) sum[d] = 0.0;
                for (int i = 0; i < nchunks; ++i) { /* pass 2: rescale and fold, i ascending */
                    int t0 = i * chunk, t1 = t0 + chunk < n ? t0 + chunk : n;
                    double m, l;
                    range_stats(L, qrow, b, kvh, t0, t1, scale, s, &m, &l, acc);
                    double w = (m == -INFINITY) ? 0.0 : exp(m - M);
                    Lsum += w * l;
                    for (int d = 0; d < D; ++d) sum[d] += w * acc[d];
                }
                for (int d = 0; d < D; ++d) o[d] = sum[d] / Lsum;
            }
        }
        free(s);
        free(acc);
        free(sum);
    }
    return failed ? 3 : 0;
}

/* ---- exported entry points (ctypes) ---- */

int oracle_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *seq_lens,
                  int B, int Hq, int Hkv, int D, int S_max, float scale, double *out) {
    kv_layout L = {k, v, NULL, Hkv, D, S_max, 0, 0, 0, 1.0, 1.0};
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] > S_max) return 2;
    return decode_all(&L, q, seq_lens, B, 1, Hq, (double)scale, 0, out);
}

int oracle_decode_split(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int S_max,
                        float scale, int chunk, double *out) {
    kv_layout L = {k, v, NULL, Hkv, D, S_max, 0, 0, 0, 1.0, 1.0};
    if (chunk <= 0) return 1;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] > S_max) return 2;
    return decode_all(&L, q, seq_lens, B, 1, Hq, (double)scale, chunk, out);
}

int oracle_paged_decode(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                        const int32_t *seq_lens, const int32_t *page_table, int B, int Hq, int Hkv,
                        int D, int page_size, int num_pages, int max_pages, float scale,
                        double *out) {
    kv_layout L = {k_pool, v_pool, page_table, Hkv, D, 0, page_size, max_pages, 0, 1.0, 1.0};
    if (page_size <= 0 || max_pages < 0) return 1;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] > page_size * max_pages) return 2;
        int used = (seq_lens[b] + page_size - 1) / page_size;
        for (int i = 0; i < used; ++i) {
            int p = page_table[(size_t)b * max_pages + i];
            if (p < 0 || p >= num_pages) return 2;
        }
    }
    return decode_all(&L, q, seq_lens, B, 1, Hq, (double)scale, 0, out);
}

int oracle_paged_decode_split(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                              const int32_t *seq_lens, const int32_t *page_table, int B, int Hq,
                              int Hkv, int D, int page_size, int num_pages, int max_pages,
                              float scale, int chunk, double *out) {
    kv_layout L = {k_pool, v_pool, page_table, Hkv, D, 0, page_size, max_pages, 0, 1.0, 1.0};
    if (page_size <= 0 || max_pages < 0 || chunk <= 0) return 1;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] > page_size * max_pages) return 2;
        int used = (seq_lens[b] + page_size - 1) / page_size;
        for (int i = 0; i < used; ++i) {
            int p = page_table[(size_t)b * max_pages + i];
            if (p < 0 || p >= num_pages) return 2;
        }
    }
    return decode_all(&L, q, seq_lens, B, 1, Hq, (double)scale, chunk, out);
}

/* The same over an E4M3 cache with per-tensor scales (chunk > 0: split mode). */
int oracle_decode_fp8(const uint16_t *q, const uint8_t *k, const uint8_t *v, const int32_t *seq_lens,
                      int B, int Hq, int Hkv, int D, int S_max, float scale, float k_scale,
                      float v_scale, int chunk, double *out) {
    kv_layout L = {k, v, NULL, Hkv, D, S_max, 0, 0, 1, (double)k_scale, (double)v_scale};
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] > S_max) return 2;
    return decode_all(&L, q, seq_lens, B, 1, Hq, (double)scale, chunk, out);
}

int oracle_paged_decode_fp8(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                            const int32_t *seq_lens, const int32_t *page_table, int B, int Hq,
                            int Hkv, int D, int page_size, int num_pages, int max_pages,
                            float scale, float k_scale, float v_scale, int chunk, double *out) {
    kv_layout L = {k_pool, v_pool, page_table, Hkv, D, 0, page_size, max_pages, 1, (double)k_scale,
                   (double)v_scale};
    if (page_size <= 0 || max_pages < 0) return 1;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] > page_size * max_pages) return 2;
        int used = (seq_lens[b] + page_size - 1) / page_size;
        for (int i = 0; i < used; ++i) {
            int p = page_table[(size_t)b * max_pages + i];
            if (p < 0 || p >= num_pages) return 2;
        }
    }
    return decode_all(&L, q, seq_lens, B, 1, Hq, (double)scale, chunk, out);
}

/* Multi-query decode over a bf16 cache: q and out are [B][M][Hq][D]. */
int oracle_decode_mq(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const int32_t *seq_lens, int B, int M, int Hq, int Hkv, int D, int S_max,
                     float scale, int chunk, double *out) {
    kv_layout L = {k, v, NULL, Hkv, D, S_max, 0, 0, 0, 1.0, 1.0};
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] > S_max) return 2;
    return decode_all(&L, q, seq_lens, B, M, Hq, (double)scale, chunk, out);
}

int oracle_paged_decode_mq(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                           const int32_t *seq_lens, const int32_t *page_table, int B, int M, int Hq,
                           int Hkv, int D, int page_size, int num_pages, int max_pages, float scale,
                           int chunk, double *out) {
    kv_layout L = {k_pool, v_pool, page_table, Hkv, D, 0, page_size, max_pages, 0, 1.0, 1.0};
    if (page_size <= 0 || max_pages < 0) return 1;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] > page_size * max_pages) return 2;
        int used = (seq_lens[b] + page_size - 1) / page_size;
        for (int i = 0; i < used; ++i) {
            int p = page_table[(size_t)b * max_pages + i];
            if (p < 0 || p >= num_pages) return 2;
        }
    }
    return decode_all(&L, q, seq_lens, B, M, Hq, (double)scale, chunk, out);
}

/* Threads the OpenMP runtime will use for the next call (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
