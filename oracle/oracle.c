/*
 * Oracle for fused grouped-query attention: the plain fp64 CPU definition.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's
 * CPU-baseline leg call it; the HIP library never links, loads or calls it,
 * and it shares no source with the HIP library.
 *
 * What it computes (the definition, not the fast method):
 *
 *  - Decode (glia honeycrisp "attention.rs" page: module doc comment, and
 *    the Params struct and window_start of its flash-decode kernel): for
 *    every head h of the single query, each cached position s gets the score
 *    scale * <q[h], K[h / repeat][s]>, the scores go through a softmax, and
 *    the output row of head h is the softmax-weighted sum of the V rows of
 *    KV head h / repeat, with repeat = num_heads / kv_heads. The optional
 *    sliding window keeps only positions s >= total_seq - window (window = 0,
 *    or window >= total_seq, keeps all). Positions outside the window are
 *    left out of the sum entirely; the page's kernel instead gives them the
 *    score -1e4, whose weight is exactly zero in fp32 and fp64 whenever some
 *    attended score exceeds -1e4 + 104, so the two readings agree on every
 *    input used here.
 *
 *  - Causal prefill (aprender-gpu "prefill_fused.rs" page: module doc
 *    "Algorithm" steps 1-3 and the kernel parameter list): Q[M, q_stride],
 *    K/V[M, kv_stride], O[M, q_stride] fp32 row-major; Q head h lives at
 *    columns [h*d, (h+1)*d) and reads KV head h / heads_per_kv (integer
 *    division), whose columns are [g*d, (g+1)*d) of K and V. Query row i
 *    attends key rows j = 0..i (diagonal included). The scale is fixed at
 *    1/sqrt(head_dim) evaluated in f32, as the page's kernel builder does.
 *
 *  - KV append (glia honeycrisp "attention.rs" page, KV-append and
 *    KV-append-both kernels):
 *    cache[b, g, position, :] = src[b, g, :] for K and V, nothing else written.
 *
 *  - Rotary embedding and the fused decode step (glia honeycrisp
 *    "attention.rs" page, fused RoPE + KV-append + decode kernel and its doc):
 *    rotate-half pairs element i with element i + d/2 (i < d/2) and turns
 *    each pair by the angle whose cosine and sine are cos[i], sin[i]:
 *    y[i] = x[i] cos[i] - x[i+d/2] sin[i], y[i+d/2] = x[i] sin[i] + x[i+d/2] cos[i].
 *    The step rotates the current token's q (every head) and new K row
 *    (every KV head), writes the rotated K row and the raw V row into the
 *    caches at `position`, then decodes with total_seq = position + 1.
 *
 * Each softmax is materialised and taken in two passes over the stored
 * scores of one query row: first the maximum, then the exponentials and
 * their sum; the output is the sum of V rows weighted by e_j / Z. All
 * arithmetic is fp64 on the fp32 inputs widened to double, summed in index
 * order. OpenMP only spreads independent (row, head) outputs over threads;
 * it never splits or reorders a sum.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

int oracle_num_threads(void) { return omp_get_max_threads(); }

/* The prefill scale, 1/sqrt(head_dim) in f32 ("prefill_fused.rs" page,
 * the scale constant of build_ptx). */
float oracle_prefill_scale(uint32_t head_dim)
{
    return 1.0f / sqrtf((float)head_dim);
}

/*
 * Softmax attention of one query vector over n key/value rows.
 * q: d floats; key row j at k0 + j*row_stride, value row j at v0 + j*row_stride.
 * scores: scratch of n doubles. out: d doubles.
 */
static void attend(const float *q, const float *k0, const float *v0,
                   size_t row_stride, size_t n, uint32_t d, double scale,
                   double *scores, double *out)
{
    size_t j;
    uint32_t e;

    /* every score, materialised */
    for (j = 0; j < n; ++j) {
        const float *kj = k0 + j * row_stride;
        double dot = 0.0;
        for (e = 0; e < d; ++e)
            dot += (double)q[e] * (double)kj[e];
        scores[j] = scale * dot;
    }

    /* pass 1: the maximum score */
    double mu = -INFINITY;
    for (j = 0; j < n; ++j)
        if (scores[j] > mu)
            mu = scores[j];

    /* pass 2: exponentials (stored over the scores) and their sum */
    double z = 0.0;
    for (j = 0; j < n; ++j) {
        scores[j] = exp(scores[j] - mu);
        z += scores[j];
    }

    /* output: V rows weighted by the softmax probabilities e_j / Z */
    for (e = 0; e < d; ++e)
        out[e] = 0.0;
    for (j = 0; j < n; ++j) {
        const float *vj = v0 + j * row_stride;
        double w = scores[j] / z;
        for (e = 0; e < d; ++e)
            out[e] += w * (double)vj[e];
    }
}

/*
 * Causal prefill for n_sel selected (row, head) pairs, or for every pair
 * (row-major over rows, then heads) when rows == NULL.
 * out: [n_sel, head_dim] doubles (or [m, num_q_heads, head_dim]).
 * Returns 0, or -1 on an argument it cannot evaluate.
 */
int oracle_prefill_causal(const float *q, const float *k, const float *v,
                          uint32_t m, uint32_t q_stride, uint32_t kv_stride,
                          uint32_t num_q_heads, uint32_t heads_per_kv,
                          uint32_t head_dim, size_t n_sel,
                          const uint32_t *rows, const uint32_t *heads,
                          double *out)
{
    if (heads_per_kv == 0 || head_dim == 0 || num_q_heads % heads_per_kv)
        return -1;
    size_t total = rows ? n_sel : (size_t)m * num_q_heads;
    double scale = (double)oracle_prefill_scale(head_dim);
    int bad = 0;

#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (m ? m : 1));
        if (!scores) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (size_t t = 0; t < total; ++t) {
            if (!scores)
                continue;
            uint32_t i = rows ? rows[t] : (uint32_t)(t / num_q_heads);
            uint32_t h = rows ? heads[t] : (uint32_t)(t % num_q_heads);
            if (i >= m || h >= num_q_heads) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            uint32_t g = h / heads_per_kv; /* GQA: consecutive Q heads share g */
            const float *qi = q + (size_t)i * q_stride + (size_t)h * head_dim;
            const float *k0 = k + (size_t)g * head_dim;
            const float *v0 = v + (size_t)g * head_dim;
            /* causal: keys j = 0..i */
            attend(qi, k0, v0, kv_stride, (size_t)i + 1, head_dim, scale,
                   scores, out + t * head_dim);
        }
        free(scores);
    }
    return bad ? -1 : 0;
}

/*
 * Single-query decode for n_sel selected (sequence, head) pairs, or for all
 * of them (row-major over sequences, then heads) when bs == NULL.
 * q: [batch, num_heads, head_dim]; caches: [batch, kv_heads, max_seq, head_dim].
 * out: [n_sel, head_dim] doubles (or [batch, num_heads, head_dim]).
 */
int oracle_decode(const float *q, const float *k_cache, const float *v_cache,
                  uint32_t batch, uint32_t num_heads, uint32_t kv_heads,
                  uint32_t head_dim, uint32_t max_seq, uint32_t total_seq,
                  uint32_t window, float scale, size_t n_sel,
                  const uint32_t *bs, const uint32_t *hs, double *out)
{
    if (kv_heads == 0 || head_dim == 0 || num_heads % kv_heads ||
        total_seq == 0 || total_seq > max_seq)
        return -1;
    uint32_t repeat = num_heads / kv_heads;
    uint32_t window_start =
        (window > 0 && total_seq > window) ? total_seq - window : 0;
    size_t n = (size_t)(total_seq - window_start);
    size_t total = bs ? n_sel : (size_t)batch * num_heads;
    int bad = 0;

#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * n);
        if (!scores) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (size_t t = 0; t < total; ++t) {
            if (!scores)
                continue;
            uint32_t b = bs ? bs[t] : (uint32_t)(t / num_heads);
            uint32_t h = bs ? hs[t] : (uint32_t)(t % num_heads);
            if (b >= batch || h >= num_heads) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            uint32_t g = h / repeat;
            const float *qh = q + ((size_t)b * num_heads + h) * head_dim;
            size_t base = (((size_t)b * kv_heads + g) * max_seq + window_start)
                          * head_dim;
            attend(qh, k_cache + base, v_cache + base, head_dim, n, head_dim,
                   (double)scale, scores, out + t * head_dim);
        }
        free(scores);
    }
    return bad ? -1 : 0;
}

/* KV append: cache[b, g, position, :] = src[b, g, :] for K and for V. */
int oracle_kv_append(const float *k_src, const float *v_src, float *k_cache,
                     float *v_cache, uint32_t batch, uint32_t kv_heads,
                     uint32_t head_dim, uint32_t max_seq, uint32_t position)
{
    if (position >= max_seq)
        return -1;
    for (uint32_t b = 0; b < batch; ++b)
        for (uint32_t g = 0; g < kv_heads; ++g) {
            size_t src = ((size_t)b * kv_heads + g) * head_dim;
            size_t dst = (((size_t)b * kv_heads + g) * max_seq + position)
                         * head_dim;
            for (uint32_t e = 0; e < head_dim; ++e) {
                k_cache[dst + e] = k_src[src + e];
                v_cache[dst + e] = v_src[src + e];
            }
        }
    return 0;
}

/*
 * Bulk append of the K and V rows of a prefill pass into the caches (the
 * page's KV-append kernels, taken over M rows of the prefill's packed K/V
 * layout): for j < m and every KV head g,
 *   cache[g, position + j, :] = src[j * kv_stride + g * head_dim + (0..d-1)].
 * src: [m, kv_stride]; caches: [kv_heads, max_seq, head_dim] (one sequence).
 */
int oracle_kv_append_rows(const float *k_src, const float *v_src, float *k_cache,
                          float *v_cache, uint32_t m, uint32_t kv_stride,
                          uint32_t kv_heads, uint32_t head_dim, uint32_t max_seq,
                          uint32_t position)
{
    if ((uint64_t)position + m > max_seq ||
        (uint64_t)kv_stride < (uint64_t)kv_heads * head_dim)
        return -1;
    for (uint32_t j = 0; j < m; ++j)
        for (uint32_t g = 0; g < kv_heads; ++g) {
            size_t src = (size_t)j * kv_stride + (size_t)g * head_dim;
            size_t dst = ((size_t)g * max_seq + position + j) * head_dim;
            for (uint32_t e = 0; e < head_dim; ++e) {
                k_cache[dst + e] = k_src[src + e];
                v_cache[dst + e] = v_src[src + e];
            }
        }
    return 0;
}

/*
 * Decode of a batch whose sequences have their own lengths: sequence b
 * attends its rows [w0_b, seq_lens[b]) with w0_b from the page's window rule
 * applied to seq_lens[b]. A sequence of length 0 attends nothing and its
 * outputs are 0 (an idle batch slot). Lengths above max_seq are rejected.
 * Shapes as oracle_decode; out: [batch, num_heads, head_dim] doubles.
 */
int oracle_decode_varlen(const float *q, const float *k_cache, const float *v_cache,
                         const uint32_t *seq_lens, uint32_t batch,
                         uint32_t num_heads, uint32_t kv_heads, uint32_t head_dim,
                         uint32_t max_seq, uint32_t window, float scale,
                         double *out)
{
    if (kv_heads == 0 || head_dim == 0 || num_heads % kv_heads)
        return -1;
    for (uint32_t b = 0; b < batch; ++b)
        if (seq_lens[b] > max_seq)
            return -1;
    uint32_t repeat = num_heads / kv_heads;
    size_t total = (size_t)batch * num_heads;
    int bad = 0;

#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (max_seq ? max_seq : 1));
        if (!scores) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (size_t t = 0; t < total; ++t) {
            if (!scores)
                continue;
            uint32_t b = (uint32_t)(t / num_heads);
            uint32_t h = (uint32_t)(t % num_heads);
            uint32_t len = seq_lens[b];
            double *o = out + t * head_dim;
            if (len == 0) {
                for (uint32_t e = 0; e < head_dim; ++e)
                    o[e] = 0.0;
                continue;
            }
            uint32_t w0 = (window > 0 && len > window) ? len - window : 0;
            uint32_t g = h / repeat;
            const float *qh = q + ((size_t)b * num_heads + h) * head_dim;
            size_t base = (((size_t)b * kv_heads + g) * max_seq + w0) * head_dim;
            attend(qh, k_cache + base, v_cache + base, head_dim, (size_t)(len - w0),
                   head_dim, (double)scale, scores, o);
        }
        free(scores);
    }
    return bad ? -1 : 0;
}

/* Rotate-half rotary embedding of one vector of d elements (d even), in fp64
 * on the fp32 input; out may not alias x. */
static void rope(const float *x, const float *cs, const float *sn, uint32_t d,
                 double *out)
{
    uint32_t half = d / 2;
    for (uint32_t i = 0; i < half; ++i) {
        double a = x[i], b = x[i + half], c = cs[i], s = sn[i];
        out[i] = a * c - b * s;
        out[i + half] = a * s + b * c;
    }
}

/* Rotary embedding of n vectors of d elements: x [n, d] -> out [n, d] fp64. */
int oracle_rope(const float *x, const float *cos_t, const float *sin_t,
                size_t n, uint32_t d, double *out)
{
    if (d == 0 || d % 2)
        return -1;
    for (size_t r = 0; r < n; ++r)
        rope(x + r * d, cos_t, sin_t, d, out + r * d);
    return 0;
}

/*
 * One fused decode step with rotary embedding: rotate q (all heads) and the
 * new K rows, write rotated K and raw V at `position`, decode over
 * [w0, position]. The caches are updated in place with the rotated K rows
 * rounded to fp32 (what a cache of fp32 holds); the scores of the new row use
 * the fp64 rotation of q and k. out: [batch, num_heads, head_dim] doubles.
 */
int oracle_decode_rope_append(const float *q_raw, const float *k_raw,
                              const float *v_raw, const float *cos_t,
                              const float *sin_t, float *k_cache,
                              float *v_cache, uint32_t batch,
                              uint32_t num_heads, uint32_t kv_heads,
                              uint32_t head_dim, uint32_t max_seq,
                              uint32_t position, uint32_t window, float scale,
                              double *out)
{
    if (kv_heads == 0 || head_dim == 0 || head_dim % 2 ||
        num_heads % kv_heads || position >= max_seq)
        return -1;
    uint32_t repeat = num_heads / kv_heads;
    uint32_t total_seq = position + 1;
    uint32_t window_start =
        (window > 0 && total_seq > window) ? total_seq - window : 0;
    size_t n = (size_t)(total_seq - window_start);
    size_t d = head_dim;
    double *qr = (double *)malloc(sizeof(double) * d * num_heads * batch);
    double *kr = (double *)malloc(sizeof(double) * d * kv_heads * batch);
    if (!qr || !kr) {
        free(qr);
        free(kr);
        return -1;
    }
    oracle_rope(q_raw, cos_t, sin_t, (size_t)batch * num_heads, head_dim, qr);
    oracle_rope(k_raw, cos_t, sin_t, (size_t)batch * kv_heads, head_dim, kr);
    /* the append: rotated K (as fp32) and raw V at `position` */
    for (uint32_t b = 0; b < batch; ++b)
        for (uint32_t g = 0; g < kv_heads; ++g) {
            size_t src = ((size_t)b * kv_heads + g) * d;
            size_t dst = (((size_t)b * kv_heads + g) * max_seq + position) * d;
            for (size_t e = 0; e < d; ++e) {
                k_cache[dst + e] = (float)kr[src + e];
                v_cache[dst + e] = v_raw[src + e];
            }
        }
    int bad = 0;
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * n);
        if (!scores) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (size_t t = 0; t < (size_t)batch * num_heads; ++t) {
            if (!scores)
                continue;
            uint32_t b = (uint32_t)(t / num_heads), h = (uint32_t)(t % num_heads);
            uint32_t g = h / repeat;
            const double *qh = qr + t * d;
            size_t base = (((size_t)b * kv_heads + g) * max_seq + window_start) * d;
            const float *k0 = k_cache + base, *v0 = v_cache + base;
            size_t j, e;
            /* scores: cached rows as stored; the new row from the fp64 rotation */
            for (j = 0; j < n; ++j) {
                double dot = 0.0;
                if (window_start + j == position) {
                    const double *kn = kr + ((size_t)b * kv_heads + g) * d;
                    for (e = 0; e < d; ++e)
                        dot += qh[e] * kn[e];
                } else {
                    const float *kj = k0 + j * d;
                    for (e = 0; e < d; ++e)
                        dot += qh[e] * (double)kj[e];
                }
                scores[j] = (double)scale * dot;
            }
            double mu = -INFINITY;
            for (j = 0; j < n; ++j)
                if (scores[j] > mu)
                    mu = scores[j];
            double z = 0.0;
            for (j = 0; j < n; ++j) {
                scores[j] = exp(scores[j] - mu);
                z += scores[j];
            }
            double *o = out + t * d;
            for (e = 0; e < d; ++e)
                o[e] = 0.0;
            for (j = 0; j < n; ++j) {
                const float *vj = v0 + j * d;
                double w = scores[j] / z;
                for (e = 0; e < d; ++e)
                    o[e] += w * (double)vj[e];
            }
        }
        free(scores);
    }
    free(qr);
    free(kr);
    return bad ? -1 : 0;
}
