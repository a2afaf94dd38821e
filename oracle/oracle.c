/*
 * oracle.c -- plain fp64 CPU reference for GLM-style sparse MLA prefill.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do. It shares no code, header or table with the HIP library.
 *
 * What it computes, step by step, in the order the method runs:
 *
 *  1. Indexer (spke.com PCP/DCP article, section "Warum nicht TP oder DP?":
 *     the indexer scores every earlier token so that sparse MLA attends to the
 *     2,048 best; footnote 3: one indexer key per token).  For query i at
 *     absolute position p_i and every key j <= p_i:
 *         I_ij = sum_h w_ih * max(0, sum_d qI_ihd * kI_jd)
 *     accumulated in fp64 and rounded once to fp32.  No extra scale: a scale
 *     is the caller's to fold into w.  With FP8 inputs (footnote 3: an
 *     indexer key is 128 FP8 values plus a 4-byte scale) qI and kI are the
 *     decoded E4M3 codes times their row's scale.
 *
 *  2. Top-k (same section): the k largest I_ij over j <= p_i, ties to the
 *     smaller j; all of 0..p_i when p_i + 1 <= k.  Emitted in ascending j,
 *     padded with -1.
 *
 *  3. Absorbed (MQA-form) MLA attention over the selected rows (article,
 *     footnote 1: QK over 576 dimensions, PV over 512, one latent row read
 *     per selected key serves every head; section "PCP": a row serves all 64
 *     heads).  For head h and selected j:
 *         z_j  = sm_scale * sum_{d<576} Q_ihd * K_jd
 *         LSE  = m + ln sum_j exp(z_j - m),   m = max_j z_j
 *         O_c  = sum_j exp(z_j - LSE) * K_jc,  c < 512
 *     in fp64, summing in ascending j.  FP8 rows decode as e4m3(code)*sigma_j.
 *     LSE is the mergeable log-sum-exp of the section "DCP".
 *
 * Decoders: bf16 = the 16 bits placed in the top half of an fp32.
 * OCP E4M3 (e4m3fn): byte s.eeee.mmm; e = 0 -> (-1)^s 2^-6 m/8; otherwise
 * (-1)^s 2^(e-7) (1 + m/8); e = 15 and m = 7 is NaN; no infinities.
 * 656-byte latent row (article, footnote 1: 656 bytes of FP8 KV per token in
 * FlashMLA's fp8_ds_mla format; the layout is this reading of it): bytes
 * 0..511 the E4M3 codes of the 512 latent values, bytes 512..527 four
 * little-endian fp32 scales (scale t covers latent values 128t .. 128t+127),
 * bytes 528..655 the 64 rope values in bf16. Value d < 512 decodes as
 * e4m3(code d) * scale[d / 128]; value 512 + r as bf16(rope r).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK_DIM 576
#define V_DIM 512

enum { FMT_BF16 = 0, FMT_E4M3 = 1, FMT_F64 = 2, FMT_DS656 = 3 };
#define DS656_ROW 656

/* Threads an OpenMP loop of the oracle uses (OMP_NUM_THREADS, else the cores). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

double oracle_bf16_decode(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Decode element d of row r of a KV (or query) array into a double. */
static double load_elem(int fmt, const void *base, int64_t row_elems, int64_t r, int64_t d,
                        const float *scale) {
    switch (fmt) {
    case FMT_BF16: return oracle_bf16_decode(((const uint16_t *)base)[r * row_elems + d]);
    case FMT_E4M3:
        return oracle_e4m3_decode(((const uint8_t *)base)[r * row_elems + d]) * (double)scale[r];
    case FMT_DS656: {                 /* rows of DS656_ROW bytes; row_elems unused */
        const uint8_t *row = (const uint8_t *)base + r * DS656_ROW;
        if (d < V_DIM) {
            float sc;
            memcpy(&sc, row + V_DIM + 4 * (d / 128), sizeof sc);
            return oracle_e4m3_decode(row[d]) * (double)sc;
        }
        uint16_t h;
        memcpy(&h, row + V_DIM + 16 + 2 * (d - V_DIM), sizeof h);
        return oracle_bf16_decode(h);
    }
    default: return ((const double *)base)[r * row_elems + d];
    }
}

/* ---- 1. indexer ------------------------------------------------------- */
/* One sequence, any element format. q [n * n_heads rows of head_dim];
 * k [L rows of head_dim]; q_scale [n * n_heads] and k_scale [L] are read for
 * E4M3 only (each decoded element times its row's scale); w [n, n_heads];
 * q_pos [n]; scores [n, ld], written for j <= q_pos[i]. */
static void indexer_any(int64_t n, int64_t n_heads, int64_t head_dim, int64_t L, int fmt,
                        const void *q_idx, const float *q_scale, const void *k_idx,
                        const float *k_scale, const float *w, const int32_t *q_pos, float *scores,
                        int64_t ld) {
    double *kd = (double *)malloc(sizeof(double) * (size_t)(L * head_dim));
    for (int64_t j = 0; j < L; ++j)
        for (int64_t d = 0; d < head_dim; ++d)
            kd[j * head_dim + d] = load_elem(fmt, k_idx, head_dim, j, d, k_scale);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        double *qd = (double *)malloc(sizeof(double) * (size_t)(n_heads * head_dim));
        for (int64_t h = 0; h < n_heads; ++h)
            for (int64_t d = 0; d < head_dim; ++d)
                qd[h * head_dim + d] = load_elem(fmt, q_idx, head_dim, i * n_heads + h, d, q_scale);
        int64_t p = q_pos[i];
        for (int64_t j = 0; j <= p && j < L; ++j) {
            double acc = 0.0;
            for (int64_t h = 0; h < n_heads; ++h) {
                double dot = 0.0;
                for (int64_t d = 0; d < head_dim; ++d) dot += qd[h * head_dim + d] * kd[j * head_dim + d];
                if (dot > 0.0) acc += (double)w[i * n_heads + h] * dot;
            }
            scores[i * ld + j] = (float)acc;
        }
        free(qd);
    }
    free(kd);
}

/* q_idx [n, n_heads, head_dim] bf16; k_idx [L, head_dim] bf16 (one sequence);
 * w [n, n_heads] fp32; q_pos [n]; scores [n, ld], written for j <= q_pos[i]. */
void oracle_indexer(int64_t n, int64_t n_heads, int64_t head_dim, int64_t L,
                    const uint16_t *q_idx, const uint16_t *k_idx, const float *w,
                    const int32_t *q_pos, float *scores, int64_t ld) {
    indexer_any(n, n_heads, head_dim, L, FMT_BF16, q_idx, NULL, k_idx, NULL, w, q_pos, scores, ld);
}

/* FP8 indexer inputs (article, footnote 3: an indexer key is 128 FP8 values
 * and a 4-byte scale): q_idx [n, n_heads, head_dim] and k_idx [L, head_dim]
 * E4M3 codes, q_scale [n, n_heads], k_scale [L] fp32. An element is
 * decode(code) * scale of its row; the score is then the formula above. */
void oracle_indexer_e4m3(int64_t n, int64_t n_heads, int64_t head_dim, int64_t L,
                         const uint8_t *q_idx, const float *q_scale, const uint8_t *k_idx,
                         const float *k_scale, const float *w, const int32_t *q_pos,
                         float *scores, int64_t ld) {
    indexer_any(n, n_heads, head_dim, L, FMT_E4M3, q_idx, q_scale, k_idx, k_scale, w, q_pos,
                scores, ld);
}

/* ---- 2. top-k --------------------------------------------------------- */
typedef struct {
    double s;
    int32_t j;
} scored_t;

static int by_score_desc_then_index(const void *a, const void *b) {
    const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static int by_int_asc(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* scores [n, ld] fp32 (row i valid for j <= q_pos[i]) -> indices [n, k]. */
void oracle_topk(int64_t n, const float *scores, int64_t ld, const int32_t *q_pos, int32_t k,
                 int32_t *indices) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        int64_t cnt = (int64_t)q_pos[i] + 1;
        int32_t *out = indices + i * k;
        int64_t keep;
        if (cnt <= k) {
            for (int64_t j = 0; j < cnt; ++j) out[j] = (int32_t)j;
            keep = cnt;
        } else {
            scored_t *row = (scored_t *)malloc(sizeof(scored_t) * (size_t)cnt);
            for (int64_t j = 0; j < cnt; ++j) {
                row[j].s = (double)scores[i * ld + j];
                row[j].j = (int32_t)j;
            }
            qsort(row, (size_t)cnt, sizeof(scored_t), by_score_desc_then_index);
            for (int64_t t = 0; t < k; ++t) out[t] = row[t].j;
            free(row);
            qsort(out, (size_t)k, sizeof(int32_t), by_int_asc);
            keep = k;
        }
        for (int64_t t = keep; t < k; ++t) out[t] = -1;
    }
}

/* ---- 3. absorbed MLA attention ---------------------------------------- */
/* q [n, n_heads, 576] (bf16 or f64); kv [L, 576] (bf16, e4m3 + kv_scale[L], or
 * f64), or [L, 656] bytes of 656-byte rows (FMT_DS656), for one sequence; indices [n, k] local rows (entries < 0 or > q_pos[i]
 * are skipped), or NULL for all j <= q_pos[i]; out [n, n_heads, 512] f64,
 * lse [n, n_heads] f64 (natural log).  An empty set gives O = 0, LSE = -inf. */
void oracle_attention(int64_t n, int64_t n_heads, int64_t L, int q_fmt, const void *q,
                      int kv_fmt, const void *kv, const float *kv_scale,
                      const int32_t *indices, int32_t k, const int32_t *q_pos, double sm_scale,
                      double *out, double *lse) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        int64_t p = q_pos[i];
        int64_t cap = indices ? (int64_t)k : p + 1;
        int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(cap > 0 ? cap : 1));
        int64_t ns = 0;
        if (indices) {
            for (int64_t t = 0; t < k; ++t) {
                int32_t j = indices[i * k + t];
                if (j >= 0 && j <= p && j < L) sel[ns++] = j;
            }
            qsort(sel, (size_t)ns, sizeof(int32_t), by_int_asc);
        } else {
            for (int64_t j = 0; j <= p && j < L; ++j) sel[ns++] = (int32_t)j;
        }
        double *rows = (double *)malloc(sizeof(double) * (size_t)((ns > 0 ? ns : 1) * QK_DIM));
        for (int64_t t = 0; t < ns; ++t)
            for (int64_t d = 0; d < QK_DIM; ++d)
                rows[t * QK_DIM + d] = load_elem(kv_fmt, kv, QK_DIM, sel[t], d, kv_scale);
        double *z = (double *)malloc(sizeof(double) * (size_t)(ns > 0 ? ns : 1));
        double qh[QK_DIM];
        for (int64_t h = 0; h < n_heads; ++h) {
            double *o = out + (i * n_heads + h) * V_DIM;
            for (int64_t d = 0; d < QK_DIM; ++d)
                qh[d] = load_elem(q_fmt, q, n_heads * QK_DIM, i, h * QK_DIM + d, NULL);
            for (int64_t c = 0; c < V_DIM; ++c) o[c] = 0.0;
            if (ns == 0) {
                lse[i * n_heads + h] = -INFINITY;
                continue;
            }
            double m = -INFINITY;
            for (int64_t t = 0; t < ns; ++t) {
                double dot = 0.0;
                for (int64_t d = 0; d < QK_DIM; ++d) dot += qh[d] * rows[t * QK_DIM + d];
                z[t] = sm_scale * dot;
                if (z[t] > m) m = z[t];
            }
            double l = 0.0;
            for (int64_t t = 0; t < ns; ++t) l += exp(z[t] - m);
            double L_ = m + log(l);
            lse[i * n_heads + h] = L_;
            for (int64_t t = 0; t < ns; ++t) {
                double pr = exp(z[t] - L_);
                for (int64_t c = 0; c < V_DIM; ++c) o[c] += pr * rows[t * QK_DIM + c];
            }
        }
        free(z);
        free(rows);
        free(sel);
    }
}
