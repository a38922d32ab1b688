/*
 * CPU fp64 oracle for the MLA tree-verify attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. The GPU path never calls it and shares no code with it.
 *
 * What it computes (plain definition, every product and sum in double):
 *   For request b, draft token i and head h, with P_b = kv_indptr[b+1] - kv_indptr[b]
 *   and L_b = P_b + q_len, the columns c = 0..L_b-1 are the prefix tokens followed by
 *   the draft tokens. Column c reads pool row
 *       kv_indices[kv_indptr[b] + c]           if c <  P_b   (prefix, from the pool index list)
 *       out_cache_loc[b*q_len + (c - P_b)]     if c >= P_b   (draft, freshly written slots)
 *   ("From Capture Safety to MoE Ceiling", section "The Architecture of Capture Safety":
 *   two index arrays selected by position relative to the prefix length; "The Custom
 *   sm_120 Verify Kernel", section "The Debugging Gauntlet", bug 2: prefix then draft).
 *   Column c is visible to row (i, h) iff custom_mask[mask_indptr[b] + i*L_b + c] != 0
 *   (same sections: raw mask plus per-request offsets, row stride prefix + q_len).
 *   The key of column c is all 576 values of its pool row, the value is its first 512
 *   (the shared MLA latent); the query is q_nope[b,i,h,:] followed by q_rope[b,i,h,:].
 *   s_c = scale * <q, K_c>; over visible columns: m = max s_c, lse = m + ln sum exp(s_c - m),
 *   out[e] = sum exp(s_c - lse) * V_c[e]. A row with no visible column gets out = 0, lse = -inf.
 *
 * The split variant computes the same quantity the way the split-KV flash-decode does
 * ("The Custom sm_120 Verify Kernel", section "Building the Custom Kernel": each split
 * holds partial softmax statistics of one contiguous column slice, a second pass combines
 * them): chunk = ceil(L_b / nsplit); split s covers [s*chunk, min(L_b, (s+1)*chunk));
 * per split m_s, l_s = sum exp(s_c - m_s), acc_s = sum exp(s_c - m_s) V_c over its visible
 * columns; then M = max m_s, w_s = exp(m_s - M), out = sum w_s acc_s / sum w_s l_s,
 * lse = M + ln sum w_s l_s. Splits that are empty or fully masked are skipped.
 *
 * Return value: 0 on success, -1 on a null pointer, -2 on a bad size, -3 on a slot outside
 * [0, N).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LATENT 512
#define ROPE 64
#define ROW (LATENT + ROPE)

static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q_nope, *q_rope, *kv_pool;
    int64_t N;
    const int32_t *kv_indptr, *kv_indices, *out_cache_loc;
    const uint8_t *custom_mask;
    const int32_t *mask_indptr;
    int B, q_len, H;
    double scale;
} problem;

static int check(const problem *p) {
    if (!p->q_nope || !p->q_rope || !p->kv_pool || !p->kv_indptr || !p->out_cache_loc ||
        !p->custom_mask || !p->mask_indptr)
        return -1;
    if (p->B < 0 || p->q_len < 1 || p->H < 1 || p->N < 1) return -2;
    for (int b = 0; b < p->B; ++b)
        if (p->kv_indptr[b + 1] < p->kv_indptr[b]) return -2;
    if (p->kv_indptr[p->B] > p->kv_indptr[0] && !p->kv_indices) return -1;
    for (int b = 0; b < p->B; ++b) {
        for (int32_t k = p->kv_indptr[b]; k < p->kv_indptr[b + 1]; ++k)
            if (p->kv_indices[k] < 0 || p->kv_indices[k] >= p->N) return -3;
        for (int t = 0; t < p->q_len; ++t) {
            int32_t s = p->out_cache_loc[(int64_t)b * p->q_len + t];
            if (s < 0 || s >= p->N) return -3;
        }
    }
    return 0;
}

static int64_t column_slot(const problem *p, int b, int c) {
    int prefix = p->kv_indptr[b + 1] - p->kv_indptr[b];
    if (c < prefix) return p->kv_indices[p->kv_indptr[b] + c];
    return p->out_cache_loc[(int64_t)b * p->q_len + (c - prefix)];
}

static int visible(const problem *p, int b, int i, int c) {
    int L = p->kv_indptr[b + 1] - p->kv_indptr[b] + p->q_len;
    return p->custom_mask[(int64_t)p->mask_indptr[b] + (int64_t)i * L + c] != 0;
}

/* Scores of one row for every column (masked columns get -inf). */
static void row_scores(const problem *p, int b, int i, int h, double *s) {
    int L = p->kv_indptr[b + 1] - p->kv_indptr[b] + p->q_len;
    const uint16_t *qn = p->q_nope + (((int64_t)b * p->q_len + i) * p->H + h) * LATENT;
    const uint16_t *qr = p->q_rope + (((int64_t)b * p->q_len + i) * p->H + h) * ROPE;
    for (int c = 0; c < L; ++c) {
        if (!visible(p, b, i, c)) { s[c] = -INFINITY; continue; }
        const uint16_t *k = p->kv_pool + column_slot(p, b, c) * ROW;
        double dot = 0.0;
        for (int d = 0; d < LATENT; ++d) dot += bf16_value(qn[d]) * bf16_value(k[d]);
        for (int d = 0; d < ROPE; ++d) dot += bf16_value(qr[d]) * bf16_value(k[LATENT + d]);
        s[c] = p->scale * dot;
    }
}

/* Plain definition for one row: softmax over the visible scores, then the weighted latent sum. */
static void row_plain(const problem *p, int b, int i, int h, double *s, double *out, double *lse) {
    int L = p->kv_indptr[b + 1] - p->kv_indptr[b] + p->q_len;
    row_scores(p, b, i, h, s);
    double m = -INFINITY;
    for (int c = 0; c < L; ++c) if (s[c] > m) m = s[c];
    for (int e = 0; e < LATENT; ++e) out[e] = 0.0;
    if (m == -INFINITY) { *lse = -INFINITY; return; }
    double z = 0.0;
    for (int c = 0; c < L; ++c) if (s[c] != -INFINITY) z += exp(s[c] - m);
    double l = m + log(z);
    for (int c = 0; c < L; ++c) {
        if (s[c] == -INFINITY) continue;
        double w = exp(s[c] - l);
        const uint16_t *v = p->kv_pool + column_slot(p, b, c) * ROW;
        for (int e = 0; e < LATENT; ++e) out[e] += w * bf16_value(v[e]);
    }
    *lse = l;
}

/* Split-then-combine for one row. */
static void row_split(const problem *p, int b, int i, int h, int nsplit, double *s, double *acc,
                      double *out, double *lse) {
    int L = p->kv_indptr[b + 1] - p->kv_indptr[b] + p->q_len;
    row_scores(p, b, i, h, s);
    int chunk = (L + nsplit - 1) / nsplit;
    double M = -INFINITY;
    /* statistics of each split: acc holds [m_s, l_s, acc_s[512]] per split */
    for (int sp = 0; sp < nsplit; ++sp) {
        double *st = acc + (int64_t)sp * (LATENT + 2);
        int c0 = sp * chunk, c1 = c0 + chunk < L ? c0 + chunk : L;
        double ms = -INFINITY;
        for (int c = c0; c < c1; ++c) if (s[c] > ms) ms = s[c];
        st[0] = ms;
        st[1] = 0.0;
        for (int e = 0; e < LATENT; ++e) st[2 + e] = 0.0;
        if (ms == -INFINITY) continue;  /* empty or fully masked split */
        for (int c = c0; c < c1; ++c) {
            if (s[c] == -INFINITY) continue;
            double w = exp(s[c] - ms);
            st[1] += w;
            const uint16_t *v = p->kv_pool + column_slot(p, b, c) * ROW;
            for (int e = 0; e < LATENT; ++e) st[2 + e] += w * bf16_value(v[e]);
        }
        if (ms > M) M = ms;
    }
    for (int e = 0; e < LATENT; ++e) out[e] = 0.0;
    if (M == -INFINITY) { *lse = -INFINITY; return; }
    double den = 0.0;
    for (int sp = 0; sp < nsplit; ++sp) {
        double *st = acc + (int64_t)sp * (LATENT + 2);
        if (st[0] == -INFINITY) continue;
        double w = exp(st[0] - M);
        den += w * st[1];
        for (int e = 0; e < LATENT; ++e) out[e] += w * st[2 + e];
    }
    for (int e = 0; e < LATENT; ++e) out[e] /= den;
    *lse = M + log(den);
}

static int max_len(const problem *p) {
    int mx = 0;
    for (int b = 0; b < p->B; ++b) {
        int L = p->kv_indptr[b + 1] - p->kv_indptr[b] + p->q_len;
        if (L > mx) mx = L;
    }
    return mx;
}

#define PROBLEM_ARGS                                                                             \
    const uint16_t *q_nope, const uint16_t *q_rope, const uint16_t *kv_pool, int64_t N,         \
        const int32_t *kv_indptr, const int32_t *kv_indices, const int32_t *out_cache_loc,       \
        const uint8_t *custom_mask, const int32_t *mask_indptr, int B, int q_len, int H, double scale
#define PROBLEM_INIT                                                                             \
    problem p = {q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask,  \
                 mask_indptr, B, q_len, H, scale};                                               \
    int rc = check(&p);                                                                          \
    if (rc) return rc;

/* out: double [B, q_len, H, 512]; lse: double [B, q_len, H]. nthreads <= 0: OpenMP default. */
int mla_oracle_attn(PROBLEM_ARGS, double *out, double *lse, int nthreads) {
    PROBLEM_INIT
    if (!out || !lse) return -1;
    int64_t rows = (int64_t)B * q_len * H;
    int L = max_len(&p);
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
    {
        double *s = (double *)malloc(sizeof(double) * (L > 0 ? L : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < rows; ++r) {
            int h = (int)(r % H), i = (int)((r / H) % q_len), b = (int)(r / ((int64_t)H * q_len));
            row_plain(&p, b, i, h, s, out + r * LATENT, lse + r);
        }
        free(s);
    }
    return 0;
}

/* Same result through nsplit partials and the log-sum-exp combine. */
int mla_oracle_attn_split(PROBLEM_ARGS, int nsplit, double *out, double *lse, int nthreads) {
    PROBLEM_INIT
    if (!out || !lse) return -1;
    if (nsplit < 1) return -2;
    int64_t rows = (int64_t)B * q_len * H;
    int L = max_len(&p);
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
    {
        double *s = (double *)malloc(sizeof(double) * (L > 0 ? L : 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)nsplit * (LATENT + 2));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < rows; ++r) {
            int h = (int)(r % H), i = (int)((r / H) % q_len), b = (int)(r / ((int64_t)H * q_len));
            row_split(&p, b, i, h, nsplit, s, acc, out + r * LATENT, lse + r);
        }
        free(acc);
        free(s);
    }
    return 0;
}

/* A chosen set of rows (b, i, h) only; out: double [nrows, 512], lse: double [nrows]. */
int mla_oracle_attn_rows(PROBLEM_ARGS, int64_t nrows, const int32_t *row_b, const int32_t *row_i,
                         const int32_t *row_h, double *out, double *lse, int nthreads) {
    PROBLEM_INIT
    if (!row_b || !row_i || !row_h || !out || !lse) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (row_b[r] < 0 || row_b[r] >= B || row_i[r] < 0 || row_i[r] >= q_len || row_h[r] < 0 ||
            row_h[r] >= H)
            return -2;
    int L = max_len(&p);
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
    {
        double *s = (double *)malloc(sizeof(double) * (L > 0 ? L : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r)
            row_plain(&p, row_b[r], row_i[r], row_h[r], s, out + r * LATENT, lse + r);
        free(s);
    }
    return 0;
}

/* Softmax weights of one row over its L_b columns (0 for masked columns): a debug view. */
int mla_oracle_row_weights(PROBLEM_ARGS, int b, int i, int h, double *weights) {
    PROBLEM_INIT
    if (!weights) return -1;
    if (b < 0 || b >= B || i < 0 || i >= q_len || h < 0 || h >= H) return -2;
    int L = kv_indptr[b + 1] - kv_indptr[b] + q_len;
    row_scores(&p, b, i, h, weights);
    double m = -INFINITY;
    for (int c = 0; c < L; ++c) if (weights[c] > m) m = weights[c];
    if (m == -INFINITY) { for (int c = 0; c < L; ++c) weights[c] = 0.0; return 0; }
    double z = 0.0;
    for (int c = 0; c < L; ++c) if (weights[c] != -INFINITY) z += exp(weights[c] - m);
    for (int c = 0; c < L; ++c) weights[c] = weights[c] == -INFINITY ? 0.0 : exp(weights[c] - m) / z;
    return 0;
}
