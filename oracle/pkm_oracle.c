/*
 * pkm_oracle.c -- plain, slow, fp64 CPU oracle for the product-key memory
 * lookup forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no source with the HIP
 * library (no headers, helpers, tables or constants).
 *
 * What it computes, step by step, in the order the pages give it:
 *
 *   "Product-Key Memory" (aiwiki), code listing, ProductKeyMemory.forward, and
 *   §Factorising the key space:
 *     1. q = Wq[h] . x_b                      (nn.Linear without bias)
 *     2. q^ = (q - mean)/sqrt(var + eps)*gamma + beta   (BatchNorm1d, running
 *        statistics: the inference-mode reading)
 *     3. q^ is split into its first and second halves (chunk(2)); half p is
 *        scored against its own subkey set C[h,p]: s_p[j] = q^_p . C[h,p,j]
 *     4. each half keeps its top-k, sorted by (score desc, subkey index asc)
 *     5. the k x k candidate grid: score s_0[i] + s_1[j], flat row index
 *        i_0[i]*n_keys + i_1[j]; the top-k of the grid by (score desc,
 *        flat index asc)
 *     6. softmax over the k winning scores (no temperature), max-subtracted
 *        for stability ("You could have invented transformers from memory",
 *        §Self-attention: dividing by the sum leaves only ratios)
 *     7. EmbeddingBag(mode="sum", per_sample_weights): out_b += sum_j w_j *
 *        V[flat_j]; with several heads each head contributes its own k rows
 *        and the contributions are summed.
 *   "Memory Retrieval Mechanisms: From Soft to Efficient", top-k section:
 *     the retrieved vector is the softmax-weighted sum of the k selected
 *     values, which is what steps 6-7 compute.
 *
 * Value tables are dequantised exactly from their stored bits: bf16 and OCP
 * FP8 E4M3 (E4M3FN) each have a decoder below, written from the format
 * definitions; an E4M3 row is multiplied by its fp32 row scale in fp64.
 *
 * Where the pages leave a step open the oracle takes these readings:
 *   - heads: H independent queries (own Wq, BN and subkeys) sharing one value
 *     table, outputs summed over heads; H = 1 is the listing itself;
 *   - Wq[h] is stored [D_out][D_in] (nn.Linear's weight layout);
 *   - ties: the lower subkey index wins inside a half, the lower flat index
 *     wins in the candidate grid;
 *   - non-finite inputs are undefined (never generated).
 *
 * Every floating-point step is fp64; a product of two fp32 inputs is exact
 * in fp64.  Tokens are independent (running-statistics BN), so tokens may be
 * spread over threads; each token's arithmetic is the same plain loop
 * whichever thread runs it.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PKMO_F32 0
#define PKMO_BF16 1
#define PKMO_E4M3 2

typedef struct {
    int32_t D;          /* model width; even */
    int32_t H;          /* heads */
    int32_t n;          /* subkeys per half; the table has n*n rows */
    int32_t k;          /* winners per head */
    int32_t value_type; /* PKMO_F32 / PKMO_BF16 / PKMO_E4M3 */
    int32_t pad_;
    double eps;         /* BatchNorm epsilon */
    const float *wq;    /* [H][D][D]: row f of head h is output feature f */
    const float *mean;  /* [H][D] running mean */
    const float *var;   /* [H][D] running variance */
    const float *gamma; /* [H][D] */
    const float *beta;  /* [H][D] */
    const float *subkeys; /* [H][2][n][D/2] */
    const void *values;   /* [n*n][D] of value_type */
    const float *scale;   /* [n*n] row scales (E4M3 only) */
} pkmo_model;

/* ------------------------------------------------------------------ codecs */

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 mantissa bits. */
double pkmo_bf16_to_f64(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int m = bits & 0x7F;
    double v;
    if (e == 0xFF)
        v = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)m / 128.0, -126);
    else
        v = ldexp(1.0 + (double)m / 128.0, e - 127);
    return sign ? -v : v;
}

/* OCP FP8 E4M3 ("E4M3FN"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits; no infinities; S.1111.111 is NaN; largest finite magnitude 448. */
double pkmo_e4m3_to_f64(uint8_t bits)
{
    int sign = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xF;
    int m = bits & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Value-table element V[row][d] as an exact fp64 number (times the row scale
 * for E4M3 tables). */
static double value_at(const pkmo_model *M, int64_t row, int d)
{
    int64_t off = row * (int64_t)M->D + d;
    switch (M->value_type) {
    case PKMO_F32:
        return (double)((const float *)M->values)[off];
    case PKMO_BF16:
        return pkmo_bf16_to_f64(((const uint16_t *)M->values)[off]);
    default:
        return pkmo_e4m3_to_f64(((const uint8_t *)M->values)[off]) * (double)M->scale[row];
    }
}

/* ------------------------------------------------------------------- steps */

/* Steps 1-2: query projection and inference-mode BatchNorm for one head. */
void pkmo_project_bn(const pkmo_model *M, int h, const float *x_b, double *qhat)
{
    int D = M->D;
    for (int f = 0; f < D; ++f) {
        const float *wrow = M->wq + ((int64_t)h * D + f) * D;
        double q = 0.0;
        for (int d = 0; d < D; ++d)
            q += (double)wrow[d] * (double)x_b[d];
        int64_t pf = (int64_t)h * D + f;
        qhat[f] = (q - (double)M->mean[pf]) / sqrt((double)M->var[pf] + M->eps) * (double)M->gamma[pf] +
                  (double)M->beta[pf];
    }
}

/* Step 3: score half p of q^ against every subkey of C[h,p]; s[p*n + j]. */
void pkmo_half_scores(const pkmo_model *M, int h, const double *qhat, double *s)
{
    int half = M->D / 2, n = M->n;
    for (int p = 0; p < 2; ++p) {
        const double *qp = qhat + p * half;
        for (int j = 0; j < n; ++j) {
            const float *c = M->subkeys + (((int64_t)h * 2 + p) * n + j) * half;
            double acc = 0.0;
            for (int d = 0; d < half; ++d)
                acc += qp[d] * (double)c[d];
            s[p * n + j] = acc;
        }
    }
}

typedef struct {
    double v;
    int64_t i;
} scored;

/* (score desc, index asc): the ordering every top-k here uses. */
static int by_score_then_index(const void *pa, const void *pb)
{
    const scored *a = (const scored *)pa, *b = (const scored *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    if (a->i < b->i) return -1;
    if (a->i > b->i) return 1;
    return 0;
}

/* Step 4: sort all n scores of one half and keep the first kk. */
void pkmo_topk_sorted(int n, const double *s, int kk, double *top, int32_t *idx)
{
    scored *tmp = (scored *)malloc(sizeof(scored) * (size_t)n);
    for (int j = 0; j < n; ++j) {
        tmp[j].v = s[j];
        tmp[j].i = j;
    }
    qsort(tmp, (size_t)n, sizeof(scored), by_score_then_index);
    for (int r = 0; r < kk; ++r) {
        top[r] = tmp[r].v;
        idx[r] = (int32_t)tmp[r].i;
    }
    free(tmp);
}

/* Step 5: build the explicit kk x kk grid of candidates from the two sorted
 * half lists, sort it, keep the first kout.  Returns the number of
 * candidates formed. */
int pkmo_candidates_topk(int n, int kk, const double *top0, const int32_t *idx0, const double *top1,
                         const int32_t *idx1, int kout, double *top, int32_t *flat)
{
    int nc = kk * kk;
    scored *grid = (scored *)malloc(sizeof(scored) * (size_t)nc);
    int c = 0;
    for (int i = 0; i < kk; ++i)
        for (int j = 0; j < kk; ++j) {
            grid[c].v = top0[i] + top1[j];
            grid[c].i = (int64_t)idx0[i] * n + idx1[j];
            ++c;
        }
    qsort(grid, (size_t)nc, sizeof(scored), by_score_then_index);
    for (int r = 0; r < kout; ++r) {
        top[r] = grid[r].v;
        flat[r] = (int32_t)grid[r].i;
    }
    free(grid);
    return c;
}

/* Step 6: softmax over the k winning scores; top[0] is the largest. */
void pkmo_softmax(int k, const double *top, double *w)
{
    double mx = top[0], sum = 0.0;
    for (int j = 1; j < k; ++j)
        if (top[j] > mx) mx = top[j];
    for (int j = 0; j < k; ++j) {
        w[j] = exp(top[j] - mx);
        sum += w[j];
    }
    for (int j = 0; j < k; ++j)
        w[j] /= sum;
}

/* Step 7: out_b += sum_j w_j * V[rows_j] (EmbeddingBag "sum" with per-sample
 * weights). */
void pkmo_gather_add(const pkmo_model *M, int k, const int32_t *rows, const double *w, double *out_b)
{
    for (int j = 0; j < k; ++j)
        for (int d = 0; d < M->D; ++d)
            out_b[d] += w[j] * value_at(M, rows[j], d);
}

/* ------------------------------------------------------------------ driver */

typedef struct {
    const pkmo_model *M;
    const float *x;
    int kk;
    double *out;
    int32_t *idx;
    double *top;
    double *w;
    double *qhat;
    int32_t *ncand;
    int64_t b0, b1;
} job;

static void *run_tokens(void *arg)
{
    job *J = (job *)arg;
    const pkmo_model *M = J->M;
    int D = M->D, H = M->H, n = M->n, kk = J->kk;
    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    double *s = (double *)malloc(sizeof(double) * 2 * (size_t)n);
    double *t0 = (double *)malloc(sizeof(double) * (size_t)kk);
    double *t1 = (double *)malloc(sizeof(double) * (size_t)kk);
    int32_t *i0 = (int32_t *)malloc(sizeof(int32_t) * (size_t)kk);
    int32_t *i1 = (int32_t *)malloc(sizeof(int32_t) * (size_t)kk);
    double *top = (double *)malloc(sizeof(double) * (size_t)kk);
    int32_t *flat = (int32_t *)malloc(sizeof(int32_t) * (size_t)kk);
    double *w = (double *)malloc(sizeof(double) * (size_t)kk);
    for (int64_t b = J->b0; b < J->b1; ++b) {
        const float *xb = J->x + b * D;
        if (J->out)
            for (int d = 0; d < D; ++d)
                J->out[b * D + d] = 0.0;
        for (int h = 0; h < H; ++h) {
            pkmo_project_bn(M, h, xb, q);
            pkmo_half_scores(M, h, q, s);
            pkmo_topk_sorted(n, s, kk, t0, i0);
            pkmo_topk_sorted(n, s + n, kk, t1, i1);
            int nc = pkmo_candidates_topk(n, kk, t0, i0, t1, i1, kk, top, flat);
            int64_t bh = b * H + h;
            if (J->qhat) memcpy(J->qhat + bh * D, q, sizeof(double) * (size_t)D);
            if (J->ncand) J->ncand[bh] = nc;
            if (J->idx) memcpy(J->idx + bh * kk, flat, sizeof(int32_t) * (size_t)kk);
            if (J->top) memcpy(J->top + bh * kk, top, sizeof(double) * (size_t)kk);
            if (J->w || J->out) {
                pkmo_softmax(kk, top, w);
                if (J->w) memcpy(J->w + bh * kk, w, sizeof(double) * (size_t)kk);
                if (J->out) pkmo_gather_add(M, kk, flat, w, J->out + b * D);
            }
        }
    }
    free(q); free(s); free(t0); free(t1); free(i0); free(i1); free(top); free(flat); free(w);
    return NULL;
}

/*
 * Run the lookup for tokens [0, B) of x [B][D].
 *   kk      search depth: per-half top-kk, kk*kk candidates, top-kk kept.
 *           The method itself uses kk = k; kk = k + 1 gives the exact
 *           top-(k+1), by the same exactness argument, which the tests use to
 *           measure the k | k+1 score gap.  out and w need kk == k.
 *   out     [B][D] fp64 or NULL
 *   idx     [B][H][kk] flat row indices, (score desc, flat asc), or NULL
 *   top     [B][H][kk] winning scores or NULL
 *   w       [B][H][kk] softmax weights or NULL
 *   qhat    [B][H][D] normalised queries or NULL
 *   ncand   [B][H] number of candidates formed or NULL
 * Returns 0, or -1 on bad arguments.
 */
int pkmo_run(const pkmo_model *M, int64_t B, const float *x, int kk, double *out, int32_t *idx, double *top,
             double *w, double *qhat, int32_t *ncand, int nthreads)
{
    if (!M || !x || B < 0 || kk < 1 || kk > M->n || (M->D & 1) || M->H < 1) return -1;
    if ((out || w) && kk != M->k) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B) nthreads = (int)(B > 0 ? B : 1);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    job *jobs = (job *)malloc(sizeof(job) * (size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) {
        job J = {M, x, kk, out, idx, top, w, qhat, ncand, B * t / nthreads, B * (t + 1) / nthreads};
        jobs[t] = J;
    }
    for (int t = 1; t < nthreads; ++t)
        pthread_create(&th[t], NULL, run_tokens, &jobs[t]);
    run_tokens(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        pthread_join(th[t], NULL);
    free(th);
    free(jobs);
    return 0;
}

/*
 * Steps 4-6 alone, from given half scores: scores [P][2][n] (P = tokens x
 * heads, half 0 then half 1).  Writes idx/top/w [P][k] (any may be NULL).
 * Returns 0, or -1 on bad arguments.
 */
int pkmo_select(int64_t P, int n, int k, const double *scores, int32_t *idx, double *top, double *w)
{
    if (P < 0 || n < 1 || k < 1 || k > n || !scores) return -1;
    double *t0 = (double *)malloc(sizeof(double) * (size_t)k);
    double *t1 = (double *)malloc(sizeof(double) * (size_t)k);
    int32_t *i0 = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    int32_t *i1 = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    double *tp = (double *)malloc(sizeof(double) * (size_t)k);
    int32_t *fl = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    for (int64_t p = 0; p < P; ++p) {
        const double *s = scores + p * 2 * n;
        pkmo_topk_sorted(n, s, k, t0, i0);
        pkmo_topk_sorted(n, s + n, k, t1, i1);
        pkmo_candidates_topk(n, k, t0, i0, t1, i1, k, tp, fl);
        if (idx) memcpy(idx + p * k, fl, sizeof(int32_t) * (size_t)k);
        if (top) memcpy(top + p * k, tp, sizeof(double) * (size_t)k);
        if (w) pkmo_softmax(k, tp, w + p * k);
    }
    free(t0); free(t1); free(i0); free(i1); free(tp); free(fl);
    return 0;
}

/*
 * Step 7 alone: out[b] = sum_r w[b][r] * V[rows[b][r]] for b < B, r < R,
 * rows [B][R] int32, w [B][R] fp64, out [B][D] fp64 (overwritten).
 */
int pkmo_gather(const pkmo_model *M, int64_t B, int R, const int32_t *rows, const double *w, double *out)
{
    if (!M || B < 0 || R < 0 || !rows || !w || !out) return -1;
    for (int64_t b = 0; b < B; ++b) {
        for (int d = 0; d < M->D; ++d)
            out[b * M->D + d] = 0.0;
        pkmo_gather_add(M, R, rows + b * R, w + b * R, out + b * M->D);
    }
    return 0;
}
