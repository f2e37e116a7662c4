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
 * Steps 1-3 (pkmo_scores), 4-6 (pkmo_select) and 7 (pkmo_gather) can also
 * be run on their own, to check the GPU's stages one at a time.  The
 * backward direction (gradients of a loss through steps 7 -> 1 for the
 * winners the forward selected), the training-mode batch statistics and
 * the running statistics BatchNorm1d keeps from them are at the end of the
 * file.
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
#define PKMO_INT8 3
#define PKMO_INT4 4

typedef struct {
    int32_t D;          /* model width; even */
    int32_t H;          /* heads */
    int32_t n;          /* subkeys per half; the table has n*n rows */
    int32_t k;          /* winners per head */
    int32_t value_type; /* PKMO_F32 / PKMO_BF16 / PKMO_E4M3 / PKMO_INT8 / PKMO_INT4 */
    int32_t pad_;
    double eps;         /* BatchNorm epsilon */
    const float *wq;    /* [H][D][D]: row f of head h is output feature f */
    const float *mean;  /* [H][D] running mean */
    const float *var;   /* [H][D] running variance */
    const float *gamma; /* [H][D] */
    const float *beta;  /* [H][D] */
    const float *subkeys; /* [H][2][n][D/2] */
    const void *values;   /* [n*n][D] of value_type ([n*n][D/2] bytes for INT4) */
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

/* Symmetric integer codes (the note after the code listing: the value
 * table is the layer's whole memory cost, so it is the part worth storing
 * in fewer bits): int8 is an ordinary two's complement byte; int4 is a two's
 * complement nibble, two per byte, the element with the even index in the
 * low nibble. */
double pkmo_int8_to_f64(int8_t code) { return (double)code; }

double pkmo_int4_to_f64(uint8_t nibble)
{
    int v = nibble & 0xF;
    return (double)(v >= 8 ? v - 16 : v);
}

/* Value-table element V[row][d] as an exact fp64 number (times the row scale
 * for E4M3, int8 and int4 tables). */
static double value_at(const pkmo_model *M, int64_t row, int d)
{
    int64_t off = row * (int64_t)M->D + d;
    switch (M->value_type) {
    case PKMO_F32:
        return (double)((const float *)M->values)[off];
    case PKMO_BF16:
        return pkmo_bf16_to_f64(((const uint16_t *)M->values)[off]);
    case PKMO_INT8:
        return (double)M->scale[row] * pkmo_int8_to_f64(((const int8_t *)M->values)[off]);
    case PKMO_INT4: {
        const uint8_t byte = ((const uint8_t *)M->values)[off / 2];
        return (double)M->scale[row] * pkmo_int4_to_f64((uint8_t)(d & 1 ? byte >> 4 : byte));
    }
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
 * Steps 1-3 alone: scores [B][H][2][n] of each token's two query halves
 * against their subkey sets, the same arithmetic pkmo_run ranks.
 * Returns 0, or -1 on bad arguments.
 */
int pkmo_scores(const pkmo_model *M, int64_t B, const float *x, double *scores)
{
    if (!M || !x || !scores || B < 0 || (M->D & 1) || M->H < 1) return -1;
    const int D = M->D, H = M->H, n = M->n;
    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    for (int64_t b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            pkmo_project_bn(M, h, x + b * D, q);
            pkmo_half_scores(M, h, q, scores + (b * H + h) * 2 * (int64_t)n);
        }
    free(q);
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

/* ---------------------------------------------------------------- backward */

/*
 * Gradients of L = sum_b dout_b . out_b through steps 7 -> 1.  The top-k
 * selections are piecewise constant in their inputs, so only the winning
 * scores receive gradient (the code listing's topk values feed the softmax;
 * its indices only select).  For token b, head h, winners j < k with flat
 * rows r_j = i0_j * n + i1_j and weights w_j:
 *   g_j     = dout_b . V[r_j]                         (step 7, d/dw_j)
 *   dt_j    = w_j (g_j - sum_l w_l g_l)               (step 6, softmax)
 *   ds_0[i0_j] += dt_j ;  ds_1[i1_j] += dt_j          (step 5: t_j = s_0 + s_1)
 *   dq^_p   = sum_i ds_p[i] C[h,p,i] ;  dC[h,p,i] += ds_p[i] q^_p   (step 3)
 *   xhat    = (q - mean) / sqrt(var + eps)
 *   dgamma += dq^ * xhat ;  dbeta += dq^ ;  dq = dq^ * gamma / sqrt(var + eps)
 *                                                     (step 2, running statistics)
 *   dWq[h] += dq x_b^T ;  dx_b += Wq[h]^T dq           (step 1)
 *   dV[r_j] += w_j dout_b                             (step 7, d/dV of the
 *                                                      dequantised rows)
 * Per-token quantities are computed in parallel over tokens; every
 * parameter gradient element is then summed over tokens in token order by
 * the one thread that owns it, so the result does not depend on the thread
 * count.
 */

typedef struct {
    const pkmo_model *M;
    const float *x, *dout;
    double *dx;
    /* per (token, head): */
    double *qhat, *xhat, *dqhat; /* [B][H][D] */
    double *dt, *w;              /* [B][H][k] */
    int32_t *rows;               /* [B][H][k] */
    int64_t b0, b1;
} bwd_job;

static void *backward_tokens(void *arg)
{
    bwd_job *J = (bwd_job *)arg;
    const pkmo_model *M = J->M;
    const int D = M->D, H = M->H, n = M->n, k = M->k, half = D / 2;
    double *s = (double *)malloc(sizeof(double) * 2 * (size_t)n);
    double *t0 = (double *)malloc(sizeof(double) * (size_t)k);
    double *t1 = (double *)malloc(sizeof(double) * (size_t)k);
    int32_t *i0 = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    int32_t *i1 = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    double *top = (double *)malloc(sizeof(double) * (size_t)k);
    double *g = (double *)malloc(sizeof(double) * (size_t)k);
    double *dq = (double *)malloc(sizeof(double) * (size_t)D);
    for (int64_t b = J->b0; b < J->b1; ++b) {
        const float *xb = J->x + b * D, *gb = J->dout + b * D;
        if (J->dx)
            for (int d = 0; d < D; ++d)
                J->dx[b * D + d] = 0.0;
        for (int h = 0; h < H; ++h) {
            const int64_t bh = b * H + h;
            double *qh = J->qhat + bh * D, *xh = J->xhat + bh * D, *dqh = J->dqhat + bh * D;
            double *dtj = J->dt + bh * k, *wj = J->w + bh * k;
            int32_t *rj = J->rows + bh * k;
            /* forward again: steps 1-6 */
            pkmo_project_bn(M, h, xb, qh);
            pkmo_half_scores(M, h, qh, s);
            pkmo_topk_sorted(n, s, k, t0, i0);
            pkmo_topk_sorted(n, s + n, k, t1, i1);
            pkmo_candidates_topk(n, k, t0, i0, t1, i1, k, top, rj);
            pkmo_softmax(k, top, wj);
            /* step 7 and the softmax, backwards */
            double wg = 0.0;
            for (int j = 0; j < k; ++j) {
                double acc = 0.0;
                for (int d = 0; d < D; ++d)
                    acc += (double)gb[d] * value_at(M, rj[j], d);
                g[j] = acc;
                wg += wj[j] * acc;
            }
            for (int j = 0; j < k; ++j)
                dtj[j] = wj[j] * (g[j] - wg);
            /* step 5 then 3: dq^_p = sum_j dt_j C[h,p,i_p(j)] */
            for (int d = 0; d < D; ++d)
                dqh[d] = 0.0;
            for (int j = 0; j < k; ++j) {
                const int a = rj[j] / n, c = rj[j] % n;
                const float *c0 = M->subkeys + (((int64_t)h * 2 + 0) * n + a) * half;
                const float *c1 = M->subkeys + (((int64_t)h * 2 + 1) * n + c) * half;
                for (int d = 0; d < half; ++d) {
                    dqh[d] += dtj[j] * (double)c0[d];
                    dqh[half + d] += dtj[j] * (double)c1[d];
                }
            }
            /* step 2 backwards (running statistics) and step 1's dx */
            for (int f = 0; f < D; ++f) {
                const int64_t pf = (int64_t)h * D + f;
                const double inv = 1.0 / sqrt(M->eps + (double)M->var[pf]);
                double q = 0.0;
                const float *wrow = M->wq + pf * D;
                for (int d = 0; d < D; ++d)
                    q += (double)wrow[d] * (double)xb[d];
                const double mu = M->mean[pf];
                xh[f] = inv * (q - mu);
                dq[f] = dqh[f] * (double)M->gamma[pf] * inv;
            }
            if (J->dx)
                for (int f = 0; f < D; ++f) {
                    const float *wrow = M->wq + ((int64_t)h * D + f) * D;
                    for (int d = 0; d < D; ++d)
                        J->dx[b * D + d] += dq[f] * (double)wrow[d];
                }
        }
    }
    free(s); free(t0); free(t1); free(i0); free(i1); free(top); free(g); free(dq);
    return NULL;
}

typedef struct {
    const pkmo_model *M;
    int64_t B;
    const float *x, *dout;
    const double *qhat, *xhat, *dqhat, *dt, *w;
    const int32_t *rows;
    double *dwq, *dgamma, *dbeta, *dsub, *dval;
    int t, nthreads; /* thread t owns the t-th of nthreads equal ranges of the
                        features [H*D], the subkey rows [H*2*n] and the value
                        rows [n*n] */
} own_job;

static void *owner_sums(void *arg)
{
    own_job *J = (own_job *)arg;
    const pkmo_model *M = J->M;
    const int D = M->D, H = M->H, n = M->n, k = M->k, half = D / 2;
    const int64_t B = J->B, N = (int64_t)n * n;
    const int64_t HD = (int64_t)H * D, HS = (int64_t)H * 2 * n;
    const int64_t f0 = HD * J->t / J->nthreads, f1 = HD * (J->t + 1) / J->nthreads;
    const int64_t s0 = HS * J->t / J->nthreads, s1 = HS * (J->t + 1) / J->nthreads;
    const int64_t r0 = N * J->t / J->nthreads, r1 = N * (J->t + 1) / J->nthreads;
    /* features (h, f) in [f0, f1): dWq rows, dgamma, dbeta */
    for (int64_t pf = f0; pf < f1; ++pf) {
        const int h = (int)(pf / D);
        const double scale = (double)M->gamma[pf] / sqrt(M->eps + (double)M->var[pf]);
        if (J->dwq)
            for (int d = 0; d < D; ++d)
                J->dwq[pf * D + d] = 0.0;
        if (J->dgamma) J->dgamma[pf] = 0.0;
        if (J->dbeta) J->dbeta[pf] = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            const int64_t at = (b * H + h) * D + (pf - (int64_t)h * D);
            const double dqh = J->dqhat[at];
            if (J->dgamma) J->dgamma[pf] += dqh * J->xhat[at];
            if (J->dbeta) J->dbeta[pf] += dqh;
            if (J->dwq) {
                const double dq = dqh * scale;
                const float *xb = J->x + b * D;
                for (int d = 0; d < D; ++d)
                    J->dwq[pf * D + d] += dq * (double)xb[d];
            }
        }
    }
    /* subkey rows (h, p, i) in [s0, s1) */
    if (J->dsub)
        for (int64_t sr = s0; sr < s1; ++sr) {
            const int h = (int)(sr / (2 * n)), p = (int)((sr / n) % 2), i = (int)(sr % n);
            double *out = J->dsub + sr * half;
            for (int d = 0; d < half; ++d)
                out[d] = 0.0;
            for (int64_t b = 0; b < B; ++b) {
                const int64_t bh = b * H + h;
                for (int j = 0; j < k; ++j) {
                    const int32_t r = J->rows[bh * k + j];
                    if ((p == 0 ? r / n : r % n) != i) continue;
                    const double *qp = J->qhat + bh * D + p * half;
                    for (int d = 0; d < half; ++d)
                        out[d] += J->dt[bh * k + j] * qp[d];
                }
            }
        }
    /* value rows in [r0, r1) */
    if (J->dval) {
        for (int64_t r = r0; r < r1; ++r)
            for (int d = 0; d < D; ++d)
                J->dval[r * D + d] = 0.0;
        for (int64_t bh = 0; bh < B * H; ++bh)
            for (int j = 0; j < k; ++j) {
                const int64_t r = J->rows[bh * k + j];
                if (r < r0 || r >= r1) continue;
                const float *gb = J->dout + (bh / H) * D;
                for (int d = 0; d < D; ++d)
                    J->dval[r * D + d] += J->w[bh * k + j] * (double)gb[d];
            }
    }
    return NULL;
}

/*
 * Gradients for tokens [0, B) of x [B][D] given dout [B][D] (dL/dout).  Each
 * output is overwritten, or skipped when NULL:
 *   dx      [B][D]          dgamma, dbeta [H][D]
 *   dwq     [H][D][D]       dsub          [H][2][n][D/2]
 *   dval    [n*n][D]  (w.r.t. the dequantised value rows)
 * Returns 0, -1 on bad arguments, -2 if memory runs out.
 */
int pkmo_backward(const pkmo_model *M, int64_t B, const float *x, const float *dout, double *dx, double *dwq,
                  double *dgamma, double *dbeta, double *dsub, double *dval, int nthreads)
{
    if (!M || !x || !dout || B < 0 || (M->D & 1) || M->H < 1 || M->k < 1 || M->k > M->n) return -1;
    if (!M->values) return -1; /* step 7's g_j reads the value rows */
    if (nthreads < 1) nthreads = 1;
    const int D = M->D, H = M->H, k = M->k;
    const size_t bhd = (size_t)B * H * D, bhk = (size_t)B * H * k;
    double *qhat = (double *)malloc(sizeof(double) * (bhd ? bhd : 1));
    double *xhat = (double *)malloc(sizeof(double) * (bhd ? bhd : 1));
    double *dqhat = (double *)malloc(sizeof(double) * (bhd ? bhd : 1));
    double *dt = (double *)malloc(sizeof(double) * (bhk ? bhk : 1));
    double *w = (double *)malloc(sizeof(double) * (bhk ? bhk : 1));
    int32_t *rows = (int32_t *)malloc(sizeof(int32_t) * (bhk ? bhk : 1));
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    bwd_job *bj = (bwd_job *)malloc(sizeof(bwd_job) * (size_t)nthreads);
    own_job *oj = (own_job *)malloc(sizeof(own_job) * (size_t)nthreads);
    if (!qhat || !xhat || !dqhat || !dt || !w || !rows || !th || !bj || !oj) {
        free(qhat); free(xhat); free(dqhat); free(dt); free(w); free(rows); free(th); free(bj); free(oj);
        return -2;
    }
    const int tt = (int)(nthreads < (B > 0 ? B : 1) ? nthreads : (B > 0 ? B : 1));
    for (int t = 0; t < tt; ++t) {
        bwd_job J = {M, x, dout, dx, qhat, xhat, dqhat, dt, w, rows, B * t / tt, B * (t + 1) / tt};
        bj[t] = J;
    }
    for (int t = 1; t < tt; ++t)
        pthread_create(&th[t], NULL, backward_tokens, &bj[t]);
    backward_tokens(&bj[0]);
    for (int t = 1; t < tt; ++t)
        pthread_join(th[t], NULL);
    for (int t = 0; t < nthreads; ++t) {
        own_job J = {M, B, x, dout, qhat, xhat, dqhat, dt, w, rows, dwq, dgamma, dbeta, dsub, dval, t, nthreads};
        oj[t] = J;
    }
    for (int t = 1; t < nthreads; ++t)
        pthread_create(&th[t], NULL, owner_sums, &oj[t]);
    owner_sums(&oj[0]);
    for (int t = 1; t < nthreads; ++t)
        pthread_join(th[t], NULL);
    free(qhat); free(xhat); free(dqhat); free(dt); free(w); free(rows); free(th); free(bj); free(oj);
    return 0;
}

/* ------------------------------------------------- batch-statistics BN */

/*
 * Training-mode BatchNorm1d ("Product-Key Memory", §Keeping the memory in
 * use: batch normalisation of the query, computed over the batch):
 * per head h and feature f, over the B tokens,
 *   mean = (1/B) sum_b q_bf,   var = (1/B) sum_b (q_bf - mean)^2  (biased,
 * the normaliser BatchNorm1d uses), q = Wq[h] . x_b in fp64, two passes.
 * mean, var: [H][D] fp64.  Returns 0, or -1 on bad arguments (B < 1).
 */
int pkmo_batch_stats(const pkmo_model *M, int64_t B, const float *x, double *mean, double *var)
{
    if (!M || !x || !mean || !var || B < 1) return -1;
    const int D = M->D, H = M->H;
    double *col = (double *)malloc(sizeof(double) * (size_t)B);
    if (!col) return -1;
    for (int h = 0; h < H; ++h)
        for (int f = 0; f < D; ++f) {
            const float *wrow = M->wq + ((int64_t)h * D + f) * D;
            double sum = 0.0;
            for (int64_t b = 0; b < B; ++b) {
                double acc = 0.0;
                for (int d = 0; d < D; ++d)
                    acc += (double)wrow[d] * (double)x[b * D + d];
                col[b] = acc;
                sum += acc;
            }
            const double mu = sum / (double)B;
            double ss = 0.0;
            for (int64_t b = 0; b < B; ++b)
                ss += (col[b] - mu) * (col[b] - mu);
            mean[(int64_t)h * D + f] = mu;
            var[(int64_t)h * D + f] = ss / (double)B;
        }
    free(col);
    return 0;
}

/* A copy of the model whose BN statistics are the given fp64 ones: the
 * per-token steps read them through these arrays instead. */
typedef struct {
    const double *mean, *var; /* [H][D] */
} stats64;

static void project_bn_stats(const pkmo_model *M, const stats64 *S, int h, const float *x_b, double *qhat,
                             double *xhat)
{
    const int D = M->D;
    for (int f = 0; f < D; ++f) {
        const float *wrow = M->wq + ((int64_t)h * D + f) * D;
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += (double)wrow[d] * (double)x_b[d];
        const int64_t at = (int64_t)h * D + f;
        const double xh = (acc - S->mean[at]) / sqrt(S->var[at] + M->eps);
        if (xhat) xhat[f] = xh;
        qhat[f] = xh * (double)M->gamma[at] + (double)M->beta[at];
    }
}

/*
 * The lookup with batch statistics: steps 1-2 normalise with mean / var
 * (from pkmo_batch_stats), steps 3-7 are the same as pkmo_run's, at search
 * depth kk (out and w need kk == k).  Outputs as pkmo_run: out [B][D],
 * idx / top / w [B][H][kk], qhat [B][H][D]; any may be NULL.
 */
int pkmo_run_batch_stats(const pkmo_model *M, int64_t B, const float *x, int kk, const double *mean,
                         const double *var, double *out, int32_t *idx, double *top, double *w, double *qhat)
{
    if (!M || !x || !mean || !var || B < 1 || kk < 1 || kk > M->n) return -1;
    if ((out || w) && kk != M->k) return -1;
    if (out && !M->values) return -1;
    const int D = M->D, H = M->H, n = M->n;
    const stats64 S = {mean, var};
    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    double *s = (double *)malloc(sizeof(double) * 2 * (size_t)n);
    double *t0 = (double *)malloc(sizeof(double) * (size_t)kk), *t1 = (double *)malloc(sizeof(double) * (size_t)kk);
    int32_t *i0 = (int32_t *)malloc(sizeof(int32_t) * (size_t)kk), *i1 = (int32_t *)malloc(sizeof(int32_t) * (size_t)kk);
    double *tp = (double *)malloc(sizeof(double) * (size_t)kk), *wj = (double *)malloc(sizeof(double) * (size_t)kk);
    int32_t *fl = (int32_t *)malloc(sizeof(int32_t) * (size_t)kk);
    for (int64_t b = 0; b < B; ++b) {
        if (out)
            for (int d = 0; d < D; ++d)
                out[b * D + d] = 0.0;
        for (int h = 0; h < H; ++h) {
            project_bn_stats(M, &S, h, x + b * D, q, NULL);
            pkmo_half_scores(M, h, q, s);
            pkmo_topk_sorted(n, s, kk, t0, i0);
            pkmo_topk_sorted(n, &s[n], kk, t1, i1);
            pkmo_candidates_topk(n, kk, t0, i0, t1, i1, kk, tp, fl);
            const int64_t bh = b * H + h;
            if (qhat) memcpy(qhat + bh * D, q, sizeof(double) * (size_t)D);
            if (idx) memcpy(idx + bh * kk, fl, sizeof(int32_t) * (size_t)kk);
            if (top) memcpy(top + bh * kk, tp, sizeof(double) * (size_t)kk);
            if (w || out) {
                pkmo_softmax(kk, tp, wj);
                if (w) memcpy(w + bh * kk, wj, sizeof(double) * (size_t)kk);
                if (out) pkmo_gather_add(M, kk, fl, wj, out + b * D);
            }
        }
    }
    free(q); free(s); free(t0); free(t1); free(i0); free(i1); free(tp); free(wj); free(fl);
    return 0;
}

/*
 * Gradients of sum(dout * out) for the lookup with batch statistics.  The
 * statistics depend on every token, so BN's backward couples them: with
 * xhat = (q - mean)/sqrt(var + eps) and, per feature, the batch means
 *   m1 = (1/B) sum_b dq^_b ,   m2 = (1/B) sum_b dq^_b xhat_b ,
 *   dgamma = B m2 ,  dbeta = B m1 ,
 *   dq_b = gamma / sqrt(var + eps) * (dq^_b - m1 - xhat_b m2).
 * Everything else is the running-statistics backward (pkmo_backward).
 * Outputs as pkmo_backward (overwritten; any may be NULL).
 */
int pkmo_backward_batch_stats(const pkmo_model *M, int64_t B, const float *x, const float *dout, const double *mean,
                              const double *var, double *dx, double *dwq, double *dgamma, double *dbeta,
                              double *dsub, double *dval)
{
    if (!M || !x || !dout || !mean || !var || B < 1 || !M->values) return -1;
    const int D = M->D, H = M->H, n = M->n, k = M->k, half = D / 2;
    const int64_t N = (int64_t)n * n;
    const stats64 S = {mean, var};
    const size_t bhd = (size_t)B * H * D;
    double *qhat = (double *)malloc(sizeof(double) * bhd), *xhat = (double *)malloc(sizeof(double) * bhd);
    double *dqh = (double *)malloc(sizeof(double) * bhd);
    double *dtv = (double *)malloc(sizeof(double) * (size_t)B * H * k), *wv = (double *)malloc(sizeof(double) * (size_t)B * H * k);
    int32_t *rows = (int32_t *)malloc(sizeof(int32_t) * (size_t)B * H * k);
    double *s = (double *)malloc(sizeof(double) * 2 * (size_t)n);
    double *t0 = (double *)malloc(sizeof(double) * (size_t)k), *t1 = (double *)malloc(sizeof(double) * (size_t)k);
    int32_t *i0 = (int32_t *)malloc(sizeof(int32_t) * (size_t)k), *i1 = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    double *tp = (double *)malloc(sizeof(double) * (size_t)k), *g = (double *)malloc(sizeof(double) * (size_t)k);
    double *m1 = (double *)malloc(sizeof(double) * (size_t)H * D), *m2 = (double *)malloc(sizeof(double) * (size_t)H * D);
    if (!qhat || !xhat || !dqh || !dtv || !wv || !rows || !s || !t0 || !t1 || !i0 || !i1 || !tp || !g || !m1 || !m2)
        return -2;
    /* per token: forward again, then back to dq^ (as pkmo_backward) */
    for (int64_t b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const int64_t bh = b * H + h;
            double *qh = qhat + bh * D, *xh = xhat + bh * D, *dq_h = dqh + bh * D;
            double *dtj = dtv + bh * k, *wj = wv + bh * k;
            int32_t *rj = rows + bh * k;
            project_bn_stats(M, &S, h, x + b * D, qh, xh);
            pkmo_half_scores(M, h, qh, s);
            pkmo_topk_sorted(n, s, k, t0, i0);
            pkmo_topk_sorted(n, s + n, k, t1, i1);
            pkmo_candidates_topk(n, k, t0, i0, t1, i1, k, tp, rj);
            pkmo_softmax(k, tp, wj);
            double wg = 0.0;
            for (int j = 0; j < k; ++j) {
                double acc = 0.0;
                for (int d = 0; d < D; ++d)
                    acc += (double)dout[b * D + d] * value_at(M, rj[j], d);
                g[j] = acc;
                wg += wj[j] * acc;
            }
            for (int j = 0; j < k; ++j)
                dtj[j] = wj[j] * g[j] - wj[j] * wg;
            for (int d = 0; d < D; ++d)
                dq_h[d] = 0.0;
            for (int j = 0; j < k; ++j) {
                const float *c0 = M->subkeys + (((int64_t)h * 2 + 0) * n + rj[j] / n) * half;
                const float *c1 = M->subkeys + (((int64_t)h * 2 + 1) * n + rj[j] % n) * half;
                for (int d = 0; d < half; ++d) {
                    dq_h[d] += dtj[j] * (double)c0[d];
                    dq_h[half + d] += dtj[j] * (double)c1[d];
                }
            }
        }
    /* batch means of dq^ and dq^ xhat, in token order */
    for (int64_t hf = 0; hf < (int64_t)H * D; ++hf) {
        const int h = (int)(hf / D), f = (int)(hf % D);
        double a = 0.0, c = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            const int64_t at = (b * H + h) * D + f;
            a += dqh[at];
            c += dqh[at] * xhat[at];
        }
        m1[hf] = a / (double)B;
        m2[hf] = c / (double)B;
        if (dbeta) dbeta[hf] = a;
        if (dgamma) dgamma[hf] = c;
    }
    /* dq, then dx and dWq */
    if (dx)
        for (int64_t i = 0; i < B * D; ++i)
            dx[i] = 0.0;
    if (dwq)
        for (int64_t i = 0; i < (int64_t)H * D * D; ++i)
            dwq[i] = 0.0;
    for (int64_t b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int f = 0; f < D; ++f) {
                const int64_t hf = (int64_t)h * D + f, at = (b * H + h) * D + f;
                const double dq = (double)M->gamma[hf] / sqrt(var[hf] + M->eps) *
                                  (dqh[at] - m1[hf] - xhat[at] * m2[hf]);
                const float *wrow = M->wq + hf * D;
                for (int d = 0; d < D; ++d) {
                    if (dx) dx[b * D + d] += dq * (double)wrow[d];
                    if (dwq) dwq[hf * D + d] += dq * (double)x[b * D + d];
                }
            }
    /* subkeys and values: as with running statistics */
    if (dsub) {
        for (int64_t i = 0; i < (int64_t)H * 2 * n * half; ++i)
            dsub[i] = 0.0;
        for (int64_t b = 0; b < B; ++b)
            for (int h = 0; h < H; ++h) {
                const int64_t bh = b * H + h;
                for (int j = 0; j < k; ++j) {
                    const int r = rows[bh * k + j];
                    double *o0 = dsub + (((int64_t)h * 2 + 0) * n + r / n) * half;
                    double *o1 = dsub + (((int64_t)h * 2 + 1) * n + r % n) * half;
                    for (int d = 0; d < half; ++d) {
                        o0[d] += dtv[bh * k + j] * qhat[bh * D + d];
                        o1[d] += dtv[bh * k + j] * qhat[bh * D + half + d];
                    }
                }
            }
    }
    if (dval) {
        for (int64_t i = 0; i < N * D; ++i)
            dval[i] = 0.0;
        for (int64_t bh = 0; bh < B * H; ++bh)
            for (int j = 0; j < k; ++j)
                for (int d = 0; d < D; ++d)
                    dval[(int64_t)rows[bh * k + j] * D + d] += wv[bh * k + j] * (double)dout[(bh / H) * D + d];
    }
    free(qhat); free(xhat); free(dqh); free(dtv); free(wv); free(rows); free(s); free(t0); free(t1);
    free(i0); free(i1); free(tp); free(g); free(m1); free(m2);
    return 0;
}

/*
 * The running statistics a training-mode BatchNorm1d keeps for inference
 * (the module's running_mean / running_var buffers; "Product-Key Memory",
 * §Keeping the memory in use, and the code listing's BatchNorm1d): after a
 * batch of B >= 2 tokens with statistics mean / var (var biased, as the
 * normalisation uses it), each running value moves a fraction `momentum`
 * of the way to the batch's value; the variance it moves to is the
 * unbiased estimate var * B / (B - 1).
 *   rmean = (1 - momentum) rmean + momentum mean
 *   rvar  = (1 - momentum) rvar  + momentum var B / (B - 1)
 * count entries of each array, fp64, updated in place.  Returns 0, or -1
 * on bad arguments.
 */
int pkmo_running_update(int64_t count, int64_t B, double momentum, const double *mean, const double *var,
                        double *rmean, double *rvar)
{
    if (count < 0 || B < 2 || !(momentum >= 0.0 && momentum <= 1.0) || !mean || !var || !rmean || !rvar) return -1;
    const double unbias = (double)B / (double)(B - 1);
    for (int64_t i = 0; i < count; ++i) {
        rmean[i] = (1.0 - momentum) * rmean[i] + momentum * mean[i];
        rvar[i] = (1.0 - momentum) * rvar[i] + momentum * (var[i] * unbias);
    }
    return 0;
}

/* ------------------------------------------------------------ slot usage */

/* Slot usage ("Product-Key Memory", §Keeping the memory in use: a slot that
 * is never selected receives no gradient): counts[r] += the number of
 * entries of rows [M] equal to r, for r < N.  Returns 0, or -1 on bad
 * arguments (a row outside [0, N)). */
int pkmo_usage(int64_t M, const int32_t *rows, int64_t N, uint32_t *counts)
{
    if (M < 0 || N < 1 || (M > 0 && !rows) || !counts) return -1;
    for (int64_t i = 0; i < M; ++i) {
        if (rows[i] < 0 || rows[i] >= N) return -1;
        counts[rows[i]] += 1;
    }
    return 0;
}
