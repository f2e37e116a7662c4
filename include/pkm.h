/*
 * pkm.h -- C ABI of the MI355X (gfx950) product-key memory lookup library.
 *
 * The library computes the inference forward pass of a product-key memory
 * layer ("Product-Key Memory", aiwiki: §Factorising the key space and the
 * ProductKeyMemory module of its code listing), for H heads that share one
 * value table:
 *
 *   a1  q[b,h,:]  = Wq[h] . x[b,:]                          (Linear, no bias)
 *   a2  q^[b,h,:] = (q - mean[h]) / sqrt(var[h] + eps) * gamma[h] + beta[h]
 *                                       (BatchNorm1d with running statistics)
 *   a3  s[b,h,p,j] = q^[b,h, p*D/2 : (p+1)*D/2] . subkeys[h,p,j,:],  p = 0,1
 *   a4  each half keeps its k best subkeys (score desc, index asc)
 *   a5  the k*k candidates s0[i] + s1[j] with flat row i0[i]*n_keys + i1[j];
 *       the k best of them (score desc, flat index asc)
 *   a6  w = softmax of the k winning scores (no temperature)
 *   a7  out[b,:] = sum_h sum_j w[b,h,j] * scale[row] * values[row,:],
 *       row = idx[b,h,j]                (EmbeddingBag "sum", per-sample
 *                                        weights; scale = 1 for fp32 and
 *                                        bf16 tables)
 *
 * The winners are the exact top-k over all n_keys^2 concatenated keys (the
 * exactness argument of §Factorising the key space); a5-a7 follow the top-k
 * then softmax read of "Memory Retrieval Mechanisms: From Soft to
 * Efficient" (top-k section).  Scores, softmax and the accumulation run in
 * fp32; the value table may be fp32, bf16, or OCP FP8 E4M3 (E4M3FN), int8 or
 * int4 with one fp32 scale per row (the page's note that the table suits a
 * lower precision).
 *
 * Conventions for every call:
 *   - Pointers to tensors are DEVICE pointers, owned by the caller, row-major
 *     and contiguous, 16-byte aligned.  The library never frees or keeps them
 *     past the call.
 *   - Calls that take a stream (a hipStream_t, NULL = the default stream)
 *     only enqueue work: they return before it runs and never synchronise the
 *     device.  Inputs must stay alive and outputs untouched until the stream
 *     reaches that point.  Results are deterministic (bitwise) for identical
 *     inputs and configuration.  Apart from pkm_create and pkm_destroy, no
 *     call allocates, copies or clears memory with the runtime: each only
 *     launches kernels on its stream, so a caller may capture the calls in a
 *     HIP graph and replay them.
 *   - One context serves one stream at a time: the workspace is shared by
 *     every call on a context.  Use one context per concurrent stream.
 *   - Argument errors are detected on the host before anything is enqueued
 *     and return PKM_E_ARG (or PKM_E_UNSUPPORTED for shapes the kernels do
 *     not handle).  A failed launch returns PKM_E_DEVICE.  Errors raised by
 *     the device while the work runs surface at the caller's next
 *     synchronisation.  pkm_last_error() gives a thread-local description of
 *     the last error.  No C++ exception crosses this interface; nothing is
 *     printed unless the environment sets PKM_LOG=1.
 *   - Non-finite inputs give undefined (but memory-safe) results.
 */
#ifndef PKM_H
#define PKM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKM_OK = 0,
    PKM_E_ARG = 1,         /* invalid argument or configuration */
    PKM_E_UNSUPPORTED = 2, /* valid for the method, not handled by the kernels or this device */
    PKM_E_NOMEM = 3,       /* device allocation failed */
    PKM_E_DEVICE = 4       /* HIP runtime or launch error */
} pkm_status;

/* Storage of the value table.  The table is the whole memory cost of the
 * layer and suits a lower precision than the rest of the model ("Product-Key
 * Memory", the note after the code listing); every format is decoded to
 * fp32 in registers and accumulated in fp32. */
typedef enum {
    PKM_VALUES_F32 = 0,      /* float32 rows */
    PKM_VALUES_BF16 = 1,     /* bfloat16 rows (uint16 bit patterns) */
    PKM_VALUES_FP8_E4M3 = 2, /* OCP E4M3FN bytes, row r scaled by value_scale[r] */
    PKM_VALUES_INT8 = 3,     /* two's complement int8 codes, row r scaled by value_scale[r] */
    PKM_VALUES_INT4 = 4      /* two's complement int4 codes, two per byte (element 2i in the
                                low nibble of byte i, 2i+1 in the high one): a row is D/2
                                bytes; row r scaled by value_scale[r] */
} pkm_value_type;

typedef struct {
    int32_t dim;        /* D: model width.  The query is split in two halves
                           (chunk(2) in the listing), so D is even; the kernels
                           need D % 64 == 0 (PKM_E_UNSUPPORTED otherwise). */
    int32_t heads;      /* H >= 1 independent queries sharing one table */
    int32_t n_keys;     /* n: subkeys per half; the table has N = n*n rows.
                           2 <= n and n*n < 2^31. The select kernel handles
                           n <= 4096 (PKM_E_UNSUPPORTED above). */
    int32_t k;          /* winners per head: 1 <= k <= n (topk needs k <= n);
                           the kernels handle k <= 64 (PKM_E_UNSUPPORTED above) */
    int32_t value_type; /* a pkm_value_type */
    float bn_eps;       /* BatchNorm epsilon, > 0 (BatchNorm1d's default is 1e-5) */
    int64_t max_batch;  /* tokens per internal chunk: pkm_forward processes any
                           B in chunks of at most this many tokens; the
                           workspace is sized for one chunk.  >= 1. */
} pkm_config;

typedef struct {
    const float *wq;          /* [H, D, D]: Wq[h] row f = output feature f
                                 (nn.Linear weight layout), q = Wq[h] . x */
    const float *bn_mean;     /* [H, D] running mean */
    const float *bn_var;      /* [H, D] running variance, >= 0 */
    const float *bn_gamma;    /* [H, D] */
    const float *bn_beta;     /* [H, D] */
    const float *subkeys;     /* [H, 2, n, D/2]: half p of head h */
    const void *values;       /* [N, D] of value_type ([N, D/2] bytes for int4), N = n*n */
    const float *value_scale; /* [N] for the E4M3, int8 and int4 tables, else ignored
                                 (may be NULL).  Finite; for int4 tables
                                 |scale| < 2^100 (the decode scales the
                                 weight by 2^24) */
} pkm_params;

typedef struct pkm_ctx pkm_ctx; /* opaque; owned by the library */

/* Validates a configuration without touching any device.  PKM_OK, PKM_E_ARG
 * or PKM_E_UNSUPPORTED. */
pkm_status pkm_config_check(const pkm_config *cfg);

/* Bytes of device workspace pkm_create allocates for cfg (written to *bytes).
 * Touches no device. */
pkm_status pkm_workspace_bytes(const pkm_config *cfg, size_t *bytes);

/* Creates a context on the current HIP device: checks that the device is
 * gfx950 (PKM_E_UNSUPPORTED otherwise) and allocates the workspace
 * (PKM_E_NOMEM on failure): the normalised queries [max_batch, H, D] fp32,
 * the half scores [max_batch, H, 2, n] fp32, idx/weight buffers
 * [max_batch, H, k] for pkm_forward calls that pass NULL for them, and room
 * for one prepared copy of Wq and the subkeys (pkm_prepare; as many bytes
 * as the two arrays).  *out receives the context, or NULL on error. */
pkm_status pkm_create(const pkm_config *cfg, pkm_ctx **out);

/* Releases the workspace and the context.  NULL is a no-op.  The caller must
 * make sure no enqueued work still uses the context. */
void pkm_destroy(pkm_ctx *ctx);

/* The whole lookup (a1-a7) for B >= 0 tokens.
 *   x        [B, D] fp32 input
 *   out      [B, D] fp32, overwritten with the weighted row sums (a7)
 *   idx      [B, H, k] int32 winning flat rows in (score desc, flat index
 *            asc) order, or NULL to keep them in the workspace
 *   weights  [B, H, k] fp32 softmax weights in the same order, or NULL
 *   stream   hipStream_t (NULL = default stream)
 * B == 0 enqueues nothing.  out must not alias any input. */
pkm_status pkm_forward(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *out, int32_t *idx,
                       float *weights, void *stream);

/* Forms of prepared parameters (pkm_prepare). */
typedef enum {
    /* Wq and the subkeys split into fp16 pieces: bit for bit the unprepared
     * results. */
    PKM_PREPARE_SPLIT = 0,
    /* Steps a1-a3 folded into one matrix per half of a head, for lookups
     * with fixed batch-norm statistics (all three steps are linear maps):
     * for head h, half p and subkey j,
     *   s[h,p,j] = x . M[h,p,j,:] + bias[h,p,j],
     *   M[h,p,j,i] = sum_f subkeys[h,p,j,f] m[f] Wq[h][f0+f, i],
     *   bias[h,p,j] = sum_f subkeys[h,p,j,f] (beta[f0+f] - mean[f0+f] m[f]),
     * m[f] = gamma[f0+f] / sqrt(var[f0+f] + eps), f0 = p D/2, f < D/2; the
     * sums in fp64, rounded once to fp32.  The lookup then runs one
     * contraction of x (2 B D 2H n flop) in place of the projection and the
     * scoring (2 B H D (D + n)), with no q^ between them.  The scores agree
     * with the unfolded ones to fp32 accuracy, not bit for bit.  Applies
     * when n_keys <= D (otherwise folding adds work and PKM_PREPARE_SPLIT's
     * form is prepared instead). */
    PKM_PREPARE_FOLD = 1
} pkm_prepare_form;

/* Prepares the parameters that are the same for every call, once, in the
 * form the contractions read, and keeps them in the context:
 *   PKM_PREPARE_SPLIT: Wq (a1) and the subkeys (a3), each row scaled by a
 *     power of two and split into two fp16 pieces in the contractions'
 *     staging order (see gemm_f32.hip).  pkm_forward, pkm_forward_stage,
 *     pkm_forward_train and pkm_half_scores on this context then read that
 *     copy instead of p->wq and p->subkeys whenever they are given these
 *     same two pointers (no per-call exponent pass over the weights, no
 *     splitting of B in the tiles), with bit for bit the unprepared
 *     results.  Uses p->wq and p->subkeys.
 *   PKM_PREPARE_FOLD: the folded matrix and shift (see pkm_prepare_form),
 *     used by pkm_forward, pkm_forward_stage and pkm_half_scores whenever
 *     they are given the same wq, subkeys, bn_mean, bn_var, bn_gamma and
 *     bn_beta pointers.  pkm_forward_train needs the projection itself and
 *     reads p as given.  Uses those six arrays.
 * The copy stands for the arrays' contents at this call: a caller that
 * changes any of them (an optimiser step, new running statistics) must call
 * pkm_prepare again, or pkm_prepare(ctx, NULL, 0, stream) to drop the copy.
 * Calls with other pointers are unaffected.  Like every call it only
 * enqueues on `stream`; forward calls on another stream must wait for it.
 * PKM_E_ARG for a NULL or misaligned array or an unknown form; on any error
 * nothing stays prepared. */
pkm_status pkm_prepare(pkm_ctx *ctx, const pkm_params *p, int form, void *stream);

/* Steps a1-a3 only, straight from the tokens: scores [B, H, 2, n] fp32 (the
 * half scores the selection ranks), from x [B, D] and p (Wq, the batch-norm
 * arrays and the subkeys; the folded form where pkm_prepare made one for
 * them), in chunks of max_batch through the context's workspace. */
pkm_status pkm_half_scores(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *scores,
                           void *stream);

/* The whole lookup (a1-a7) without a context and without allocating: for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that must not call hipMalloc, harnesses that forbid it).
 * Same arguments, results and errors as pkm_forward, with cfg in place of a
 * context.  The workspace is a static device array of 128 MiB inside the
 * library, one per GPU, held from the first call on that GPU until the
 * process ends; nothing is allocated or freed by this call, by the runtime
 * or by any library.
 *   cfg->max_batch  the most tokens per chunk; the call works in the largest
 *                   chunk (at most this) whose workspace fits the array (a
 *                   multiple of 256 tokens from 256 on; about 2560 tokens
 *                   at D = 1024, H = 4, n_keys = 1024)
 * PKM_E_UNSUPPORTED if the workspace of a single token does not fit the
 * array, or if the device is not gfx950 (checked on the first call on each
 * device).  Every call on one GPU uses that GPU's single array, which keeps
 * the last call's contents (each call rewrites what it reads): calls that
 * overlap on one GPU, on different streams or from different threads,
 * race and give undefined results; serialise them. */
pkm_status pkm_forward_noalloc(const pkm_config *cfg, const pkm_params *p, int64_t B, const float *x, float *out,
                               int32_t *idx, float *weights, void *stream);

/* For profiling and for callers that interleave other work: one stage of
 * pkm_forward's own launches, for B <= max_batch tokens (one chunk), the
 * intermediate results kept in the context's workspace between stages.
 *   stage 0  the row exponents of x, Wq and the subkeys (the powers of two
 *            the contractions scale rows by) and clearing q^'s per-half
 *            maxima
 *   stage 1  a1-a2, the projection with BN (recording q^'s maxima)
 *   stage 2  a3, the subkey scoring
 *   stage 3  a4-a7, the selection and the gather (as pkm_select_gather)
 * With a folded form prepared for p (PKM_PREPARE_FOLD): stage 0 the row
 * exponents of x, stage 1 a1-a3 as one contraction, stage 2 nothing.
 * Stages 0, 1, 2, 3 in order on one stream, with the same arguments and no
 * other call on the context in between, do exactly what pkm_forward does
 * for those tokens, with the same results.  Arguments as pkm_forward; a
 * stage reads only those it needs (x: stages 0-1; out, idx, weights:
 * stage 3).  PKM_E_ARG for a stage outside 0-3 or B > max_batch. */
pkm_status pkm_forward_stage(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *out, int32_t *idx,
                             float *weights, int stage, void *stream);

/* Steps a1-a2 only: qhat [B, H, D] fp32 = BN_h(Wq[h] . x[b]).  Uses wq and
 * the four BN arrays of p, and the context's workspace for the contraction's
 * row exponents (so, like pkm_forward, one stream per context at a time);
 * any B is done in chunks of max_batch. */
pkm_status pkm_query(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *qhat, void *stream);

/* Step a3 only: scores [B, H, 2, n] fp32 from qhat [B, H, D] and p->subkeys.
 * Uses the context's workspace for the contraction's row exponents. */
pkm_status pkm_score(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *qhat, float *scores,
                     void *stream);

/* Steps a4-a6 only: from scores [B, H, 2, n] fp32 write idx [B, H, k] int32
 * and weights [B, H, k] fp32 (both required), as pkm_forward orders them.
 * No workspace is used. */
pkm_status pkm_select(pkm_ctx *ctx, int64_t B, const float *scores, int32_t *idx, float *weights, void *stream);

/* Step a7 only: out [B, D] fp32 = sum over the rows_per_token (row, weight)
 * pairs of token b of weight * scale[row] * values[row, :].  idx and weights
 * are [B, rows_per_token] (pkm_forward uses rows_per_token = H * k, the
 * [B, H, k] layout).  Rows should lie in [0, N); the kernel clamps a row
 * outside that range into it (memory-safe, meaningless result).  Uses
 * p->values and p->value_scale only. */
pkm_status pkm_gather(pkm_ctx *ctx, const pkm_params *p, int64_t B, int32_t rows_per_token, const int32_t *idx,
                      const float *weights, float *out, void *stream);

/* Steps a4-a7 from scores [B, H, 2, n] fp32: the selection and the gather
 * ("Product-Key Memory", §Factorising the key space and the code listing's
 * forward, from the subkey scores on), out [B, D] fp32 overwritten; idx and
 * weights [B, H, k] written as pkm_select writes them, or both NULL.  The
 * same results, bit for bit, as pkm_select followed by pkm_gather, and what
 * pkm_forward runs after the scoring: for n_keys 1024 or 2048 with H * k <=
 * 512 and table rows longer than 512 bytes one fused kernel (a workgroup
 * per token selects every head, then gathers the token's rows); otherwise
 * the two kernels (idx / weights NULL then use the context's workspace).  Uses p->values and p->value_scale. */
pkm_status pkm_select_gather(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *scores, int32_t *idx,
                             float *weights, float *out, void *stream);

/* Flat exact search: the brute-force search the product search replaces
 * ("Product-Key Memory", §Factorising the key space: the product search
 * returns exactly the k best of all N = n^2 concatenated keys, with 2n
 * subkey scores instead of N key scores).  For each token b and head h,
 * every concatenated key key(a, c) = [subkeys[h,0,a,:]; subkeys[h,1,c,:]]
 * is scored against qhat[b,h,:] with one D-long fp32 dot product (the
 * product structure is not used), and the k best are written:
 *   qhat  [B, H, D] fp32 normalised queries (pkm_query's output)
 *   idx   [B, H, k] int32 flat rows a * n + c, in (score desc, flat index
 *         asc) order — the order pkm_forward uses
 *   top   [B, H, k] fp32 the scores of those keys
 * workspace is caller-owned device memory of at least
 * pkm_flat_workspace_bytes(cfg, B) bytes (16-byte aligned): it holds the
 * B * H * n^2 fp32 key scores, the contraction's row exponents, the
 * subkeys split into fp16 pieces, and the top-k's buffers (for n^2 > 4096:
 * the largest score of every group of 64 keys, the threshold derived from
 * them and per-row lists of the scores at or above it), so the call
 * allocates nothing.  Work: 2 * B * H * n^2 * D
 * flop.  B <= 65536; a smaller workspace is PKM_E_ARG. */
pkm_status pkm_flat_workspace_bytes(const pkm_config *cfg, int64_t B, size_t *bytes);
pkm_status pkm_flat_search(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *qhat, void *workspace,
                           size_t workspace_bytes, int32_t *idx, float *top, void *stream);

/* Gradients written by pkm_backward.  Parameter gradients are ADDED to what
 * the buffers hold (zero them for one batch's gradient); dx is overwritten.
 * Any member may be NULL to skip that gradient (dbn_gamma and dbn_beta go
 * together).  The float buffers are fp32 device memory, 16-byte aligned.
 *
 * The value gradient comes in one of two forms.  dvalues is the dense one.
 * The sparse one (the last three members, all set or all NULL, dvalues then
 * NULL) holds only the rows some winner selected: a batch touches at most
 * B*H*k of the n_keys^2 rows, and those rows are the only ones that move
 * ("Product-Key Memory", §Keeping the memory in use: unselected slots get
 * no gradient).  With U the number of distinct rows in idx:
 *   dvalues_rows    [U] int32, the rows in increasing order;
 *   dvalues_sparse  [U, D]: row u holds the gradient of row dvalues_rows[u]
 *                   (overwritten, not added to);
 *   dvalues_count   one int64 in device memory, set to U (0 for B = 0;
 *                   the other two may then be NULL).
 * The caller sizes the first two for min(n_keys^2, B*H*k) rows; entries
 * beyond U are left as they were.  The sparse form needs B <= max_batch.
 * Scattered into zeros it equals the dense form bit for bit. */
typedef struct {
    float *dx;        /* [B, D] */
    float *dwq;       /* [H, D, D] */
    float *dbn_gamma; /* [H, D] */
    float *dbn_beta;  /* [H, D] */
    float *dsubkeys;  /* [H, 2, n_keys, D/2] */
    float *dvalues;   /* [n_keys^2, D]: w.r.t. the dequantised value rows
                         (scale[row] * decoded value for the scaled
                         tables: E4M3, int8, int4) */
    int32_t *dvalues_rows;  /* sparse form, see above */
    float *dvalues_sparse;
    int64_t *dvalues_count;
} pkm_grads;

/* Bytes of caller-owned device workspace pkm_backward needs for cfg (it
 * works through the batch in chunks of cfg->max_batch tokens). */
pkm_status pkm_backward_workspace_bytes(const pkm_config *cfg, size_t *bytes);

/* The backward direction: gradients of a loss L given dout = dL/dout [B, D]
 * fp32, through steps a7 -> a1 for the winners a forward call selected
 * (idx, weights [B, H, k] as pkm_forward wrote them for the same x and p).
 * The top-k selections pass gradient only to the winning scores ("Product-
 * Key Memory", code listing: topk values feed the softmax, its indices only
 * select), and BN uses its running statistics, as in the forward:
 *   dL/dw_j = dout_b . V[r_j];  softmax backward to the winning scores;
 *   each score s_0[i0] + s_1[i1] passes its gradient to both half scores;
 *   half scores -> q^ (subkey rows) and -> subkeys (q^ halves);
 *   q^ -> dgamma, dbeta and q;  q -> dWq (outer products with x) and dx;
 *   dV[r_j] += w_j dout_b.
 * Every sum runs in a fixed order: results are bitwise reproducible.
 * workspace: caller-owned, >= pkm_backward_workspace_bytes(cfg) bytes,
 * 16-byte aligned; the call allocates nothing. */
pkm_status pkm_backward(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, const int32_t *idx,
                        const float *weights, const float *dout, const pkm_grads *grads, void *workspace,
                        size_t workspace_bytes, void *stream);

/* The lookup with training-mode BatchNorm: the query is normalised with the
 * statistics of this batch ("Product-Key Memory", §Keeping the memory in
 * use: batch normalisation of the queries), the one step that couples the
 * tokens.  Per head h and feature f over the B tokens: mean and biased
 * variance of q = Wq[h] . x_b (one pass: per chunk of 64 tokens the mean
 * and the sum of squared deviations, the chunks merged pairwise in a fixed
 * order), then
 * q^ = (q - mean) / sqrt(var + eps) * gamma + beta; steps a3-a7 as in
 * pkm_forward.  2 <= B <= max_batch (one pass over the whole batch).
 *   batch_mean, batch_var  [H, D] fp32, written (biased variance)
 *   running_mean, running_var  [H, D] fp32 or both NULL: updated as
 *       r = (1 - momentum) r + momentum s, the variance unbiased (s * B/(B-1))
 *   momentum  in [0, 1] (BatchNorm1d's default is 0.1)
 * p->bn_mean and p->bn_var are not read.  Other arguments as pkm_forward. */
pkm_status pkm_forward_batch_stats(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *out,
                                   int32_t *idx, float *weights, float *batch_mean, float *batch_var,
                                   float *running_mean, float *running_var, float momentum, void *stream);

/* For training with running-statistics BN: pkm_forward, plus the
 * projection before BN, which the backward needs again.
 *   q  [B, H, D] fp32, overwritten with q[b,h,:] = Wq[h] . x[b,:] (a1, before
 *      a2), 16-byte aligned, not aliasing any other argument
 * out, idx and weights are bitwise those of pkm_forward; the extra stores
 * cost about 40 us per 4,096 tokens at D = 1024, H = 4.  Errors as
 * pkm_forward (q NULL or misaligned: PKM_E_ARG). */
pkm_status pkm_forward_train(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *out, int32_t *idx,
                             float *weights, float *q, void *stream);

/* pkm_backward with the projection before BN taken from q (as
 * pkm_forward_train wrote it for the same x and p) instead of computed
 * again: one contraction less (about 0.1 ms per 4,096 tokens at D = 1024,
 * H = 4).  With that q the gradients are bitwise those of pkm_backward.
 * Other arguments, workspace and errors as pkm_backward (q NULL or
 * misaligned: PKM_E_ARG). */
pkm_status pkm_backward_with_q(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, const float *q,
                               const int32_t *idx, const float *weights, const float *dout, const pkm_grads *grads,
                               void *workspace, size_t workspace_bytes, void *stream);

/* pkm_backward for a forward with batch statistics (batch_mean, batch_var
 * as pkm_forward_batch_stats wrote them).  BN's backward then couples the
 * tokens: with xhat = (q - mean)/sqrt(var + eps) and the batch sums
 * sb = sum_b dq^_b, sg = sum_b dq^_b xhat_b,
 *   dq_b = gamma / sqrt(var + eps) * (dq^_b - sb/B - xhat_b sg/B),
 * dgamma += sg, dbeta += sb.  2 <= B <= max_batch.  p->bn_mean and
 * p->bn_var are not read.  Other arguments as pkm_backward. */
pkm_status pkm_backward_batch_stats(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x,
                                    const int32_t *idx, const float *weights, const float *dout,
                                    const float *batch_mean, const float *batch_var, const pkm_grads *grads,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* Slot usage ("Product-Key Memory", §Keeping the memory in use: a slot that
 * is never selected receives no gradient, and usage can collapse to a few
 * thousand live rows out of a million): counts[r] += the number of entries
 * of idx [B, rows_per_token] (e.g. pkm_forward's [B, H, k]) equal to r.
 * counts [n_keys^2] uint32, caller-owned, accumulated across calls.  Rows
 * outside [0, N) are clamped into it (memory-safe).  Integer counts: the
 * result does not depend on the order of the updates. */
pkm_status pkm_usage(pkm_ctx *ctx, int64_t B, int32_t rows_per_token, const int32_t *idx, uint32_t *counts,
                     void *stream);

/* A static description of a status code. */
const char *pkm_status_str(pkm_status s);

/* Thread-local description of the last error returned to this thread (""
 * if none). */
const char *pkm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKM_H */
