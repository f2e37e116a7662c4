// Host side of the C ABI declared in include/pkm.h: argument validation,
// workspace, batch chunking and the launch sequence on the caller's stream.
#include "pkm.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "pkm_internal.h"

struct pkm_ctx {
    pkm_config cfg;
    int device;
    void *workspace;
    float *qhat;     // [max_batch, H, D]
    float *scores;   // [max_batch, H, 2, n]
    int32_t *idx;    // [max_batch, H, k]
    float *weights;  // [max_batch, H, k]
    float *stat_part; // batch statistics: chunk means and squared deviations [2, chunks, H * D]
    int32_t *gemm_exp; // row exponents of the GEMM operands
    int64_t gemm_exp_ints;
    uint32_t *qmax;    // largest |q^| per (token, half of a head) [max_batch, 2H], float bits
    int32_t *sub_exp;  // row exponents of the subkeys [2H, n]
    // Prepared weights (pkm_prepare): the row exponents and fp16 pieces of
    // Wq and of the subkeys, and the arrays they were made from (NULL:
    // nothing prepared).
    int32_t *prep_wq_exp;   // [H * D]
    int32_t *prep_sub_exp;  // [2H * n]
    void *prep_wq;
    void *prep_sub;
    const float *prep_wq_src, *prep_sub_src;
    // Folded form (pkm_prepare with PKM_PREPARE_FOLD, n_keys <= D): the
    // matrix of the folded projection, batch-norm and subkeys as fp16 pieces
    // with its row exponents, the per-key shift, and the batch-norm arrays
    // it was made from.
    int prep_mode;  // 0 nothing, 1 split, 2 folded
    int32_t *fold_exp;  // [2H * n]
    float *fold_bias;   // [2H * n]
    void *fold_pieces;
    void *x_pieces;  // a chunk of x as fp16 pieces, for the folded contraction
    const float *prep_bn_src[4];  // mean, var, gamma, beta
};

namespace {

thread_local std::string g_last_error;

// Launch grids are sized from B (one wave per token-slice or per token-head):
// keep every grid well inside 2^31 workgroups.
constexpr int64_t kMaxBatch = (int64_t)1 << 30;

pkm_status fail(pkm_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    if (const char *log = getenv("PKM_LOG"); log && log[0] == '1') fprintf(stderr, "pkm: %s\n", buf);
    return s;
}

pkm_status ok()
{
    g_last_error.clear();
    return PKM_OK;
}

bool log_on()
{
    const char *log = getenv("PKM_LOG");
    return log && log[0] == '1';
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Row exponents the forward's contractions need for a chunk of mb tokens:
// the query projection (mb + H*D rows) or the subkey scoring (2H (mb + n)).
int64_t forward_exp_ints(const pkm_config &c)
{
    const int64_t q = c.max_batch + (int64_t)c.heads * c.dim, sc = 2 * (int64_t)c.heads * (c.max_batch + c.n_keys);
    return q > sc ? q : sc;
}

// Workspace pieces for one chunk of c.max_batch tokens: q^, scores, idx,
// weights, the batch statistics' partial sums (only with batch_stats), the
// GEMM row exponents, q^'s per-half maxima and the subkeys' row exponents;
// then (only with prepared) the prepared weights: Wq's and the subkeys' row
// exponents and fp16 pieces.  False on size overflow.
constexpr int kPieces = 16;
bool workspace_layout(const pkm_config &c, size_t sizes[kPieces], bool batch_stats = true, bool prepared = true)
{
    const double mb = (double)c.max_batch;
    const double total = mb * c.heads * ((double)c.dim + 2.0 * c.n_keys + 2.0 * c.k) * 4.0;
    if (total > 1.0e15) return false;
    const size_t m = (size_t)c.max_batch, H = (size_t)c.heads;
    sizes[0] = round_up(m * H * (size_t)c.dim * sizeof(float));
    sizes[1] = round_up(m * H * 2 * (size_t)c.n_keys * sizeof(float));
    sizes[2] = round_up(m * H * (size_t)c.k * sizeof(int32_t));
    sizes[3] = round_up(m * H * (size_t)c.k * sizeof(float));
    sizes[4] = batch_stats ? round_up((size_t)pkm::stat_part_floats(c.max_batch, H * c.dim) * sizeof(float)) : 0;
    sizes[5] = round_up((size_t)forward_exp_ints(c) * sizeof(int32_t));
    sizes[6] = round_up(m * 2 * H * sizeof(uint32_t));
    sizes[7] = round_up(2 * H * (size_t)c.n_keys * sizeof(int32_t));
    sizes[8] = prepared ? round_up(H * (size_t)c.dim * sizeof(int32_t)) : 0;
    sizes[9] = prepared ? sizes[7] : 0;
    sizes[10] = prepared ? round_up((size_t)pkm::gemm_presplit_bytes(c.heads * c.dim, c.dim, 1)) : 0;
    sizes[11] = prepared ? round_up((size_t)pkm::gemm_presplit_bytes(c.n_keys, c.dim / 2, 2 * c.heads)) : 0;
    // the folded form, where it applies (n_keys <= D); pkm_prepare builds
    // its fp32 matrix in pieces 10-11 first (as large: n_keys <= D)
    const bool fold = prepared && c.n_keys <= c.dim;
    sizes[12] = fold ? round_up(2 * H * (size_t)c.n_keys * sizeof(int32_t)) : 0;
    sizes[13] = fold ? round_up(2 * H * (size_t)c.n_keys * sizeof(float)) : 0;
    sizes[14] = fold ? round_up((size_t)pkm::gemm_presplit_bytes(2 * c.heads * c.n_keys, c.dim, 1)) : 0;
    sizes[15] = fold ? round_up((size_t)pkm::gemm_presplit_bytes((int)c.max_batch, c.dim, 1)) : 0;
    return true;
}

// Points the context's workspace pieces into w (laid out by
// workspace_layout).
void assign_workspace(pkm_ctx *ctx, char *w, const size_t sizes[kPieces])
{
    char *piece[kPieces];
    piece[0] = w;
    for (int i = 1; i < kPieces; ++i) piece[i] = piece[i - 1] + sizes[i - 1];
    ctx->workspace = w;
    ctx->qhat = reinterpret_cast<float *>(piece[0]);
    ctx->scores = reinterpret_cast<float *>(piece[1]);
    ctx->idx = reinterpret_cast<int32_t *>(piece[2]);
    ctx->weights = reinterpret_cast<float *>(piece[3]);
    ctx->stat_part = sizes[4] ? reinterpret_cast<float *>(piece[4]) : nullptr;
    ctx->gemm_exp = reinterpret_cast<int32_t *>(piece[5]);
    ctx->gemm_exp_ints = (int64_t)(sizes[5] / sizeof(int32_t));
    ctx->qmax = reinterpret_cast<uint32_t *>(piece[6]);
    ctx->sub_exp = reinterpret_cast<int32_t *>(piece[7]);
    ctx->prep_wq_exp = reinterpret_cast<int32_t *>(piece[8]);
    ctx->prep_sub_exp = reinterpret_cast<int32_t *>(piece[9]);
    ctx->prep_wq = piece[10];
    ctx->prep_sub = piece[11];
    ctx->prep_wq_src = ctx->prep_sub_src = nullptr;
    ctx->prep_mode = 0;
    ctx->fold_exp = sizes[12] ? reinterpret_cast<int32_t *>(piece[12]) : nullptr;
    ctx->fold_bias = sizes[13] ? reinterpret_cast<float *>(piece[13]) : nullptr;
    ctx->fold_pieces = sizes[14] ? piece[14] : nullptr;
    ctx->x_pieces = sizes[15] ? piece[15] : nullptr;
    for (auto &b : ctx->prep_bn_src) b = nullptr;
}

pkm_status check_config(const pkm_config *c)
{
    if (!c) return fail(PKM_E_ARG, "config is NULL");
    if (c->dim < 2 || (c->dim & 1)) return fail(PKM_E_ARG, "dim must be even and >= 2 (got %d)", c->dim);
    if (c->heads < 1) return fail(PKM_E_ARG, "heads must be >= 1 (got %d)", c->heads);
    if (c->n_keys < 2) return fail(PKM_E_ARG, "n_keys must be >= 2 (got %d)", c->n_keys);
    if ((int64_t)c->n_keys * c->n_keys >= ((int64_t)1 << 31))
        return fail(PKM_E_ARG, "n_keys^2 must be < 2^31 (got n_keys = %d)", c->n_keys);
    if (c->k < 1 || c->k > c->n_keys) return fail(PKM_E_ARG, "k must be in [1, n_keys] (got %d)", c->k);
    if (c->value_type < PKM_VALUES_F32 || c->value_type > PKM_VALUES_INT4)
        return fail(PKM_E_ARG, "unknown value_type %d", c->value_type);
    if (!(c->bn_eps > 0.0f) || !(c->bn_eps < 1.0e30f)) return fail(PKM_E_ARG, "bn_eps must be finite and > 0");
    if (c->max_batch < 1 || c->max_batch > kMaxBatch || c->max_batch * c->heads > ((int64_t)1 << 31))
        return fail(PKM_E_ARG, "max_batch must be in [1, 2^30] with max_batch * heads <= 2^31");
    if ((int64_t)c->heads * c->dim >= ((int64_t)1 << 30)) return fail(PKM_E_ARG, "heads * dim too large");
    size_t sizes[kPieces];
    if (!workspace_layout(*c, sizes)) return fail(PKM_E_ARG, "workspace size overflows");
    if (c->dim % 64 != 0) return fail(PKM_E_UNSUPPORTED, "dim must be a multiple of 64 (got %d)", c->dim);
    if (c->k > 64) return fail(PKM_E_UNSUPPORTED, "k > 64 is not supported (got %d)", c->k);
    if (c->n_keys > 4096) return fail(PKM_E_UNSUPPORTED, "n_keys > 4096 is not supported (got %d)", c->n_keys);
    return ok();
}

pkm_status check_ctx(const pkm_ctx *ctx)
{
    if (!ctx) return fail(PKM_E_ARG, "context is NULL");
    return PKM_OK;
}

pkm_status check_batch(const pkm_config &c, int64_t B)
{
    if (B < 0) return fail(PKM_E_ARG, "B must be >= 0 (got %lld)", (long long)B);
    if (B > kMaxBatch || B * c.heads > ((int64_t)1 << 31))
        return fail(PKM_E_ARG, "B = %lld is too large for one call (B <= 2^30 and B * heads <= 2^31)", (long long)B);
    return PKM_OK;
}

pkm_status need(const void *p, const char *name)
{
    if (!p) return fail(PKM_E_ARG, "%s is NULL", name);
    if (!aligned16(p)) return fail(PKM_E_ARG, "%s is not 16-byte aligned", name);
    return PKM_OK;
}

pkm_status check_query_params(const pkm_params *p)
{
    if (!p) return fail(PKM_E_ARG, "params is NULL");
    pkm_status s;
    if ((s = need(p->wq, "wq")) || (s = need(p->bn_mean, "bn_mean")) || (s = need(p->bn_var, "bn_var")) ||
        (s = need(p->bn_gamma, "bn_gamma")) || (s = need(p->bn_beta, "bn_beta")))
        return s;
    return PKM_OK;
}

pkm_status check_value_params(const pkm_config &c, const pkm_params *p)
{
    if (!p) return fail(PKM_E_ARG, "params is NULL");
    pkm_status s;
    if ((s = need(p->values, "values"))) return s;
    if (c.value_type >= PKM_VALUES_FP8_E4M3 && (s = need(p->value_scale, "value_scale"))) return s;
    return PKM_OK;
}

pkm_status launched(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(PKM_E_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
    return PKM_OK;
}

pkm::GemmArgs query_args(const pkm_config &c, const pkm_params *p, int64_t B, const float *x, float *qhat,
                         int32_t *exp_ws, int64_t exp_ints)
{
    pkm::GemmArgs a{};
    a.exp_ws = exp_ws;
    a.exp_ws_ints = exp_ints;
    a.A = x;
    a.lda = c.dim;
    a.strideA = 0;
    a.B = p->wq;
    a.ldb = c.dim;
    a.strideB = 0;
    a.C = qhat;
    a.ldc = (int64_t)c.heads * c.dim;
    a.strideC = 0;
    a.M = (int)B;
    a.N = c.heads * c.dim;
    a.K = c.dim;
    a.batch = 1;
    a.bn_mean = p->bn_mean;
    a.bn_var = p->bn_var;
    a.bn_gamma = p->bn_gamma;
    a.bn_beta = p->bn_beta;
    a.bn_eps = c.bn_eps;
    return a;
}

pkm::GemmArgs score_args(const pkm_config &c, const pkm_params *p, int64_t B, const float *qhat, float *scores,
                         int32_t *exp_ws, int64_t exp_ints)
{
    const int half = c.dim / 2;
    pkm::GemmArgs a{};
    a.exp_ws = exp_ws;
    a.exp_ws_ints = exp_ints;
    a.A = qhat;  // head h, half p starts at column (2h + p) * D/2
    a.lda = (int64_t)c.heads * c.dim;
    a.strideA = half;
    a.B = p->subkeys;  // [2H][n][D/2]
    a.ldb = half;
    a.strideB = (int64_t)c.n_keys * half;
    a.C = scores;  // [B][2H][n]
    a.ldc = (int64_t)2 * c.heads * c.n_keys;
    a.strideC = c.n_keys;
    a.M = (int)B;
    a.N = c.n_keys;
    a.K = half;
    a.batch = 2 * c.heads;
    a.stream_out = true;  // read once, by the select
    return a;
}

// In chunks of max_batch tokens: the context's row-exponent workspace is
// sized for one.  With qmax, the projection also records the largest |q^|
// of every (token, half of a head) there and computes the subkeys' row
// exponents in its pre-pass, and the scoring takes its row exponents from
// both instead of reading q^ and the subkeys once more (no pre-pass).
pkm_status run_query(const pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *qhat,
                     uint32_t *qmax, hipStream_t st)
{
    const pkm_config &c = ctx->cfg;
    for (int64_t b0 = 0; b0 < B; b0 += c.max_batch) {
        const int64_t nb = B - b0 < c.max_batch ? B - b0 : c.max_batch;
        pkm::GemmArgs a = query_args(c, p, nb, x + b0 * c.dim, qhat + b0 * (int64_t)c.heads * c.dim, ctx->gemm_exp,
                                     ctx->gemm_exp_ints);
        if (qmax) {
            a.row_seg_max = qmax;
            a.seg_cols = c.dim / 2;
            a.zero_ptr = qmax;
            a.zero_n = nb * 2 * c.heads;
            // the subkeys' row exponents for the scoring, in the same pre-pass
            a.extra_exp.base = p->subkeys;
            a.extra_exp.rows_per_batch = c.n_keys;
            a.extra_exp.batch = 2 * c.heads;
            a.extra_exp.stride = (int64_t)c.n_keys * (c.dim / 2);
            a.extra_exp.ld = c.dim / 2;
            a.extra_exp.K = c.dim / 2;
            a.extra_exp.out = ctx->sub_exp;
        }
        if (pkm_status s = launched(pkm::launch_gemm_nt_f32(a, st), "query projection")) return s;
    }
    return PKM_OK;
}

pkm_status run_score(const pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *qhat, float *scores,
                     const uint32_t *qmax, hipStream_t st)
{
    const pkm_config &c = ctx->cfg;
    for (int64_t b0 = 0; b0 < B; b0 += c.max_batch) {
        const int64_t nb = B - b0 < c.max_batch ? B - b0 : c.max_batch;
        pkm::GemmArgs a = score_args(c, p, nb, qhat + b0 * (int64_t)c.heads * c.dim,
                                     scores + b0 * (int64_t)2 * c.heads * c.n_keys, ctx->gemm_exp, ctx->gemm_exp_ints);
        if (qmax) {
            a.a_rowmax = qmax;
            a.a_rowmax_ld = 2 * c.heads;
            a.b_exp_given = ctx->sub_exp;
        }
        if (pkm_status s = launched(pkm::launch_gemm_nt_f32(a, st), "subkey scoring")) return s;
    }
    return PKM_OK;
}

// Flat search workspace for B tokens: key scores [B, H, n^2] fp32, the two
// top-k merge buffers of packed keys, the contraction's row exponents, and
// for rows of more than 4096 keys the threshold's pieces: group maxima
// [B, H, G] (G = ceil(n^2 / 64)), theta's top-k [B, H, k] (indices, scores),
// the list counts [B, H] and the lists [B, H, kFlatListCap] of packed keys.
// The merge buffers serve the top-k over rows of G group maxima then, else
// over the n^2 scores.  Last, the subkeys split into fp16 pieces for the
// contraction (H * 2 sets of n rounded up to 32 rows, D/2 * 4 bytes each).
// False if B is out of range.
constexpr int64_t kFlatMaxBatch = 65536;
constexpr int kFlatPieces = 10;
constexpr int64_t kFlatDirectMax = 4096;  // longest row topped without a threshold
bool flat_layout(const pkm_config &c, int64_t B, size_t sizes[kFlatPieces])
{
    if (B < 0 || B > kFlatMaxBatch) return false;
    const int64_t rows = B * c.heads, N = (int64_t)c.n_keys * c.n_keys;
    if ((double)rows * (double)N * 4.0 > 1.0e15) return false;
    const bool threshold = N > kFlatDirectMax;
    const int64_t G = (N + 63) / 64;
    const int64_t keys = pkm::flat_topk_keys_per_row(threshold ? G : N, c.k);
    for (int i = 0; i < kFlatPieces; ++i) sizes[i] = 0;
    sizes[0] = round_up((size_t)(rows * N) * sizeof(float));
    sizes[1] = round_up((size_t)(rows * keys) * sizeof(uint64_t));
    sizes[2] = round_up((size_t)(rows * ((keys + 2047) / 2048) * c.k) * sizeof(uint64_t));
    sizes[3] = round_up((size_t)(c.heads * (B + 2 * (int64_t)c.n_keys)) * sizeof(int32_t));  // row exponents
    if (threshold) {
        sizes[4] = round_up((size_t)(rows * G) * sizeof(float));
        sizes[5] = round_up((size_t)(rows * c.k) * sizeof(int32_t));
        sizes[6] = round_up((size_t)(rows * c.k) * sizeof(float));
        sizes[7] = round_up((size_t)rows * sizeof(uint32_t));
        sizes[8] = round_up((size_t)(rows * pkm::kFlatListCap) * sizeof(uint64_t));
    }
    sizes[9] = round_up((size_t)c.heads * 2 * ((c.n_keys + 31) / 32) * 32 * (size_t)(c.dim / 2) * 4);
    return true;
}

size_t total_bytes(const size_t *sizes, int n)
{
    size_t t = 0;
    for (int i = 0; i < n; ++i) t += sizes[i];
    return t;
}

pkm::GemmArgs flat_args(const pkm_config &c, const pkm_params *p, int64_t B, const float *qhat, float *scores,
                        int32_t *exp_ws, int64_t exp_ints)
{
    const int half = c.dim / 2;
    pkm::GemmArgs a{};
    a.exp_ws = exp_ws;
    a.exp_ws_ints = exp_ints;
    a.A = qhat;  // head h starts at column h * D
    a.lda = (int64_t)c.heads * c.dim;
    a.strideA = c.dim;
    a.B = p->subkeys;                               // first halves: [h][0][a][:]
    a.B2 = p->subkeys + (int64_t)c.n_keys * half;   // second halves: [h][1][c][:]
    a.ldb = half;
    a.strideB = (int64_t)c.n_keys * c.dim;          // one head's two subkey sets
    a.split_k = half;
    a.key_n = c.n_keys;
    a.C = scores;  // [B][H][n^2]
    a.ldc = (int64_t)c.heads * c.n_keys * c.n_keys;
    a.strideC = (int64_t)c.n_keys * c.n_keys;
    a.M = (int)B;
    a.N = c.n_keys * c.n_keys;
    a.K = c.dim;
    a.batch = c.heads;
    return a;
}

// Backward workspace for chunks of mb = max_batch tokens (mb32 = mb rounded
// up to 32, the GEMMs' K granularity).
constexpr int kBwdPieces = 18;
bool backward_layout(const pkm_config &c, size_t sizes[kBwdPieces])
{
    const size_t mb = (size_t)c.max_batch, mb32 = (mb + 31) / 32 * 32, H = (size_t)c.heads, D = (size_t)c.dim;
    const size_t HD = H * D, k = (size_t)c.k, n = (size_t)c.n_keys, N = n * n;
    const double total = (double)mb32 * (double)HD * 7.0 + 2.0 * H * n * mb32 + 4.0 * N +
                         (double)pkm::kMaxKSplits * ((double)HD * D + (double)mb * D);
    if (total * 4.0 > 1.0e15) return false;
    const size_t f = sizeof(float), u = sizeof(uint32_t);
    sizes[0] = round_up(mb * HD * f);       // q (before BN)
    sizes[1] = round_up(mb * H * k * f);    // dt
    sizes[2] = round_up(mb * HD * f);       // dq^
    sizes[3] = round_up(mb * HD * f);       // dq
    sizes[4] = round_up(HD * mb32 * f);     // dq transposed
    sizes[5] = round_up(D * mb32 * f);      // x transposed
    sizes[6] = round_up(D * HD * f);        // Wq transposed
    sizes[7] = round_up(2 * HD * f);        // this batch's sums of dq^ xhat and dq^
    sizes[8] = round_up(2 * H * n * mb32 * f);  // half-score gradients G
    sizes[9] = round_up((size_t)pkm::colsum_chunks((int64_t)mb) * HD * f);
    sizes[10] = sizes[9];
    sizes[11] = round_up(N * u);            // per-row counts
    sizes[12] = round_up(N * u);            // fill cursors
    sizes[13] = round_up(N * u);            // row offsets
    sizes[14] = round_up((size_t)pkm::scan_blocks((int)N) * u);
    sizes[15] = round_up(mb * H * k * u);   // occurrence lists
    // split-K partial products of the dWq and dx GEMMs
    sizes[16] = round_up((size_t)pkm::kMaxKSplits * (HD * D > mb * D ? HD * D : mb * D) * f);
    // row exponents of the GEMM operands: q recompute (mb + HD rows), dWq
    // (H (D + D)), dx (mb + D)
    const size_t e_q = mb + HD, e_w = H * 2 * D, e_x = mb + D;
    sizes[17] = round_up((e_q > e_w ? (e_q > e_x ? e_q : e_x) : (e_w > e_x ? e_w : e_x)) * sizeof(int32_t));
    return true;
}

pkm_status check_grads(const pkm_grads *g)
{
    if (!g) return fail(PKM_E_ARG, "grads is NULL");
    const void *ptrs[] = {g->dx, g->dwq, g->dbn_gamma, g->dbn_beta, g->dsubkeys, g->dvalues, g->dvalues_sparse};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return fail(PKM_E_ARG, "gradient buffers must be 16-byte aligned");
    if ((g->dbn_gamma == nullptr) != (g->dbn_beta == nullptr))
        return fail(PKM_E_ARG, "dbn_gamma and dbn_beta go together");
    const int sparse = (g->dvalues_rows != nullptr) + (g->dvalues_sparse != nullptr) + (g->dvalues_count != nullptr);
    if (sparse != 0 && sparse != 3)
        return fail(PKM_E_ARG, "dvalues_rows, dvalues_sparse and dvalues_count go together");
    if (sparse && g->dvalues) return fail(PKM_E_ARG, "dvalues and the sparse value gradient exclude each other");
    if (sparse && ((uintptr_t)g->dvalues_rows % 4 || (uintptr_t)g->dvalues_count % 8))
        return fail(PKM_E_ARG, "dvalues_rows and dvalues_count must be aligned to their element size");
    return PKM_OK;
}

pkm_status check_forward_args(const pkm_config &c, const pkm_params *p, const float *x, const float *out,
                              const int32_t *idx, const float *weights)
{
    pkm_status s;
    if ((s = check_query_params(p)) || (s = need(p->subkeys, "subkeys")) || (s = check_value_params(c, p))) return s;
    if ((s = need(x, "x")) || (s = need(out, "out"))) return s;
    if ((idx && !aligned16(idx)) || (weights && !aligned16(weights)))
        return fail(PKM_E_ARG, "idx / weights must be 16-byte aligned");
    return PKM_OK;
}

// One stage of the forward for nb <= max_batch tokens, intermediates in the
// context's workspace: 0 the row exponents of x, Wq and the subkeys (and
// clearing q^'s maxima), 1 the projection with BN (recording q^'s maxima),
// 2 the subkey scoring, 3 the selection and the gather (one fused kernel
// where select_gather_fusable, else two).  keep: write idx / w out.
// Whether p names the arrays the context's folded form was made from.
bool folded_for(const pkm_ctx *ctx, const pkm_params *p)
{
    return ctx->prep_mode == 2 && ctx->prep_wq_src == p->wq && ctx->prep_sub_src == p->subkeys &&
           ctx->prep_bn_src[0] == p->bn_mean && ctx->prep_bn_src[1] == p->bn_var &&
           ctx->prep_bn_src[2] == p->bn_gamma && ctx->prep_bn_src[3] == p->bn_beta;
}

pkm_status forward_stage(const pkm_ctx *ctx, const pkm_params *p, int64_t nb, const float *x, float *out,
                         int32_t *ci, float *cw, bool keep, int stage, hipStream_t st, float *q_pre = nullptr,
                         float *scores_out = nullptr)
{
    const pkm_config &c = ctx->cfg;
    const int64_t H = c.heads, k = c.k;
    float *scores = scores_out ? scores_out : ctx->scores;
    // Folded (and no projection wanted): the half scores in one contraction
    // of x with the folded matrix, stage 0 x's row exponents and fp16
    // pieces, stage 1 the contraction, stage 2 nothing.
    if (!q_pre && folded_for(ctx, p) && stage <= 2) {
        if (stage == 2) return PKM_OK;
        if (stage == 0)
            return launched(pkm::launch_exp_split(x, c.dim, (int)nb, c.dim, ctx->gemm_exp, ctx->x_pieces, st),
                            "row exponents and split");
        pkm::GemmArgs a{};
        a.exp_ws = ctx->gemm_exp;
        a.exp_ws_ints = ctx->gemm_exp_ints;
        a.A = x;
        a.lda = c.dim;
        a.M = (int)nb;
        a.N = 2 * c.heads * c.n_keys;
        a.K = c.dim;
        a.batch = 1;
        a.b_exp_given = ctx->fold_exp;
        a.b_presplit = ctx->fold_pieces;
        a.a_presplit = ctx->x_pieces;
        a.ldb = c.dim;
        a.C = scores;  // [nb][2H][n]
        a.ldc = 2 * (int64_t)c.heads * c.n_keys;
        a.stream_out = true;  // read once, by the select
        a.col_bias = ctx->fold_bias;
        a.exp_phase = 2;  // x's exponents written by stage 0
        return launched(pkm::launch_gemm_nt_f32(a, st), "folded scoring");
    }
    // Wq and the subkeys from their prepared form when p names the arrays
    // pkm_prepare took them from (the same pieces and exponents the tiles
    // would compute, so the same results)
    const bool prep = ctx->prep_mode == 1 && ctx->prep_wq_src == p->wq && ctx->prep_sub_src == p->subkeys;
    if (stage <= 1) {
        pkm::GemmArgs a = query_args(c, p, nb, x, ctx->qhat, ctx->gemm_exp, ctx->gemm_exp_ints);
        a.row_seg_max = ctx->qmax;
        a.seg_cols = c.dim / 2;
        a.C_pre = q_pre;  // the projection before BN as well, when asked for
        a.zero_ptr = ctx->qmax;
        a.zero_n = nb * 2 * c.heads;
        if (prep) {  // the pre-pass does x alone
            a.b_exp_given = ctx->prep_wq_exp;
            a.b_presplit = ctx->prep_wq;
        } else {
            // the subkeys' row exponents for the scoring, in the same pre-pass
            a.extra_exp.base = p->subkeys;
            a.extra_exp.rows_per_batch = c.n_keys;
            a.extra_exp.batch = 2 * c.heads;
            a.extra_exp.stride = (int64_t)c.n_keys * (c.dim / 2);
            a.extra_exp.ld = c.dim / 2;
            a.extra_exp.K = c.dim / 2;
            a.extra_exp.out = ctx->sub_exp;
        }
        a.exp_phase = stage == 0 ? 1 : 2;
        return launched(pkm::launch_gemm_nt_f32(a, st), stage == 0 ? "row exponents" : "query projection");
    }
    if (stage == 2) {
        pkm::GemmArgs a = score_args(c, p, nb, ctx->qhat, scores, ctx->gemm_exp, ctx->gemm_exp_ints);
        a.a_rowmax = ctx->qmax;
        a.a_rowmax_ld = 2 * c.heads;
        a.b_exp_given = prep ? ctx->prep_sub_exp : ctx->sub_exp;
        if (prep) a.b_presplit = ctx->prep_sub;
        return launched(pkm::launch_gemm_nt_f32(a, st), "subkey scoring");
    }
    if (pkm::select_gather_fusable(c.heads, c.n_keys, c.k, c.value_type, c.dim))
        return launched(pkm::launch_select_gather(scores, nb, c.heads, c.n_keys, c.k, p->values, p->value_scale,
                                                  c.value_type, c.dim, c.n_keys * c.n_keys, keep ? ci : nullptr,
                                                  keep ? cw : nullptr, out, st),
                        "select and gather");
    pkm_status s;
    if ((s = launched(pkm::launch_select(scores, nb, c.heads, c.n_keys, c.k, ci, cw, st), "select"))) return s;
    return launched(pkm::launch_gather(p->values, p->value_scale, c.value_type, c.dim, c.n_keys * c.n_keys, nb,
                                       (int)(H * k), ci, cw, out, st),
                    "gather");
}

// a1-a7 over B tokens in chunks of the context's max_batch, every chunk
// through the context's workspace, its four stages in order; launches only.
pkm_status forward_chunks(const pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *out,
                          int32_t *idx, float *weights, hipStream_t st, float *q_pre = nullptr)
{
    pkm_status s;
    const pkm_config &c = ctx->cfg;
    const int64_t H = c.heads, D = c.dim, k = c.k;
    const bool keep = idx || weights;
    for (int64_t b0 = 0; b0 < B; b0 += c.max_batch) {
        const int64_t nb = B - b0 < c.max_batch ? B - b0 : c.max_batch;
        int32_t *ci = idx ? idx + b0 * H * k : ctx->idx;
        float *cw = weights ? weights + b0 * H * k : ctx->weights;
        for (int stage = 0; stage < 4; ++stage)
            if ((s = forward_stage(ctx, p, nb, x + b0 * D, out + b0 * D, ci, cw, keep, stage, st,
                                   q_pre ? q_pre + b0 * H * D : nullptr)))
                return s;
    }
    return PKM_OK;
}

// ------------------------------------------------------------------ scratch
//
// The allocation-free forward (pkm_forward_noalloc) keeps its workspace in
// this file-scope device array: every GPU the library runs on holds its own
// copy for the life of the process.  In host code the array's name is not a
// device address; its address on each device comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// used afterwards.
constexpr size_t kScratchBytes = (size_t)128 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
char *g_scratch_ptr[kMaxDevices];  // scratch's address on each device, once taken

pkm_status scratch_on_current_device(int *device, char **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PKM_E_DEVICE, "no HIP device: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(PKM_E_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return fail(PKM_E_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
            return fail(PKM_E_UNSUPPORTED, "device %d is %s; the kernels are built for gfx950", dev, prop.gcnArchName);
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(PKM_E_DEVICE, "address of the scratch array on device %d: %s", dev, hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = static_cast<char *>(ptr);
    }
    *device = dev;
    *out = g_scratch_ptr[dev];
    return PKM_OK;
}

size_t noalloc_bytes(pkm_config c, int64_t mb)
{
    c.max_batch = mb;
    size_t sizes[kPieces];
    if (!workspace_layout(c, sizes, false, false)) return SIZE_MAX;
    return total_bytes(sizes, kPieces);
}

// The chunk the allocation-free forward works in: the most tokens, at most
// c.max_batch, whose workspace fits the scratch array (a multiple of 256
// from 256 tokens on, the contractions' tile height).  Sets c.max_batch.
pkm_status noalloc_chunk(pkm_config &c)
{
    const size_t one = noalloc_bytes(c, 1);
    if (one > kScratchBytes)
        return fail(PKM_E_UNSUPPORTED, "one token's workspace (%zu bytes) exceeds the %zu-byte scratch array", one,
                    kScratchBytes);
    int64_t lo = 1, hi = c.max_batch;  // the workspace grows with the chunk
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (noalloc_bytes(c, mid) <= kScratchBytes) lo = mid;
        else hi = mid - 1;
    }
    c.max_batch = lo >= 256 ? lo / 256 * 256 : lo;
    return PKM_OK;
}

}  // namespace

extern "C" {

pkm_status pkm_config_check(const pkm_config *cfg) { return check_config(cfg); }

pkm_status pkm_workspace_bytes(const pkm_config *cfg, size_t *bytes)
{
    if (pkm_status s = check_config(cfg)) return s;
    if (!bytes) return fail(PKM_E_ARG, "bytes is NULL");
    size_t sizes[kPieces];
    workspace_layout(*cfg, sizes);
    *bytes = 0;
    for (size_t piece : sizes) *bytes += piece;
    return ok();
}

pkm_status pkm_create(const pkm_config *cfg, pkm_ctx **out)
{
    if (!out) return fail(PKM_E_ARG, "out is NULL");
    *out = nullptr;
    if (pkm_status s = check_config(cfg)) return s;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PKM_E_DEVICE, "no HIP device: %s", hipGetErrorString(e));
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(PKM_E_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(PKM_E_UNSUPPORTED, "device %d is %s; the kernels are built for gfx950", dev, prop.gcnArchName);
    size_t sizes[kPieces];
    workspace_layout(*cfg, sizes);
    size_t total = 0;
    for (size_t piece : sizes) total += piece;
    void *ws = nullptr;
    e = hipMalloc(&ws, total);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(PKM_E_NOMEM, "workspace of %zu bytes: %s", total, hipGetErrorString(e));
    }
    pkm_ctx *ctx = new (std::nothrow) pkm_ctx;
    if (!ctx) {
        (void)hipFree(ws);
        return fail(PKM_E_NOMEM, "host allocation failed");
    }
    ctx->cfg = *cfg;
    ctx->device = dev;
    assign_workspace(ctx, static_cast<char *>(ws), sizes);
    if (log_on())
        fprintf(stderr, "pkm: context on device %d (%s): D=%d H=%d n=%d k=%d values=%d max_batch=%lld workspace=%zu\n",
                dev, prop.gcnArchName, cfg->dim, cfg->heads, cfg->n_keys, cfg->k, cfg->value_type,
                (long long)cfg->max_batch, total);
    *out = ctx;
    return ok();
}

void pkm_destroy(pkm_ctx *ctx)
{
    if (!ctx) return;
    (void)hipFree(ctx->workspace);
    delete ctx;
}

pkm_status pkm_forward(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *out, int32_t *idx,
                       float *weights, void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx)) || (s = check_batch(ctx->cfg, B))) return s;
    if (B == 0) return ok();
    if ((s = check_forward_args(ctx->cfg, p, x, out, idx, weights))) return s;
    if ((s = forward_chunks(ctx, p, B, x, out, idx, weights, static_cast<hipStream_t>(stream)))) return s;
    return ok();
}

pkm_status pkm_prepare(pkm_ctx *ctx, const pkm_params *p, int flags, void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx))) return s;
    ctx->prep_wq_src = ctx->prep_sub_src = nullptr;
    for (auto &b : ctx->prep_bn_src) b = nullptr;
    ctx->prep_mode = 0;
    if (!p) return ok();  // only dropped
    if (flags != PKM_PREPARE_SPLIT && flags != PKM_PREPARE_FOLD) return fail(PKM_E_ARG, "unknown flags %d", flags);
    if ((s = need(p->wq, "wq")) || (s = need(p->subkeys, "subkeys"))) return s;
    const pkm_config &c = ctx->cfg;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (flags == PKM_PREPARE_FOLD && ctx->fold_pieces) {
        if ((s = check_query_params(p))) return s;
        // the fp32 folded matrix is built where the split form would go
        float *M = static_cast<float *>(ctx->prep_wq);
        const int rows = 2 * c.heads * c.n_keys;
        if ((s = launched(pkm::launch_fold(p->wq, p->bn_mean, p->bn_var, p->bn_gamma, p->bn_beta, c.bn_eps,
                                           p->subkeys, c.dim, c.heads, c.n_keys, M, ctx->fold_bias, st),
                          "fold")) ||
            (s = launched(pkm::launch_presplit(M, 0, c.dim, rows, c.dim, 1, ctx->fold_exp, ctx->fold_pieces, st),
                          "folded split")))
            return s;
        ctx->prep_bn_src[0] = p->bn_mean;
        ctx->prep_bn_src[1] = p->bn_var;
        ctx->prep_bn_src[2] = p->bn_gamma;
        ctx->prep_bn_src[3] = p->bn_beta;
        ctx->prep_mode = 2;
    } else {
        if ((s = launched(pkm::launch_presplit(p->wq, 0, c.dim, c.heads * c.dim, c.dim, 1, ctx->prep_wq_exp,
                                               ctx->prep_wq, st),
                          "Wq split")) ||
            (s = launched(pkm::launch_presplit(p->subkeys, (int64_t)c.n_keys * (c.dim / 2), c.dim / 2, c.n_keys,
                                               c.dim / 2, 2 * c.heads, ctx->prep_sub_exp, ctx->prep_sub, st),
                          "subkey split")))
            return s;
        ctx->prep_mode = 1;
    }
    ctx->prep_wq_src = p->wq;
    ctx->prep_sub_src = p->subkeys;
    return ok();
}

pkm_status pkm_half_scores(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *scores,
                           void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx)) || (s = check_batch(ctx->cfg, B))) return s;
    if (B == 0) return ok();
    if (!p) return fail(PKM_E_ARG, "params is NULL");
    if ((s = check_query_params(p)) || (s = need(p->subkeys, "subkeys")) || (s = need(x, "x")) ||
        (s = need(scores, "scores")))
        return s;
    const pkm_config &c = ctx->cfg;
    const int64_t D = c.dim, per = 2 * (int64_t)c.heads * c.n_keys;
    for (int64_t b0 = 0; b0 < B; b0 += c.max_batch) {
        const int64_t nb = B - b0 < c.max_batch ? B - b0 : c.max_batch;
        for (int stage = 0; stage < 3; ++stage)
            if ((s = forward_stage(ctx, p, nb, x + b0 * D, nullptr, nullptr, nullptr, false, stage,
                                   static_cast<hipStream_t>(stream), nullptr, scores + b0 * per)))
                return s;
    }
    return ok();
}

pkm_status pkm_forward_train(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *out, int32_t *idx,
                             float *weights, float *q, void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx)) || (s = check_batch(ctx->cfg, B))) return s;
    if (B == 0) return ok();
    if ((s = check_forward_args(ctx->cfg, p, x, out, idx, weights)) || (s = need(q, "q"))) return s;
    if ((s = forward_chunks(ctx, p, B, x, out, idx, weights, static_cast<hipStream_t>(stream), q))) return s;
    return ok();
}

pkm_status pkm_forward_noalloc(const pkm_config *cfg, const pkm_params *p, int64_t B, const float *x, float *out,
                               int32_t *idx, float *weights, void *stream)
{
    pkm_status s;
    if ((s = check_config(cfg)) || (s = check_batch(*cfg, B))) return s;
    pkm_ctx ctx{};
    ctx.cfg = *cfg;
    if ((s = noalloc_chunk(ctx.cfg))) return s;
    if (B == 0) return ok();
    if ((s = check_forward_args(ctx.cfg, p, x, out, idx, weights))) return s;
    char *base = nullptr;
    if ((s = scratch_on_current_device(&ctx.device, &base))) return s;
    size_t sizes[kPieces];
    workspace_layout(ctx.cfg, sizes, false, false);  // as noalloc_bytes sized it
    assign_workspace(&ctx, base, sizes);
    if ((s = forward_chunks(&ctx, p, B, x, out, idx, weights, static_cast<hipStream_t>(stream)))) return s;
    return ok();
}

pkm_status pkm_forward_stage(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *out, int32_t *idx,
                             float *weights, int stage, void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx)) || (s = check_batch(ctx->cfg, B))) return s;
    if (stage < 0 || stage > 3) return fail(PKM_E_ARG, "stage must be 0, 1, 2 or 3 (got %d)", stage);
    if (B > ctx->cfg.max_batch)
        return fail(PKM_E_ARG, "B = %lld is larger than max_batch = %lld: the stages work on one chunk",
                    (long long)B, (long long)ctx->cfg.max_batch);
    if (B == 0) return ok();
    if ((s = check_forward_args(ctx->cfg, p, x, out, idx, weights))) return s;
    const bool keep = idx || weights;
    if ((s = forward_stage(ctx, p, B, x, out, idx ? idx : ctx->idx, weights ? weights : ctx->weights, keep, stage,
                           static_cast<hipStream_t>(stream))))
        return s;
    return ok();
}

pkm_status pkm_query(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *qhat, void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx)) || (s = check_batch(ctx->cfg, B))) return s;
    if (B == 0) return ok();
    if ((s = check_query_params(p))) return s;
    if ((s = need(x, "x")) || (s = need(qhat, "qhat"))) return s;
    if ((s = run_query(ctx, p, B, x, qhat, nullptr, static_cast<hipStream_t>(stream)))) return s;
    return ok();
}

pkm_status pkm_score(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *qhat, float *scores, void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx)) || (s = check_batch(ctx->cfg, B))) return s;
    if (B == 0) return ok();
    if (!p) return fail(PKM_E_ARG, "params is NULL");
    if ((s = need(p->subkeys, "subkeys")) || (s = need(qhat, "qhat")) || (s = need(scores, "scores"))) return s;
    if ((s = run_score(ctx, p, B, qhat, scores, nullptr, static_cast<hipStream_t>(stream)))) return s;
    return ok();
}

pkm_status pkm_select(pkm_ctx *ctx, int64_t B, const float *scores, int32_t *idx, float *weights, void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx)) || (s = check_batch(ctx->cfg, B))) return s;
    if (B == 0) return ok();
    if ((s = need(scores, "scores")) || (s = need(idx, "idx")) || (s = need(weights, "weights"))) return s;
    const pkm_config &c = ctx->cfg;
    if ((s = launched(pkm::launch_select(scores, B, c.heads, c.n_keys, c.k, idx, weights,
                                         static_cast<hipStream_t>(stream)),
                      "select")))
        return s;
    return ok();
}

pkm_status pkm_gather(pkm_ctx *ctx, const pkm_params *p, int64_t B, int32_t rows_per_token, const int32_t *idx,
                      const float *weights, float *out, void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx)) || (s = check_batch(ctx->cfg, B))) return s;
    if (B == 0) return ok();
    const pkm_config &c = ctx->cfg;
    if ((s = check_value_params(c, p))) return s;
    if (rows_per_token < 1) return fail(PKM_E_ARG, "rows_per_token must be >= 1 (got %d)", rows_per_token);
    if ((s = need(idx, "idx")) || (s = need(weights, "weights")) || (s = need(out, "out"))) return s;
    if ((s = launched(pkm::launch_gather(p->values, p->value_scale, c.value_type, c.dim, c.n_keys * c.n_keys, B,
                                         rows_per_token, idx,
                                         weights, out, static_cast<hipStream_t>(stream)),
                      "gather")))
        return s;
    return ok();
}

pkm_status pkm_select_gather(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *scores, int32_t *idx,
                             float *weights, float *out, void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx)) || (s = check_batch(ctx->cfg, B))) return s;
    if (B == 0) return ok();
    const pkm_config &c = ctx->cfg;
    if ((s = check_value_params(c, p))) return s;
    if ((s = need(scores, "scores")) || (s = need(out, "out"))) return s;
    if ((idx == nullptr) != (weights == nullptr)) return fail(PKM_E_ARG, "idx and weights go together (both or neither)");
    if (idx && ((s = need(idx, "idx")) || (s = need(weights, "weights")))) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t H = c.heads, k = c.k, N = (int64_t)c.n_keys * c.n_keys;
    if (pkm::select_gather_fusable(c.heads, c.n_keys, c.k, c.value_type, c.dim)) {
        if ((s = launched(pkm::launch_select_gather(scores, B, c.heads, c.n_keys, c.k, p->values, p->value_scale,
                                                    c.value_type, c.dim, (int)N, idx, weights, out, st),
                          "select and gather")))
            return s;
        return ok();
    }
    // the two kernels, in chunks of max_batch when the selection goes to the workspace
    for (int64_t b0 = 0; b0 < B; b0 += idx ? B : c.max_batch) {
        const int64_t nb = idx ? B : (B - b0 < c.max_batch ? B - b0 : c.max_batch);
        int32_t *ci = idx ? idx : ctx->idx;
        float *cw = idx ? weights : ctx->weights;
        if ((s = launched(pkm::launch_select(scores + b0 * H * 2 * c.n_keys, nb, c.heads, c.n_keys, c.k, ci, cw, st),
                          "select")) ||
            (s = launched(pkm::launch_gather(p->values, p->value_scale, c.value_type, c.dim, (int)N, nb, (int)(H * k),
                                             ci, cw, out + b0 * c.dim, st),
                          "gather")))
            return s;
    }
    return ok();
}

pkm_status pkm_flat_workspace_bytes(const pkm_config *cfg, int64_t B, size_t *bytes)
{
    if (pkm_status s = check_config(cfg)) return s;
    if (!bytes) return fail(PKM_E_ARG, "bytes is NULL");
    size_t sizes[kFlatPieces];
    if (!flat_layout(*cfg, B, sizes)) return fail(PKM_E_ARG, "flat search B must be in [0, %lld]", (long long)kFlatMaxBatch);
    *bytes = total_bytes(sizes, kFlatPieces);
    return ok();
}

pkm_status pkm_flat_search(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *qhat, void *workspace,
                           size_t workspace_bytes, int32_t *idx, float *top, void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx))) return s;
    const pkm_config &c = ctx->cfg;
    size_t sizes[kFlatPieces];
    if (!flat_layout(c, B, sizes)) return fail(PKM_E_ARG, "flat search B must be in [0, %lld]", (long long)kFlatMaxBatch);
    if (B == 0) return ok();
    if (!p) return fail(PKM_E_ARG, "params is NULL");
    if ((s = need(p->subkeys, "subkeys")) || (s = need(qhat, "qhat")) || (s = need(workspace, "workspace")) ||
        (s = need(idx, "idx")) || (s = need(top, "top")))
        return s;
    const size_t need_bytes = total_bytes(sizes, kFlatPieces);
    if (workspace_bytes < need_bytes)
        return fail(PKM_E_ARG, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *piece[kFlatPieces];
    piece[0] = static_cast<char *>(workspace);
    for (int i = 1; i < kFlatPieces; ++i) piece[i] = piece[i - 1] + sizes[i - 1];
    float *scores = reinterpret_cast<float *>(piece[0]);
    uint64_t *buf0 = reinterpret_cast<uint64_t *>(piece[1]);
    uint64_t *buf1 = reinterpret_cast<uint64_t *>(piece[2]);
    int32_t *exps = reinterpret_cast<int32_t *>(piece[3]);
    const int64_t rows = B * c.heads, N = (int64_t)c.n_keys * c.n_keys;
    const bool threshold = N > kFlatDirectMax;
    pkm::GemmArgs a = flat_args(c, p, B, qhat, scores, exps, (int64_t)(sizes[3] / sizeof(int32_t)));
    a.b_split = piece[9];
    a.b_split_bytes = (int64_t)sizes[9];
    float *gmax = threshold ? reinterpret_cast<float *>(piece[4]) : nullptr;
    if (gmax) {
        const int64_t G = (N + 63) / 64;
        a.group_max = gmax;  // [B][H][G], like the scores
        a.group_ld = c.heads * G;
        a.group_stride = G;
    }
    if ((s = launched(pkm::launch_gemm_nt_f32_product(a, st), "flat key scoring"))) return s;
    if (threshold)
        s = launched(pkm::launch_flat_topk_threshold(scores, gmax, rows, N, c.k, buf0, buf1,
                                                     reinterpret_cast<int32_t *>(piece[5]),
                                                     reinterpret_cast<float *>(piece[6]),
                                                     reinterpret_cast<uint32_t *>(piece[7]),
                                                     reinterpret_cast<uint64_t *>(piece[8]), idx, top, st),
                     "flat top-k");
    else
        s = launched(pkm::launch_flat_topk(scores, rows, N, c.k, buf0, buf1, idx, top, st), "flat top-k");
    if (s) return s;
    return ok();
}

pkm_status pkm_backward_workspace_bytes(const pkm_config *cfg, size_t *bytes)
{
    if (pkm_status s = check_config(cfg)) return s;
    if (!bytes) return fail(PKM_E_ARG, "bytes is NULL");
    size_t sizes[kBwdPieces];
    if (!backward_layout(*cfg, sizes)) return fail(PKM_E_ARG, "backward workspace size overflows");
    *bytes = 0;
    for (size_t piece : sizes) *bytes += piece;
    return ok();
}

}  // extern "C"

namespace {

// The backward for running statistics (mean, var = p's) or, with batch
// true, for the statistics of this batch (mean, var given; one chunk).
pkm_status run_backward(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, const int32_t *idx,
                        const float *weights, const float *dout, const float *mean, const float *var, bool batch,
                        const pkm_grads *grads, void *workspace, size_t workspace_bytes, void *stream,
                        const float *q_given = nullptr)
{
    pkm_status s;
    const pkm_config &c = ctx->cfg;
    size_t sizes[kBwdPieces];
    backward_layout(c, sizes);  // checked by the caller
    (void)workspace_bytes;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(workspace);
    void *piece[kBwdPieces];
    for (int i = 0; i < kBwdPieces; ++i) {
        piece[i] = w;
        w += sizes[i];
    }
    float *Q = static_cast<float *>(piece[0]), *dt = static_cast<float *>(piece[1]);
    float *dqh = static_cast<float *>(piece[2]), *dq = static_cast<float *>(piece[3]);
    float *dqT = static_cast<float *>(piece[4]), *xT = static_cast<float *>(piece[5]);
    float *wqT = static_cast<float *>(piece[6]);
    float *sum_g = static_cast<float *>(piece[7]), *sum_b = sum_g + (size_t)c.heads * c.dim;
    float *G = static_cast<float *>(piece[8]);
    float *part_g = static_cast<float *>(piece[9]), *part_b = static_cast<float *>(piece[10]);
    uint32_t *count = static_cast<uint32_t *>(piece[11]), *cursor = static_cast<uint32_t *>(piece[12]);
    uint32_t *offs = static_cast<uint32_t *>(piece[13]), *block_sum = static_cast<uint32_t *>(piece[14]);
    uint32_t *list = static_cast<uint32_t *>(piece[15]);
    float *partial = static_cast<float *>(piece[16]);
    const int64_t partial_floats = (int64_t)(sizes[16] / sizeof(float));
    int32_t *exps = static_cast<int32_t *>(piece[17]);
    const int64_t exp_ints = (int64_t)(sizes[17] / sizeof(int32_t));

    const int H = c.heads, D = c.dim, k = c.k, n = c.n_keys, HD = H * D, N = n * n;
    // the dense value gradient or the sparse one (one chunk, checked)
    float *dval = grads->dvalues_sparse ? grads->dvalues_sparse : grads->dvalues;
    if (grads->dx &&
        (s = launched(pkm::launch_transpose(p->wq, D, HD, D, wqT, HD, HD, nullptr, nullptr, nullptr, nullptr, 0.0f, st),
                      "Wq transpose")))
        return s;
    for (int64_t b0 = 0; b0 < B; b0 += c.max_batch) {
        const int64_t nb = B - b0 < c.max_batch ? B - b0 : c.max_batch;
        const int nb32 = (int)((nb + 31) / 32 * 32);
        const float *xc = x + b0 * D, *doutc = dout + b0 * D, *wc = weights + b0 * H * k;
        const int32_t *ic = idx + b0 * H * k;
        // everything but the value gradient flows through the scores
        const bool through_scores = grads->dx || grads->dwq || grads->dbn_gamma || grads->dsubkeys;
        if (!through_scores) {
            if (dval &&
                (s = launched(pkm::launch_value_grad(ic, nb * H * k, N, D, H * k, wc, doutc, count, cursor, offs,
                                                     block_sum, list, dval, grads->dvalues_rows,
                                                     grads->dvalues_count, st),
                              "value gradient")))
                return s;
            continue;
        }
        // q before BN: the forward's (pkm_forward_train), or computed again
        const float *Qc = q_given ? q_given + b0 * HD : Q;
        if (!q_given) {
            pkm::GemmArgs qa = query_args(c, p, nb, xc, Q, exps, exp_ints);
            qa.bn_mean = qa.bn_var = qa.bn_gamma = qa.bn_beta = nullptr;
            if ((s = launched(pkm::launch_gemm_nt_f32(qa, st), "query recompute"))) return s;
        }
        if ((s = launched(pkm::launch_value_backward(p->values, p->value_scale, c.value_type, D, N, nb, H, k, ic, wc,
                                                     doutc, dt, st),
                          "value backward")))
            return s;
        if (grads->dsubkeys &&
            (s = launched(pkm::launch_fill(reinterpret_cast<uint32_t *>(G), (int64_t)2 * H * n * nb32, 0u, st),
                          "clear")))
            return s;
        if ((s = launched(pkm::launch_dqhat(p->subkeys, var, p->bn_gamma, c.bn_eps, D, n, nb, H, k, ic, dt, dqh, dq, G,
                                            nb32, st),
                          "query gradient")))
            return s;
        if ((grads->dbn_gamma || batch) &&
            (s = launched(pkm::launch_bn_grads(dqh, Qc, mean, var, c.bn_eps, nb, HD, part_g, part_b, grads->dbn_gamma,
                                               grads->dbn_beta, batch ? sum_g : nullptr, batch ? sum_b : nullptr, st),
                          "BN gradients")))
            return s;
        if (batch && (s = launched(pkm::launch_bn_batch_dq(dqh, Qc, nb, HD, mean, var, p->bn_gamma, c.bn_eps, sum_g,
                                                           sum_b, dq, st),
                                   "batch BN backward")))
            return s;
        if (grads->dwq) {
            if ((s = launched(pkm::launch_transpose(dq, HD, (int)nb, HD, dqT, nb32, nb32, nullptr, nullptr, nullptr,
                                                    nullptr, 0.0f, st),
                              "dq transpose")) ||
                (s = launched(pkm::launch_transpose(xc, D, (int)nb, D, xT, nb32, nb32, nullptr, nullptr, nullptr,
                                                    nullptr, 0.0f, st),
                              "x transpose")))
                return s;
            pkm::GemmArgs a{};
            a.A = dqT;
            a.lda = nb32;
            a.strideA = (int64_t)D * nb32;
            a.B = xT;
            a.ldb = nb32;
            a.strideB = 0;
            a.C = grads->dwq;
            a.ldc = D;
            a.strideC = (int64_t)D * D;
            a.M = D;
            a.N = D;
            a.K = nb32;
            a.batch = H;
            a.accumulate = true;
            a.partial = partial;
            a.partial_floats = partial_floats;
            a.exp_ws = exps;
            a.exp_ws_ints = exp_ints;
            if ((s = launched(pkm::launch_gemm_nt_f32(a, st), "dWq"))) return s;
        }
        if (grads->dsubkeys &&
            (s = launched(pkm::launch_dsub(G, nb32, nb, Qc, H, D, n, mean, var, p->bn_gamma, p->bn_beta, c.bn_eps,
                                           grads->dsubkeys, st),
                          "subkey gradient")))
            return s;
        if (grads->dx) {
            pkm::GemmArgs a{};
            a.A = dq;
            a.lda = HD;
            a.B = wqT;
            a.ldb = HD;
            a.C = grads->dx + b0 * D;
            a.ldc = D;
            a.M = (int)nb;
            a.N = D;
            a.K = HD;
            a.batch = 1;
            a.partial = partial;
            a.partial_floats = partial_floats;
            a.exp_ws = exps;
            a.exp_ws_ints = exp_ints;
            if ((s = launched(pkm::launch_gemm_nt_f32(a, st), "dx"))) return s;
        }
        if (dval && (s = launched(pkm::launch_value_grad(ic, nb * H * k, N, D, H * k, wc, doutc, count, cursor, offs,
                                                         block_sum, list, dval, grads->dvalues_rows,
                                                         grads->dvalues_count, st),
                                  "value gradient")))
            return s;
    }
    return ok();
}

// Arguments of either backward; batch: the BN statistics come from the
// caller, not from p.
pkm_status check_backward_args(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, const int32_t *idx,
                               const float *weights, const float *dout, const pkm_grads *grads, void *workspace,
                               size_t workspace_bytes, bool batch)
{
    pkm_status s;
    if ((s = check_ctx(ctx)) || (s = check_batch(ctx->cfg, B))) return s;
    const pkm_config &c = ctx->cfg;
    size_t sizes[kBwdPieces];
    if (!backward_layout(c, sizes)) return fail(PKM_E_ARG, "backward workspace size overflows");
    size_t need_bytes = 0;
    for (size_t piece : sizes) need_bytes += piece;
    if (B == 0) return PKM_OK;
    if (!p) return fail(PKM_E_ARG, "params is NULL");
    if (batch) {
        if ((s = need(p->wq, "wq")) || (s = need(p->bn_gamma, "bn_gamma")) || (s = need(p->bn_beta, "bn_beta")))
            return s;
    } else if ((s = check_query_params(p))) {
        return s;
    }
    if ((s = need(p->subkeys, "subkeys")) || (s = check_value_params(c, p))) return s;
    if ((s = need(x, "x")) || (s = need(idx, "idx")) || (s = need(weights, "weights")) || (s = need(dout, "dout")) ||
        (s = need(workspace, "workspace")) || (s = check_grads(grads)))
        return s;
    if (workspace_bytes < need_bytes)
        return fail(PKM_E_ARG, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need_bytes);
    if (grads->dvalues_sparse && B > c.max_batch)
        return fail(PKM_E_ARG, "the sparse value gradient needs B <= max_batch (got B = %lld)", (long long)B);
    return PKM_OK;
}

// B = 0: the sparse value gradient's row count is still written (zero);
// its row buffers have no entries then and may be NULL.
pkm_status empty_backward(const pkm_grads *grads, void *stream)
{
    if (!grads || !grads->dvalues_count) return ok();
    if ((uintptr_t)grads->dvalues_count % 8) return fail(PKM_E_ARG, "dvalues_count must be 8-byte aligned");
    return launched(pkm::launch_fill(reinterpret_cast<uint32_t *>(grads->dvalues_count), 2, 0u,
                                     static_cast<hipStream_t>(stream)),
                    "clear");
}

}  // namespace

extern "C" {

pkm_status pkm_backward(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, const int32_t *idx,
                        const float *weights, const float *dout, const pkm_grads *grads, void *workspace,
                        size_t workspace_bytes, void *stream)
{
    if (pkm_status s = check_backward_args(ctx, p, B, x, idx, weights, dout, grads, workspace, workspace_bytes, false))
        return s;
    if (B == 0) return empty_backward(grads, stream);
    return run_backward(ctx, p, B, x, idx, weights, dout, p->bn_mean, p->bn_var, false, grads, workspace,
                        workspace_bytes, stream);
}

pkm_status pkm_backward_with_q(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, const float *q,
                               const int32_t *idx, const float *weights, const float *dout, const pkm_grads *grads,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    if (pkm_status s = check_backward_args(ctx, p, B, x, idx, weights, dout, grads, workspace, workspace_bytes, false))
        return s;
    if (B == 0) return empty_backward(grads, stream);
    if (pkm_status s = need(q, "q")) return s;
    return run_backward(ctx, p, B, x, idx, weights, dout, p->bn_mean, p->bn_var, false, grads, workspace,
                        workspace_bytes, stream, q);
}

pkm_status pkm_backward_batch_stats(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x,
                                    const int32_t *idx, const float *weights, const float *dout,
                                    const float *batch_mean, const float *batch_var, const pkm_grads *grads,
                                    void *workspace, size_t workspace_bytes, void *stream)
{
    if (pkm_status s = check_backward_args(ctx, p, B, x, idx, weights, dout, grads, workspace, workspace_bytes, true))
        return s;
    if (B == 0) return empty_backward(grads, stream);
    if (B < 2 || B > ctx->cfg.max_batch)
        return fail(PKM_E_ARG, "batch statistics need 2 <= B <= max_batch (got B = %lld)", (long long)B);
    pkm_status s;
    if ((s = need(batch_mean, "batch_mean")) || (s = need(batch_var, "batch_var"))) return s;
    return run_backward(ctx, p, B, x, idx, weights, dout, batch_mean, batch_var, true, grads, workspace,
                        workspace_bytes, stream);
}

pkm_status pkm_forward_batch_stats(pkm_ctx *ctx, const pkm_params *p, int64_t B, const float *x, float *out,
                                   int32_t *idx, float *weights, float *batch_mean, float *batch_var,
                                   float *running_mean, float *running_var, float momentum, void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx)) || (s = check_batch(ctx->cfg, B))) return s;
    if (B == 0) return ok();
    const pkm_config &c = ctx->cfg;
    if (B < 2 || B > c.max_batch)
        return fail(PKM_E_ARG, "batch statistics need 2 <= B <= max_batch (got B = %lld)", (long long)B);
    if (!p) return fail(PKM_E_ARG, "params is NULL");
    if ((s = need(p->wq, "wq")) || (s = need(p->bn_gamma, "bn_gamma")) || (s = need(p->bn_beta, "bn_beta")) ||
        (s = need(p->subkeys, "subkeys")) || (s = check_value_params(c, p)))
        return s;
    if ((s = need(x, "x")) || (s = need(out, "out")) || (s = need(batch_mean, "batch_mean")) ||
        (s = need(batch_var, "batch_var")))
        return s;
    if ((idx && !aligned16(idx)) || (weights && !aligned16(weights)))
        return fail(PKM_E_ARG, "idx / weights must be 16-byte aligned");
    if ((running_mean == nullptr) != (running_var == nullptr))
        return fail(PKM_E_ARG, "running_mean and running_var go together");
    if ((running_mean && !aligned16(running_mean)) || (running_var && !aligned16(running_var)))
        return fail(PKM_E_ARG, "running statistics must be 16-byte aligned");
    if (!(momentum >= 0.0f && momentum <= 1.0f)) return fail(PKM_E_ARG, "momentum must be in [0, 1]");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int HD = c.heads * c.dim;
    int32_t *ci = idx ? idx : ctx->idx;
    float *cw = weights ? weights : ctx->weights;
    pkm::GemmArgs qa = query_args(c, p, B, x, ctx->qhat, ctx->gemm_exp, ctx->gemm_exp_ints);
    qa.bn_mean = qa.bn_var = qa.bn_gamma = qa.bn_beta = nullptr;
    // With half-heads of whole 256-column groups the normalisation records
    // q^'s per-half maxima and the projection's pre-pass the subkeys' row
    // exponents, so the scoring needs no pre-pass of its own (as in
    // pkm_forward); otherwise the scoring computes its exponents.
    uint32_t *qmax = (c.dim / 2) % 256 == 0 ? ctx->qmax : nullptr;
    if (qmax) {
        qa.zero_ptr = qmax;
        qa.zero_n = B * 2 * c.heads;
        qa.extra_exp.base = p->subkeys;
        qa.extra_exp.rows_per_batch = c.n_keys;
        qa.extra_exp.batch = 2 * c.heads;
        qa.extra_exp.stride = (int64_t)c.n_keys * (c.dim / 2);
        qa.extra_exp.ld = c.dim / 2;
        qa.extra_exp.K = c.dim / 2;
        qa.extra_exp.out = ctx->sub_exp;
    }
    if ((s = launched(pkm::launch_gemm_nt_f32(qa, st), "query projection")) ||
        (s = launched(pkm::launch_batch_stats(ctx->qhat, B, HD, ctx->stat_part, batch_mean, batch_var, running_mean,
                                              running_var, momentum, st),
                      "batch statistics")) ||
        (s = launched(pkm::launch_bn_apply(ctx->qhat, B, HD, batch_mean, batch_var, p->bn_gamma, p->bn_beta, c.bn_eps,
                                           qmax, c.dim / 2, st),
                      "batch normalisation")) ||
        (s = run_score(ctx, p, B, ctx->qhat, ctx->scores, qmax, st)) ||
        (s = launched(pkm::launch_select(ctx->scores, B, c.heads, c.n_keys, c.k, ci, cw, st), "select")) ||
        (s = launched(pkm::launch_gather(p->values, p->value_scale, c.value_type, c.dim, c.n_keys * c.n_keys, B,
                                         c.heads * c.k, ci, cw, out, st),
                      "gather")))
        return s;
    return ok();
}

pkm_status pkm_usage(pkm_ctx *ctx, int64_t B, int32_t rows_per_token, const int32_t *idx, uint32_t *counts,
                     void *stream)
{
    pkm_status s;
    if ((s = check_ctx(ctx)) || (s = check_batch(ctx->cfg, B))) return s;
    if (rows_per_token < 1) return fail(PKM_E_ARG, "rows_per_token must be >= 1 (got %d)", rows_per_token);
    if (B == 0) return ok();
    if ((s = need(idx, "idx")) || (s = need(counts, "counts"))) return s;
    const pkm_config &c = ctx->cfg;
    if ((s = launched(pkm::launch_usage(idx, B * rows_per_token, c.n_keys * c.n_keys, counts,
                                        static_cast<hipStream_t>(stream)),
                      "usage")))
        return s;
    return ok();
}

const char *pkm_status_str(pkm_status s)
{
    switch (s) {
    case PKM_OK: return "ok";
    case PKM_E_ARG: return "invalid argument";
    case PKM_E_UNSUPPORTED: return "unsupported configuration or device";
    case PKM_E_NOMEM: return "device allocation failed";
    case PKM_E_DEVICE: return "HIP runtime error";
    }
    return "unknown status";
}

const char *pkm_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
