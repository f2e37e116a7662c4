// Internal launch interface between the host library (pkm_api.cpp) and the
// gfx950 kernels.  Every launcher enqueues on `stream` and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkm {

// C[g][m][n] = sum_k A[g][m][k] * B[g][n][k]  (both operands K-contiguous),
// for g < batch, m < M, n < N; K % 32 == 0; fp32 operands, fp32-accurate
// result (fp16 pieces on the matrix cores, see gemm_f32.hip).  With bn_* non-null the epilogue
// applies inference BatchNorm to column n:
//   (c - mean[n]) / sqrt(var[n] + eps) * gamma[n] + beta[n].
// stream_out: store C with non-temporal stores (for a result read once by a
// later kernel: it is written through to HBM while the GEMM is compute-bound
// instead of staying dirty in the caches and being written back during
// whatever memory-bound kernel runs next).
struct GemmArgs {
    const float *A;
    int64_t lda, strideA;
    const float *B;
    int64_t ldb, strideB;
    float *C;
    int64_t ldc, strideC;
    // Optional, with the BN epilogue (staged, not streamed): the values
    // before BN as well, same layout as C (the projection a training
    // backward needs again).
    float *C_pre;
    int M, N, K, batch;
    const float *bn_mean, *bn_var, *bn_gamma, *bn_beta;
    float bn_eps;
    bool stream_out;
    // Product-key B operand (B2 non-null): row j of B is the concatenation
    // [B[j / key_n][0, split_k), B2[j % key_n][0, K - split_k)], both with
    // row stride ldb and batch stride strideB; split_k = K / 2, a multiple
    // of 32; needs b_split.
    const float *B2;
    int split_k, key_n;
    // accumulate: C += A . B^T instead of C = A . B^T (no BN, no streaming).
    bool accumulate;
    // Optional split-K workspace (plain or accumulate contractions only):
    // when the 256x256 grid has fewer tiles than CUs, K is cut into up to
    // kMaxKSplits ranges whose partial products go to `partial` and are then
    // summed in split order (bitwise reproducible).  Needs
    // splits * batch * M * N floats; with partial == nullptr or too small a
    // capacity the contraction runs unsplit on smaller tiles.
    float *partial;
    int64_t partial_floats;
    // Row-exponent workspace (required): the launcher writes one int32 per
    // row of A and of B -- gemm_exp_ints(a) of them -- and the kernel scales
    // each row by that power of two before splitting it into fp16 pieces,
    // undoing both in the epilogue.
    int32_t *exp_ws;
    int64_t exp_ws_ints;
    // Optional, with a staged (non-streamed) epilogue: record per output row
    // and segment of seg_cols columns (seg_cols % 32 == 0, N % seg_cols ==
    // 0) the largest |C| as float bits, by atomic max into
    // row_seg_max[row * (N / seg_cols) + col / seg_cols]; the pre-pass first
    // zeroes zero_n uint32s at zero_ptr (the caller's choice of what to clear).
    uint32_t *row_seg_max;
    int seg_cols;
    uint32_t *zero_ptr;
    int64_t zero_n;
    // Optional: A's row maxima known beforehand (float bits): row m of batch
    // entry g has largest magnitude a_rowmax[m * a_rowmax_ld + g], turned
    // into exponents by the kernel itself.
    const uint32_t *a_rowmax;
    int a_rowmax_ld;
    // Optional: B's row exponents computed beforehand ([batch][N]).  With
    // both this and a_rowmax the contraction needs no pre-pass.
    const int32_t *b_exp_given;
    // Optional, with b_exp_given (not with accumulate): B's rows already
    // scaled by those exponents and split into fp16 pieces by
    // launch_presplit (16-byte aligned), so the tiles copy them instead of
    // splitting B.  Bitwise the same results as splitting in the tiles.
    const void *b_presplit;
    // Optional, with b_presplit, stream_out and batch 1: A's rows split the
    // same way by launch_exp_split, which also wrote their exponents to the
    // start of exp_ws (run the contraction with exp_phase 2).
    const void *a_presplit;
    // Optional, with stream_out: a per-column term added to every result,
    // col_bias[g * N + n] for batch entry g (the folded lookup's batch-norm
    // shift).
    const float *col_bias;
    // Optional: one more set of row exponents for a later contraction,
    // computed in this one's pre-pass (rows_per_batch * batch rows of K
    // floats, row m of entry g at base + g * stride + m * ld).
    struct {
        const float *base;
        int64_t rows_per_batch, stride, ld;
        int batch, K;
        int32_t *out;
    } extra_exp;
    // Optional, product-key B operand only: per row of C and group of 64
    // consecutive columns, the group's largest value (by order key) at
    // group_max[m * group_ld + g * group_stride + n / 64].
    float *group_max;
    int64_t group_ld, group_stride;
    // Product-key B operand only: a workspace of b_split_bytes >=
    // gemm_split_bytes(a) bytes (16-byte aligned) into which the subkey rows
    // are split into fp16 pieces once, so the contraction copies them
    // instead of splitting every virtual key row in every tile.
    void *b_split;
    int64_t b_split_bytes;
    // Which part of the work a launch does: 0 the row-exponent pre-pass
    // (when one is needed) then the contraction; 1 the pre-pass only; 2 the
    // contraction only, its exponents computed by an earlier phase-1 launch
    // with the same arguments and workspace.
    int exp_phase;
    // set by the launcher
    int k_chunk;  // K per split (0: no split)
    const int32_t *a_exp, *b_exp, *b2_exp;
};
constexpr int kMaxKSplits = 4;
// int32s of row exponents a contraction needs: batch * (M + N), or
// batch * (M + 2 key_n) with a product-key B operand.
int64_t gemm_exp_ints(const GemmArgs &a);
// bytes of the pre-split key rows: batch * 2 sets * key_n rounded up to 32
// rows * split_k * (two fp16 pieces)
int64_t gemm_split_bytes(const GemmArgs &a);
hipError_t launch_gemm_nt_f32(const GemmArgs &a, hipStream_t stream);
// A B operand of launch_gemm_nt_f32 prepared once for many contractions
// (weights): rows [batch][rows][K] fp32 (row m of entry g at B + g * stride
// + m * ld, K % 32 == 0) -> their row exponents exp [batch * rows] int32 and
// their fp16 pieces at out (gemm_presplit_bytes(rows, K, batch) bytes,
// 16-byte aligned), for GemmArgs::b_exp_given and b_presplit.
int64_t gemm_presplit_bytes(int rows, int K, int batch);
hipError_t launch_presplit(const float *B, int64_t stride, int64_t ld, int rows, int K, int batch, int32_t *exp,
                           void *out, hipStream_t stream);
// A plain A operand [M][K] (row stride lda): its row exponents (exp_out [M])
// and fp16 pieces (out, gemm_presplit_bytes(M, K, 1) bytes, 16-byte
// aligned) in one pass, for GemmArgs::a_presplit.  K % 32 == 0.
hipError_t launch_exp_split(const float *A, int64_t lda, int M, int K, int32_t *exp_out, void *out,
                            hipStream_t stream);
// The projection, inference batch-norm and subkeys folded, for the lookup
// with fixed statistics: M [2H][n][D] and bias [2H][n] fp32 (fp64
// accumulation, one rounding) with, for g = 2h + p, the half scores
// s[b][g][j] = x[b] . M[g][j] + bias[g][j].  D % 64 == 0.
hipError_t launch_fold(const float *wq, const float *mean, const float *var, const float *gamma, const float *beta,
                       float eps, const float *subkeys, int D, int H, int n, float *M, float *bias,
                       hipStream_t stream);
// The same contraction with a product-key B operand (b_split required) and
// 32 x 256 tiles, suited to a few dozen rows of A (the flat exact search
// over all keys).
hipError_t launch_gemm_nt_f32_product(const GemmArgs &a, hipStream_t stream);

// Per (token, head): exact top-k of each half's n scores, the exact top-k of
// the k*k candidates and the softmax.  scores [B][H][2][n] -> idx, w
// [B][H][k].  k <= 64, n <= 4096.  The staircase of candidate cells the
// kernel ranks first is a table in the library's device code (one row per
// k), so the call needs no workspace.
hipError_t launch_select(const float *scores, int64_t B, int H, int n, int k, int32_t *idx, float *w,
                         hipStream_t stream);

// a4-a7 in one kernel, one workgroup per token: the selection of every
// head, then the gather of the token's H k rows (value_type as
// launch_gather), bitwise the same as launch_select followed by
// launch_gather.  idx / w [B][H][k] are written when non-NULL (both or
// neither).  Only for the shapes select_gather_fusable accepts (n_keys 1024
// or 2048, H k <= 512, table rows longer than 512 bytes).
bool select_gather_fusable(int H, int n, int k, int value_type, int D);
hipError_t launch_select_gather(const float *scores, int64_t B, int H, int n, int k, const void *values,
                                const float *scale, int value_type, int D, int N, int32_t *idx, float *w, float *out,
                                hipStream_t stream);

// The candidate cells (i, j) with (i+1)(j+1) <= k: staircase_cells(k) of
// them (at most 280 for k <= 64), padded to kMaxStaircaseCells per k.
constexpr int kMaxStaircaseCells = 320;
int staircase_cells(int k);

// out[b][:] = sum_r w[b][r] * scale[row] * values[row][:], row = idx[b][r],
// r < R, N table rows (rows are clamped into [0, N)).  value_type: 0 f32,
// 1 bf16, 2 E4M3 (+ row scale).
// Exact top-k (k <= 64, k <= len) of each of `rows` rows of `len` fp32
// scores, by (score desc, index asc): idx [rows][k] int32 and top [rows][k].
// buf0 holds rows * flat_topk_keys_per_row(len, k) packed keys, buf1 rows *
// ceil(flat_topk_keys_per_row(len, k) / 2048) * k.
int64_t flat_topk_keys_per_row(int64_t len, int k);
hipError_t launch_flat_topk(const float *scores, int64_t rows, int64_t len, int k, uint64_t *buf0, uint64_t *buf1,
                            int32_t *idx, float *top, hipStream_t stream);
// The same top-k for rows longer than 4096 with group maxima: gmax [rows][G]
// holds the largest score of each group of 64 (G = ceil(len / 64)).  The
// k-th largest group maximum, theta, is found first (launch_flat_topk over
// gmax, with buf0 / buf1 sized for rows of G and tidx / ttop [rows][k]);
// then the scores >= theta go to list [rows][kFlatListCap] (count [rows]
// counts them) and the list's top-k is the row's.  A row whose list
// overflows is scanned in full by one wave.
constexpr int kFlatListCap = 512;
hipError_t launch_flat_topk_threshold(const float *scores, const float *gmax, int64_t rows, int64_t len, int k,
                                      uint64_t *buf0, uint64_t *buf1, int32_t *tidx, float *ttop, uint32_t *count,
                                      uint64_t *list, int32_t *idx, float *top, hipStream_t stream);

hipError_t launch_gather(const void *values, const float *scale, int value_type, int D, int N, int64_t B, int R,
                         const int32_t *idx, const float *w, float *out, hipStream_t stream);

// ---- backward direction (backward.hip)
hipError_t launch_fill(uint32_t *p, int64_t count, uint32_t value, hipStream_t st);
// out[c][r] = in[r][c] (optionally BN of column c) for r < R, c < C; zero for
// R <= r < Rp.
hipError_t launch_transpose(const float *in, int64_t ld_in, int R, int C, float *out, int64_t ld_out, int Rp,
                            const float *mean, const float *var, const float *gamma, const float *beta, float eps,
                            hipStream_t st);
// dt [B][H][k]: softmax backward of g_j = dout_b . V[idx_j].
hipError_t launch_value_backward(const void *values, const float *scale, int value_type, int D, int N, int64_t B,
                                 int H, int k, const int32_t *idx, const float *w, const float *dout, float *dt,
                                 hipStream_t st);
// dqhat, dq [B][H][D] and the half-score gradients G [2H][n][ldG] (columns
// b < B; G must be zero beforehand).
hipError_t launch_dqhat(const float *subkeys, const float *var, const float *gamma, float eps, int D, int n, int64_t B,
                        int H, int k, const int32_t *idx, const float *dt, float *dqhat, float *dq, float *G,
                        int64_t ldG, hipStream_t st);
// dsub [2H][n][D/2] += sum over b < B (in order) of G[g][i][b] * BN(q)[b]
// restricted to head h = g / 2, half p = g % 2; q [B][H*D] before BN.
hipError_t launch_dsub(const float *G, int64_t ldG, int64_t B, const float *q, int H, int D, int n, const float *mean,
                       const float *var, const float *gamma, const float *beta, float eps, float *dsub,
                       hipStream_t st);
// ---- batch statistics (batch_norm.hip)
// mean, var [cols] of q [B][cols] (biased var; B >= 2); part holds
// stat_part_floats(B, cols) floats; running stats updated when non-NULL.
int stat_chunks(int64_t B);
int64_t stat_part_floats(int64_t B, int cols);
hipError_t launch_batch_stats(const float *q, int64_t B, int cols, float *part, float *mean, float *var,
                              float *running_mean, float *running_var, float momentum, hipStream_t st);
// q = BN(q) in place with the given statistics (cols % 4 == 0).  With
// row_max non-NULL (cols and seg_cols multiples of 256): also each row's
// largest |q| per segment of seg_cols columns, by atomic max of the float
// bits into row_max[row * (cols / seg_cols) + col / seg_cols], which must
// start at zero.
hipError_t launch_bn_apply(float *q, int64_t B, int cols, const float *mean, const float *var, const float *gamma,
                           const float *beta, float eps, uint32_t *row_max, int seg_cols, hipStream_t st);
// BN backward with batch statistics: dq from dq^, q and the column sums
// sum_g = sum dq^ xhat, sum_b = sum dq^ of the batch
hipError_t launch_bn_batch_dq(const float *dqh, const float *q, int64_t B, int cols, const float *mean,
                              const float *var, const float *gamma, float eps, const float *sum_g, const float *sum_b,
                              float *dq, hipStream_t st);

// dgamma, dbeta [cols] += column sums over B rows of dqhat * xhat and dqhat,
// xhat = (q - mean) / sqrt(var + eps); part_g / part_b hold
// colsum_chunks(B) * cols floats each.
int colsum_chunks(int64_t B);
// (either may be NULL), and the sums themselves are written to sum_g /
// sum_b when those are non-NULL.
hipError_t launch_bn_grads(const float *dqhat, const float *q, const float *mean, const float *var, float eps,
                           int64_t B, int cols, float *part_g, float *part_b, float *dgamma, float *dbeta,
                           float *sum_g, float *sum_b, hipStream_t st);
// dval [N][D] += sum over the M occurrences o (row idx[o]) of w[o] *
// dout[o / per_token]; count, cursor, offs [N], block_sum [scan_blocks(N)],
// list [M] are scratch.
int64_t scan_blocks(int N);
// counts [N] += occurrences of each row among idx [M] (clamped into [0, N))
hipError_t launch_usage(const int32_t *idx, int64_t M, int N, uint32_t *counts, hipStream_t st);
// rows non-NULL: the sparse form instead -- the U distinct rows among idx in
// increasing order to rows [U], their sums to dval [U][D] (not added to),
// U to *row_count (device int64).
hipError_t launch_value_grad(const int32_t *idx, int64_t M, int N, int D, int per_token, const float *w,
                             const float *dout, uint32_t *count, uint32_t *cursor, uint32_t *offs,
                             uint32_t *block_sum, uint32_t *list, float *dval, int32_t *rows, int64_t *row_count,
                             hipStream_t st);

}  // namespace pkm
