// BatchNorm of the query with batch statistics (the training-mode reading
// of "Product-Key Memory", §Keeping the memory in use: the query is batch-
// normalised over the batch).  Per column c = h * D + f of q [B][H*D]:
//   mean = (1/B) sum_b q,  var = (1/B) sum_b (q - mean)^2   (biased)
// in one pass over q: each 64-row chunk's mean and sum of squared
// deviations from it (the chunk held in registers), then the chunks merged
// in order by the pairwise update of Chan, Golub and LeVeque ("Updating
// formulae and a pairwise algorithm for computing sample variances", 1979):
//   d = m_b - m_a,  m = m_a + d n_b / n,  M2 = M2_a + M2_b + d^2 n_a n_b / n
// (fixed order: bitwise reproducible); the running statistics move by
// r = (1 - m) r + m s (variance unbiased, times B / (B - 1)); q is then
// normalised in place, optionally recording each row's largest |q^| per
// segment of columns (the scoring's row exponents).  The backward with batch statistics couples the
// rows through the column sums of dq^ (sb) and dq^ * xhat (sg):
//   dq = gamma / sqrt(var + eps) * (dq^ - sb / B - xhat * sg / B).
#include "pkm_internal.h"
#include "wave_ops.h"

namespace pkm {
namespace {

constexpr int kStatChunk = 64;

unsigned grid_of(int64_t items, int per_block) { return (unsigned)((items + per_block - 1) / per_block); }

// part[0][chunk][col], part[1][chunk][col]: the chunk's mean of q and its
// sum of squared deviations from that mean, the chunk's rows in registers
__global__ __launch_bounds__(256) void colstat_chunk_kernel(const float *__restrict__ q, int64_t B, int cols,
                                                            int chunks, float *__restrict__ part)
{
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= cols) return;
    const int64_t r0 = (int64_t)blockIdx.y * kStatChunk;
    const int n = (int)min((int64_t)kStatChunk, B - r0);
    float v[kStatChunk];
#pragma unroll
    for (int i = 0; i < kStatChunk; ++i) v[i] = q[(r0 + min(i, n - 1)) * cols + col];  // rows past B unused
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kStatChunk; ++i)
        if (i < n) s += v[i];
    const float m = s / (float)n;
    float m2 = 0.0f;
#pragma unroll
    for (int i = 0; i < kStatChunk; ++i)
        if (i < n) m2 = fmaf(v[i] - m, v[i] - m, m2);
    part[(int64_t)blockIdx.y * cols + col] = m;
    part[((int64_t)chunks + blockIdx.y) * cols + col] = m2;
}

// The chunks merged in order into the column's mean and biased variance;
// the running statistics updated when given
__global__ __launch_bounds__(256) void colstat_merge_kernel(const float *__restrict__ part, int chunks, int cols,
                                                            int64_t B, float *__restrict__ mean,
                                                            float *__restrict__ var, float momentum,
                                                            float *__restrict__ rmean, float *__restrict__ rvar)
{
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= cols) return;
    float n = 0.0f, m = 0.0f, m2 = 0.0f;
#pragma unroll 8
    for (int c = 0; c < chunks; ++c) {
        const float nc = (float)min((int64_t)kStatChunk, B - (int64_t)c * kStatChunk);
        const float mc = part[(int64_t)c * cols + col];
        const float m2c = part[((int64_t)chunks + c) * cols + col];
        const float nn = n + nc;
        const float d = mc - m;
        m += d * (nc / nn);
        m2 += m2c + d * d * (n * nc / nn);
        n = nn;
    }
    const float v = m2 / (float)B;
    mean[col] = m;
    var[col] = v;
    if (rmean) {
        const float unbiased = v * ((float)B / (float)(B - 1));
        rmean[col] = (1.0f - momentum) * rmean[col] + momentum * m;
        rvar[col] = (1.0f - momentum) * rvar[col] + momentum * unbiased;
    }
}

// q = (q - mean) gamma / sqrt(var + eps) + beta, in place; float4 per thread.
// ROW_MAX: also the largest |q^| of each row per segment of seg_cols columns
// (seg_cols and cols multiples of 256, so a wave's 256 columns lie in one
// segment of one row), as float bits by atomic max into
// row_max[row * (cols / seg_cols) + col / seg_cols] (zeroed beforehand).
template <bool ROW_MAX>
__global__ __launch_bounds__(256) void bn_apply_kernel(float *__restrict__ q, int64_t B, int cols,
                                                       const float *__restrict__ mean, const float *__restrict__ var,
                                                       const float *__restrict__ gamma, const float *__restrict__ beta,
                                                       float eps, uint32_t *__restrict__ row_max, int seg_cols)
{
    const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;  // float4 index
    if (i4 * 4 >= B * cols) return;
    const int col = (int)((i4 * 4) % cols);
    float4 v = reinterpret_cast<float4 *>(q)[i4];
    const float4 m = *reinterpret_cast<const float4 *>(mean + col);
    const float4 s = *reinterpret_cast<const float4 *>(var + col);
    const float4 g = *reinterpret_cast<const float4 *>(gamma + col);
    const float4 b = *reinterpret_cast<const float4 *>(beta + col);
    v.x = (v.x - m.x) * (g.x / sqrtf(s.x + eps)) + b.x;
    v.y = (v.y - m.y) * (g.y / sqrtf(s.y + eps)) + b.y;
    v.z = (v.z - m.z) * (g.z / sqrtf(s.z + eps)) + b.z;
    v.w = (v.w - m.w) * (g.w / sqrtf(s.w + eps)) + b.w;
    reinterpret_cast<float4 *>(q)[i4] = v;
    if constexpr (ROW_MAX) {
        // every lane of the wave is live: B * cols is a multiple of 256
        float mx = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        mx = fmaxf(mx, __uint_as_float(xor_lane<1>(__float_as_uint(mx))));
        mx = fmaxf(mx, __uint_as_float(xor_lane<2>(__float_as_uint(mx))));
        mx = fmaxf(mx, __uint_as_float(xor_lane<4>(__float_as_uint(mx))));
        mx = fmaxf(mx, __uint_as_float(xor_lane<8>(__float_as_uint(mx))));
        mx = fmaxf(mx, __uint_as_float(xor_lane<16>(__float_as_uint(mx))));
        mx = fmaxf(mx, __uint_as_float(xor_lane<32>(__float_as_uint(mx))));
        if ((threadIdx.x & 63) == 0) {
            const int64_t row = i4 * 4 / cols;
            atomicMax(&row_max[row * (cols / seg_cols) + col / seg_cols], __float_as_uint(mx));
        }
    }
}

// dq = gamma / sqrt(var + eps) * (dq^ - sb / B - xhat * sg / B), xhat = (q - mean) / sqrt(var + eps)
__global__ __launch_bounds__(256) void bn_batch_dq_kernel(const float *__restrict__ dqh, const float *__restrict__ q,
                                                          int64_t B, int cols, const float *__restrict__ mean,
                                                          const float *__restrict__ var,
                                                          const float *__restrict__ gamma, float eps,
                                                          const float *__restrict__ sum_g,
                                                          const float *__restrict__ sum_b, float *__restrict__ dq)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= B * cols) return;
    const int col = (int)(i % cols);
    const float inv = 1.0f / sqrtf(var[col] + eps);
    const float xh = (q[i] - mean[col]) * inv;
    const float rb = 1.0f / (float)B;
    dq[i] = gamma[col] * inv * (dqh[i] - sum_b[col] * rb - xh * (sum_g[col] * rb));
}

}  // namespace

int stat_chunks(int64_t B) { return (int)((B + kStatChunk - 1) / kStatChunk); }
int64_t stat_part_floats(int64_t B, int cols) { return 2 * (int64_t)stat_chunks(B) * cols; }

hipError_t launch_batch_stats(const float *q, int64_t B, int cols, float *part, float *mean, float *var,
                              float *running_mean, float *running_var, float momentum, hipStream_t st)
{
    if (B < 2) return hipErrorInvalidValue;
    const int chunks = stat_chunks(B);
    if (chunks > 65535) return hipErrorInvalidConfiguration;
    const dim3 g2(grid_of(cols, 256), chunks), g1(grid_of(cols, 256));
    hipLaunchKernelGGL(colstat_chunk_kernel, g2, dim3(256), 0, st, q, B, cols, chunks, part);
    hipLaunchKernelGGL(colstat_merge_kernel, g1, dim3(256), 0, st, part, chunks, cols, B, mean, var, momentum,
                       running_mean, running_var);
    return hipGetLastError();
}

hipError_t launch_bn_apply(float *q, int64_t B, int cols, const float *mean, const float *var, const float *gamma,
                           const float *beta, float eps, uint32_t *row_max, int seg_cols, hipStream_t st)
{
    if (B <= 0) return hipSuccess;
    if (cols % 4) return hipErrorInvalidValue;
    const dim3 grid(grid_of(B * cols / 4, 256));
    if (row_max) {
        if (cols % 256 || seg_cols <= 0 || seg_cols % 256 || cols % seg_cols) return hipErrorInvalidValue;
        hipLaunchKernelGGL(bn_apply_kernel<true>, grid, dim3(256), 0, st, q, B, cols, mean, var, gamma, beta, eps,
                           row_max, seg_cols);
    } else {
        hipLaunchKernelGGL(bn_apply_kernel<false>, grid, dim3(256), 0, st, q, B, cols, mean, var, gamma, beta, eps,
                           nullptr, 0);
    }
    return hipGetLastError();
}

hipError_t launch_bn_batch_dq(const float *dqh, const float *q, int64_t B, int cols, const float *mean,
                              const float *var, const float *gamma, float eps, const float *sum_g, const float *sum_b,
                              float *dq, hipStream_t st)
{
    if (B <= 0) return hipSuccess;
    hipLaunchKernelGGL(bn_batch_dq_kernel, dim3(grid_of(B * cols, 256)), dim3(256), 0, st, dqh, q, B, cols, mean, var,
                       gamma, eps, sum_g, sum_b, dq);
    return hipGetLastError();
}

}  // namespace pkm
