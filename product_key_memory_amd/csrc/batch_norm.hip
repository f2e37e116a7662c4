// BatchNorm of the query with batch statistics (the training-mode reading
// of "Product-Key Memory", §Keeping the memory in use: the query is batch-
// normalised over the batch).  Per column c = h * D + f of q [B][H*D]:
//   mean = (1/B) sum_b q,  var = (1/B) sum_b (q - mean)^2   (biased)
// in two passes, each as partial sums over 64-row chunks added in chunk
// order (fixed order: bitwise reproducible); the running statistics move
// by r = (1 - m) r + m s (variance unbiased, times B / (B - 1)); q is then
// normalised in place.  The backward with batch statistics couples the
// rows through the column sums of dq^ (sb) and dq^ * xhat (sg):
//   dq = gamma / sqrt(var + eps) * (dq^ - sb / B - xhat * sg / B).
#include "pkm_internal.h"

namespace pkm {
namespace {

constexpr int kStatChunk = 64;

unsigned grid_of(int64_t items, int per_block) { return (unsigned)((items + per_block - 1) / per_block); }

// part[chunk][col]: sum over the chunk's rows of q (SQUARES false) or of
// (q - mean[col])^2 (SQUARES true)
template <bool SQUARES>
__global__ __launch_bounds__(256) void colstat_partial_kernel(const float *__restrict__ q, int64_t B, int cols,
                                                              const float *__restrict__ mean,
                                                              float *__restrict__ part)
{
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= cols) return;
    const int64_t r0 = (int64_t)blockIdx.y * kStatChunk, r1 = min(B, r0 + kStatChunk);
    const float mu = SQUARES ? mean[col] : 0.0f;
    float s = 0.0f;
    for (int64_t r = r0; r < r1; ++r) {
        const float v = q[r * cols + col];
        if (SQUARES)
            s = fmaf(v - mu, v - mu, s);
        else
            s += v;
    }
    part[(int64_t)blockIdx.y * cols + col] = s;
}

// out[col] = (sum over chunks, in order) / B
__global__ __launch_bounds__(256) void colstat_final_kernel(const float *__restrict__ part, int chunks, int cols,
                                                            int64_t B, float *__restrict__ out)
{
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= cols) return;
    float s = 0.0f;
    for (int c = 0; c < chunks; ++c) s += part[(int64_t)c * cols + col];
    out[col] = s / (float)B;
}

__global__ __launch_bounds__(256) void running_update_kernel(const float *__restrict__ mean,
                                                             const float *__restrict__ var, int cols, int64_t B,
                                                             float momentum, float *__restrict__ rmean,
                                                             float *__restrict__ rvar)
{
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= cols) return;
    const float unbiased = var[col] * ((float)B / (float)(B - 1));
    rmean[col] = (1.0f - momentum) * rmean[col] + momentum * mean[col];
    rvar[col] = (1.0f - momentum) * rvar[col] + momentum * unbiased;
}

// q = (q - mean) gamma / sqrt(var + eps) + beta, in place; float4 per thread
__global__ __launch_bounds__(256) void bn_apply_kernel(float *__restrict__ q, int64_t B, int cols,
                                                       const float *__restrict__ mean, const float *__restrict__ var,
                                                       const float *__restrict__ gamma, const float *__restrict__ beta,
                                                       float eps)
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

hipError_t launch_batch_stats(const float *q, int64_t B, int cols, float *part, float *mean, float *var,
                              float *running_mean, float *running_var, float momentum, hipStream_t st)
{
    if (B < 2) return hipErrorInvalidValue;
    const int chunks = stat_chunks(B);
    if (chunks > 65535) return hipErrorInvalidConfiguration;
    const dim3 g2(grid_of(cols, 256), chunks), g1(grid_of(cols, 256));
    hipLaunchKernelGGL(colstat_partial_kernel<false>, g2, dim3(256), 0, st, q, B, cols, nullptr, part);
    hipLaunchKernelGGL(colstat_final_kernel, g1, dim3(256), 0, st, part, chunks, cols, B, mean);
    hipLaunchKernelGGL(colstat_partial_kernel<true>, g2, dim3(256), 0, st, q, B, cols, mean, part);
    hipLaunchKernelGGL(colstat_final_kernel, g1, dim3(256), 0, st, part, chunks, cols, B, var);
    if (running_mean)
        hipLaunchKernelGGL(running_update_kernel, g1, dim3(256), 0, st, mean, var, cols, B, momentum, running_mean,
                           running_var);
    return hipGetLastError();
}

hipError_t launch_bn_apply(float *q, int64_t B, int cols, const float *mean, const float *var, const float *gamma,
                           const float *beta, float eps, hipStream_t st)
{
    if (B <= 0) return hipSuccess;
    if (cols % 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bn_apply_kernel, dim3(grid_of(B * cols / 4, 256)), dim3(256), 0, st, q, B, cols, mean, var,
                       gamma, beta, eps);
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
