// Step a7: out[b,:] = sum_r w[b,r] * scale[row] * values[row,:], row = idx[b,r]
// -- the gather and weighted sum EmbeddingBag(mode="sum", per_sample_weights)
// performs in one pass ("Product-Key Memory", the note after the code
// listing: the table is never touched as a dense matrix, only the selected
// rows are read).
//
// This is the HBM-bound step: every selected row is a random 0.5-4 KiB read.
// A wave64 owns one (token, column slice) -- or a whole token when its rows
// are exactly two slices long (gather_two_slices): each lane reads 16 contiguous bytes
// of a row (4 fp32, 8 bf16, 16 E4M3 or int8, or 32 int4 values), so one
// row-slice is one fully coalesced 1 KiB request, and keeps its fp32 partial
// sums in registers.  Scaled formats (E4M3, int8, int4) fold the row's scale
// into the weight.  The
// token's (row, weight) pairs are read once into lanes and broadcast with
// v_readlane, so every row address is a scalar base plus the lane offset.
// Sixteen row loads are issued before any is consumed to keep enough bytes in
// flight per wave (non-temporal when the launch seldom repeats a row).  Rows are summed in their given order, so results are
// bitwise reproducible.  A row index outside [0, N) is clamped into range
// (memory-safe; the result for such a row is meaningless).
#include "gather_dev.h"
#include "pkm_internal.h"

namespace pkm {
namespace {

using namespace gdev;

// Waves per workgroup: eight for the slice kernel (measured 4 / 8 / 16 at
// the default shape and large_memory: 8 the fastest for the bf16, E4M3 and
// int8 tables), four for the paired kernel (int4 rows: 8 was 12 % slower).
constexpr int WAVES = 8;
constexpr int PAIR_WAVES = 4;
constexpr int kPairSplit = 2;  // waves per token in gather_pair_kernel

template <int VT, bool NT>
__global__ __launch_bounds__(64 * WAVES) void gather_kernel(const uint8_t *__restrict__ values,
                                                            const float *__restrict__ scale, int D, int N, int64_t B, int R,
                                                            int slices, const int32_t *__restrict__ idx,
                                                            const float *__restrict__ w, float *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
    if (slices == 2) {  // one wave per token reads its rows whole
        if (wid < B) gather_two_slices<VT, NT>(values, scale, D, N, R, idx + wid * R, w + wid * R, out + wid * D, lane);
        return;
    }
    if (wid >= B * slices) return;
    const int64_t b = wid / slices;
    const int s = (int)(wid - b * slices);
    gather_slice<VT, NT>(values, scale, D, N, R, s, idx + b * R, w + b * R, out + b * D, lane);
}

// Rows of at most 512 bytes (an int4 row at D = 1024, for one) fill only 32
// lanes.  Then SPLIT waves share a token (gather_pair_share) and their sums
// are combined in a fixed order: odd rows onto even rows within a wave, then
// the later waves onto the first through LDS.  (Measured at D = 1024, int4:
// SPLIT 2 is the fastest of 1, 2 and 4, all near 4 TB/s: 512-byte random
// rows.)
template <int VT, int SPLIT, bool NT>
__global__ __launch_bounds__(64 * PAIR_WAVES) void gather_pair_kernel(const uint8_t *__restrict__ values,
                                                                 const float *__restrict__ scale, int D, int N,
                                                                 int64_t B, int R, const int32_t *__restrict__ idx,
                                                                 const float *__restrict__ w,
                                                                 float *__restrict__ out)
{
    constexpr int EPL = Fmt<VT>::EPL;
    __shared__ float part[SPLIT > 1 ? SPLIT - 1 : 1][PAIR_WAVES / SPLIT][EPL][32];
    const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) % SPLIT, slot = (threadIdx.x >> 6) / SPLIT;
    const int64_t b = (int64_t)blockIdx.x * (PAIR_WAVES / SPLIT) + slot;
    if ((int64_t)blockIdx.x * (PAIR_WAVES / SPLIT) >= B) return;  // whole workgroup past the end
    const bool live = b < B;
    const int64_t bb = live ? b : 0;
    float acc[EPL];
    gather_pair_share<VT, SPLIT, NT>(values, scale, D, N, R, wave, live, idx + bb * R, w + bb * R, acc, lane);
    const int half = lane >> 5;
    const bool active = (lane & 31) * EPL < D;
    if constexpr (SPLIT > 1) {
        if (wave > 0 && half == 0) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) part[wave - 1][slot][e][lane] = acc[e];
        }
        __syncthreads();
    }
    if (live && wave == 0 && half == 0 && active) {
#pragma unroll
        for (int q = 0; q < SPLIT - 1; ++q)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] += part[q][slot][e][lane];
        float4 *o = reinterpret_cast<float4 *>(out + b * D + (lane & 31) * EPL);
#pragma unroll
        for (int e = 0; e < EPL / 4; ++e) o[e] = make_float4(acc[4 * e], acc[4 * e + 1], acc[4 * e + 2], acc[4 * e + 3]);
    }
}
template <int VT>
hipError_t launch(const void *values, const float *scale, int D, int N, int64_t B, int R, const int32_t *idx,
                  const float *w, float *out, hipStream_t stream)
{
    const bool nt = B * R < N;
    const uint8_t *v = static_cast<const uint8_t *>(values);
    if (elem_bytes<VT>(D) <= 512) {
        constexpr int SPLIT = kPairSplit;
        const int64_t blocks = (B + PAIR_WAVES / SPLIT - 1) / (PAIR_WAVES / SPLIT);
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        if (nt)
            hipLaunchKernelGGL((gather_pair_kernel<VT, SPLIT, true>), dim3((unsigned)blocks), dim3(64 * PAIR_WAVES),
                               0, stream, v, scale, D, N, B, R, idx, w, out);
        else
            hipLaunchKernelGGL((gather_pair_kernel<VT, SPLIT, false>), dim3((unsigned)blocks), dim3(64 * PAIR_WAVES),
                               0, stream, v, scale, D, N, B, R, idx, w, out);
        return hipGetLastError();
    }
    const int width = 64 * Fmt<VT>::EPL;  // columns per wave
    const int slices = (D + width - 1) / width;
    const int64_t waves = B * (slices == 2 ? 1 : slices);  // two slices: one wave per token
    const int64_t blocks = (waves + WAVES - 1) / WAVES;
    if (nt)
        hipLaunchKernelGGL((gather_kernel<VT, true>), dim3((unsigned)blocks), dim3(64 * WAVES), 0, stream, v, scale,
                           D, N, B, R, slices, idx, w, out);
    else
        hipLaunchKernelGGL((gather_kernel<VT, false>), dim3((unsigned)blocks), dim3(64 * WAVES), 0, stream, v, scale,
                           D, N, B, R, slices, idx, w, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gather(const void *values, const float *scale, int value_type, int D, int N, int64_t B, int R,
                         const int32_t *idx, const float *w, float *out, hipStream_t stream)
{
    if (B <= 0) return hipSuccess;
    switch (value_type) {
    case 0: return launch<0>(values, scale, D, N, B, R, idx, w, out, stream);
    case 1: return launch<1>(values, scale, D, N, B, R, idx, w, out, stream);
    case 2: return launch<2>(values, scale, D, N, B, R, idx, w, out, stream);
    case 3: return launch<3>(values, scale, D, N, B, R, idx, w, out, stream);
    default: return launch<4>(values, scale, D, N, B, R, idx, w, out, stream);
    }
}

}  // namespace pkm
