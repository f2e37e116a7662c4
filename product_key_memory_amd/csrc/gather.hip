// Step a7: out[b,:] = sum_r w[b,r] * scale[row] * values[row,:], row = idx[b,r]
// -- the gather and weighted sum EmbeddingBag(mode="sum", per_sample_weights)
// performs in one pass ("Product-Key Memory", the note after the code
// listing: the table is never touched as a dense matrix, only the selected
// rows are read).
//
// This is the HBM-bound step: every selected row is a random 0.5-4 KiB read.
// A wave64 owns one (token, column slice): each lane reads 16 contiguous bytes
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
#include "pkm_internal.h"

namespace pkm {
namespace {

constexpr int WAVES = 4;
constexpr int UNROLL = 16;  // row loads in flight per wave
constexpr int kPairSplit = 2;  // waves per token in gather_pair_kernel

template <int VT>
struct Fmt;
template <>
struct Fmt<0> {  // fp32
    static constexpr int EPL = 4;
    static constexpr int BYTES = 4;
};
template <>
struct Fmt<1> {  // bf16
    static constexpr int EPL = 8;
    static constexpr int BYTES = 2;
};
template <>
struct Fmt<2> {  // OCP E4M3 + row scale
    static constexpr int EPL = 16;
    static constexpr int BYTES = 1;
};
template <>
struct Fmt<3> {  // int8 + row scale
    static constexpr int EPL = 16;
    static constexpr int BYTES = 1;
};
template <>
struct Fmt<4> {  // two's complement int4, two per byte (even element low) + row scale
    static constexpr int EPL = 32;
    static constexpr int BYTES = 0;  // half a byte per element: see elem_bytes
};

// bytes of a row up to element c (c a multiple of EPL)
template <int VT>
__host__ __device__ __forceinline__ int64_t elem_bytes(int64_t c)
{
    return VT == 4 ? c / 2 : c * Fmt<VT>::BYTES;
}

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

// One lane's 16 bytes of a table row.  NT: a non-temporal load, for
// launches that read fewer rows than the table holds (B R < N), where a row
// is seldom read twice and keeping it would only displace the rest of the
// step's data (the default shape: 2-3 % faster steps).  With more reads than
// rows (e.g. 16,384 tokens of 128 rows over 1M rows) repeats are common and
// plain loads let the caches serve them (2 % faster there).
template <bool NT>
__device__ __forceinline__ uint4 load_row_piece(const uint8_t *p)
{
    if constexpr (NT) {
        const u4v t = __builtin_nontemporal_load(reinterpret_cast<const u4v *>(p));
        return make_uint4(t[0], t[1], t[2], t[3]);
    }
    return *reinterpret_cast<const uint4 *>(p);
}

template <int VT>
__device__ __forceinline__ void accumulate(float (&acc)[Fmt<VT>::EPL], const uint4 &v, float wt)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (VT == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(wt, __uint_as_float(w[i]), acc[i]);
    } else if constexpr (VT == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(wt, __uint_as_float(w[i] << 16), acc[2 * i]);
            acc[2 * i + 1] = fmaf(wt, __uint_as_float(w[i] & 0xFFFF0000u), acc[2 * i + 1]);
        }
    } else if constexpr (VT == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const floatx2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
            const floatx2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
            acc[4 * i + 0] = fmaf(wt, lo.x, acc[4 * i + 0]);
            acc[4 * i + 1] = fmaf(wt, lo.y, acc[4 * i + 1]);
            acc[4 * i + 2] = fmaf(wt, hi.x, acc[4 * i + 2]);
            acc[4 * i + 3] = fmaf(wt, hi.y, acc[4 * i + 3]);
        }
    } else if constexpr (VT == 3) {
        // byte j of a word, sign-extended (signed bit-field extract)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[4 * i + j] = fmaf(wt, (float)(int32_t)__builtin_amdgcn_sbfe((int)w[i], 8 * j, 8), acc[4 * i + j]);
    } else {
        // Nibble j of word i is element 8 i + j.  Flipping bit 3 of every
        // nibble turns the two's complement value v into v + 8 in [0, 15];
        // nibbles j and j + 4 then sit in the low bits of the word's two
        // fp16 halves after one shift and mask, each half the fp16
        // subnormal (v + 8) 2^-24, which the mixed fp16/fp32 FMA widens
        // exactly: acc += (wt 2^24) ((v + 8) 2^-24) = wt (v + 8), two
        // instructions per element instead of extract, convert and FMA.
        // The caller takes the 8 sum(wt) back off (int4_offset_sum).
        const float wt24 = wt * 0x1p24f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t x = w[i] ^ 0x88888888u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const halfx2 h = __builtin_bit_cast(halfx2, (x >> (4 * j)) & 0x000F000Fu);
                acc[8 * i + j] = fmaf(wt24, (float)h.x, acc[8 * i + j]);
                acc[8 * i + j + 4] = fmaf(wt24, (float)h.y, acc[8 * i + j + 4]);
            }
        }
    }
}

// int4 rows accumulate wt (v + 8) (see accumulate): subtract 8 times the sum
// of the weights the lane applied, once, exactly scaled (one rounding).
template <int VT>
__device__ __forceinline__ void int4_offset_sum(float (&acc)[Fmt<VT>::EPL], float wsum)
{
    if constexpr (VT == 4)
#pragma unroll
        for (int e = 0; e < Fmt<VT>::EPL; ++e) acc[e] = fmaf(-8.0f, wsum, acc[e]);
}

template <int VT, bool NT>
__global__ __launch_bounds__(64 * WAVES) void gather_kernel(const uint8_t *__restrict__ values,
                                                            const float *__restrict__ scale, int D, int N, int64_t B, int R,
                                                            int slices, const int32_t *__restrict__ idx,
                                                            const float *__restrict__ w, float *__restrict__ out)
{
    constexpr int EPL = Fmt<VT>::EPL;
    constexpr bool SCALED = VT >= 2;
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
    if (wid >= B * slices) return;
    const int64_t b = wid / slices;
    const int s = (int)(wid - b * slices);
    const int c0 = (s * 64 + lane) * EPL;  // first column of this lane
    const bool active = c0 < D;
    const int64_t row_bytes = elem_bytes<VT>(D);
    const uint8_t *col = values + (active ? elem_bytes<VT>(c0) : 0);

    float acc[EPL], wsum = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;

    const int32_t *ib = idx + b * R;
    const float *wb = w + b * R;
    for (int r0 = 0; r0 < R; r0 += 64) {
        const int nr = min(64, R - r0);
        const int my_row = lane < nr ? ib[r0 + lane] : 0;
        const float my_w = lane < nr ? wb[r0 + lane] : 0.0f;
        int r = 0;
        for (; r + UNROLL <= nr; r += UNROLL) {
            uint4 v[UNROLL];
            float wt[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int row = min(max(__builtin_amdgcn_readlane(my_row, r + u), 0), N - 1);
                wt[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), r + u));
                if constexpr (SCALED) wt[u] *= scale[row];
                v[u] = active ? load_row_piece<NT>(col + (int64_t)row * row_bytes) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                accumulate<VT>(acc, v[u], wt[u]);
                if constexpr (VT == 4) wsum += wt[u];
            }
        }
        for (; r < nr; ++r) {
            const int row = min(max(__builtin_amdgcn_readlane(my_row, r), 0), N - 1);
            float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), r));
            if constexpr (SCALED) wt *= scale[row];
            const uint4 v = active ? load_row_piece<NT>(col + (int64_t)row * row_bytes) : make_uint4(0, 0, 0, 0);
            accumulate<VT>(acc, v, wt);
            if constexpr (VT == 4) wsum += wt;
        }
    }
    int4_offset_sum<VT>(acc, wsum);
    if (active) {
        float4 *o = reinterpret_cast<float4 *>(out + b * D + c0);
#pragma unroll
        for (int e = 0; e < EPL / 4; ++e) o[e] = make_float4(acc[4 * e], acc[4 * e + 1], acc[4 * e + 2], acc[4 * e + 3]);
    }
}

// Rows of at most 512 bytes (an int4 row at D = 1024, for one) fill only 32
// lanes.  Then SPLIT waves share a token, each taking a contiguous share of
// its rows, and within a wave the two halves take alternate rows (lanes 0-31
// the even ones, 32-63 the odd ones), each lane loading its 16 bytes of its
// half's row, so every lane issues a full load.  The sums are combined in a
// fixed order: odd rows onto even rows within a wave, then the later waves
// onto the first through LDS.  (Measured at D = 1024, int4: SPLIT 2 is the
// fastest of 1, 2 and 4, all near 4 TB/s: 512-byte random rows.)
template <int VT, int SPLIT, bool NT>
__global__ __launch_bounds__(64 * WAVES) void gather_pair_kernel(const uint8_t *__restrict__ values,
                                                                 const float *__restrict__ scale, int D, int N,
                                                                 int64_t B, int R, const int32_t *__restrict__ idx,
                                                                 const float *__restrict__ w,
                                                                 float *__restrict__ out)
{
    constexpr int EPL = Fmt<VT>::EPL;
    constexpr bool SCALED = VT >= 2;
    __shared__ float part[SPLIT > 1 ? SPLIT - 1 : 1][WAVES / SPLIT][EPL][32];
    const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) % SPLIT, slot = (threadIdx.x >> 6) / SPLIT;
    const int64_t b = (int64_t)blockIdx.x * (WAVES / SPLIT) + slot;
    if ((int64_t)blockIdx.x * (WAVES / SPLIT) >= B) return;  // whole workgroup past the end
    const bool live = b < B;
    const int half = lane >> 5;
    const int c0 = (lane & 31) * EPL;
    const bool active = c0 < D;
    const int64_t row_bytes = elem_bytes<VT>(D);
    const uint8_t *col = values + (active ? elem_bytes<VT>(c0) : 0);

    float acc[EPL], wsum = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;

    const int share = (R + SPLIT - 1) / SPLIT;
    const int rb = live ? min(R, wave * share) : 0, re = live ? min(R, rb + share) : 0;
    const int32_t *ib = idx + (live ? b : 0) * R;
    const float *wb = w + (live ? b : 0) * R;
    for (int r0 = rb; r0 < re; r0 += 64) {
        const int nr = min(64, re - r0);
        const int my_row = lane < nr ? ib[r0 + lane] : 0;
        // the weights, times the row scales, for up to 64 rows at once
        float my_w = lane < nr ? wb[r0 + lane] : 0.0f;
        if constexpr (SCALED) my_w *= lane < nr ? scale[min(max(my_row, 0), N - 1)] : 0.0f;
        const int pairs = (nr + 1) >> 1;
        for (int t0 = 0; t0 < pairs; t0 += UNROLL) {
            uint4 v[UNROLL];
            float wt[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                // the pair's two rows by readlane (it reads a lane whatever the
                // execution mask, unlike a cross-lane shuffle), then this half's
                const int je = min(2 * (t0 + u), nr - 1), jo = min(2 * (t0 + u) + 1, nr - 1);
                const int row_e = __builtin_amdgcn_readlane(my_row, je), row_o = __builtin_amdgcn_readlane(my_row, jo);
                const float w_e = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), je));
                const float w_o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), jo));
                const bool ok = 2 * (t0 + u) + half < nr;
                const int row = min(max(half ? row_o : row_e, 0), N - 1);
                wt[u] = ok ? (half ? w_o : w_e) : 0.0f;
                v[u] = active && ok ? load_row_piece<NT>(col + (int64_t)row * row_bytes) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                accumulate<VT>(acc, v[u], wt[u]);
                if constexpr (VT == 4) wsum += wt[u];
            }
        }
    }
    int4_offset_sum<VT>(acc, wsum);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += __shfl_xor(acc[e], 32, 64);
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
        float4 *o = reinterpret_cast<float4 *>(out + b * D + c0);
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
        const int64_t blocks = (B + WAVES / SPLIT - 1) / (WAVES / SPLIT);
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        if (nt)
            hipLaunchKernelGGL((gather_pair_kernel<VT, SPLIT, true>), dim3((unsigned)blocks), dim3(64 * WAVES), 0,
                               stream, v, scale, D, N, B, R, idx, w, out);
        else
            hipLaunchKernelGGL((gather_pair_kernel<VT, SPLIT, false>), dim3((unsigned)blocks), dim3(64 * WAVES), 0,
                               stream, v, scale, D, N, B, R, idx, w, out);
        return hipGetLastError();
    }
    const int width = 64 * Fmt<VT>::EPL;  // columns per wave
    const int slices = (D + width - 1) / width;
    const int64_t waves = B * slices;
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
