// Device code of step a7 (the weighted gather-sum) shared by the gather
// kernels and by the fused select-and-gather kernel: the table formats, the
// loads of a lane's 16 bytes of a row, their decode and accumulation, and
// one wave's share of a token's rows.  Every function sums rows in the order
// given, so every kernel built from them is bitwise reproducible and two
// kernels that give a wave the same share agree bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkm {
namespace gdev {

constexpr int UNROLL = 16;  // row loads in flight per wave

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

// One wave's column slice s of token rows: lane l owns columns
// (64 s + l) EPL .. + EPL - 1 and sums the R rows ib[r] with weights wb[r]
// (ib / wb in global memory or LDS) in order r = 0 .. R - 1, then writes
// its columns of out_row.
template <int VT, bool NT, int UN = UNROLL>
__device__ __forceinline__ void gather_slice(const uint8_t *__restrict__ values, const float *__restrict__ scale, int D,
                                             int N, int R, int s, const int32_t *ib, const float *wb,
                                             float *__restrict__ out_row, int lane)
{
    constexpr int EPL = Fmt<VT>::EPL;
    constexpr bool SCALED = VT >= 2;
    const int c0 = (s * 64 + lane) * EPL;  // first column of this lane
    const bool active = c0 < D;
    const int64_t row_bytes = elem_bytes<VT>(D);
    const uint8_t *col = values + (active ? elem_bytes<VT>(c0) : 0);

    float acc[EPL], wsum = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;

    for (int r0 = 0; r0 < R; r0 += 64) {
        const int nr = min(64, R - r0);
        const int my_row = lane < nr ? ib[r0 + lane] : 0;
        // the weights, times the row scales, for up to 64 rows at once (one
        // load per lane rather than one per row)
        float my_w = lane < nr ? wb[r0 + lane] : 0.0f;
        if constexpr (SCALED) my_w *= lane < nr ? scale[min(max(my_row, 0), N - 1)] : 0.0f;
        int r = 0;
        for (; r + UN <= nr; r += UN) {
            uint4 v[UN];
            float wt[UN];
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                const int row = min(max(__builtin_amdgcn_readlane(my_row, r + u), 0), N - 1);
                wt[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), r + u));
                v[u] = active ? load_row_piece<NT>(col + (int64_t)row * row_bytes) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                accumulate<VT>(acc, v[u], wt[u]);
                if constexpr (VT == 4) wsum += wt[u];
            }
        }
        for (; r < nr; ++r) {
            const int row = min(max(__builtin_amdgcn_readlane(my_row, r), 0), N - 1);
            const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), r));
            const uint4 v = active ? load_row_piece<NT>(col + (int64_t)row * row_bytes) : make_uint4(0, 0, 0, 0);
            accumulate<VT>(acc, v, wt);
            if constexpr (VT == 4) wsum += wt;
        }
    }
    int4_offset_sum<VT>(acc, wsum);
    if (active) {
        float4 *o = reinterpret_cast<float4 *>(out_row + c0);
#pragma unroll
        for (int e = 0; e < EPL / 4; ++e) o[e] = make_float4(acc[4 * e], acc[4 * e + 1], acc[4 * e + 2], acc[4 * e + 3]);
    }
}

// A token's rows spanning exactly two column slices, read whole by one wave:
// lane l owns columns l EPL .. + EPL - 1 of the first slice and
// (64 + l) EPL .. of the second, the two pieces of a row loaded back to back
// (UN rows, 2 UN pieces in flight).  Measured at the default shape against
// two waves each reading one slice of every row: the stand-alone bf16 gather
// 180.8 -> 177.9 us, the fused select-gather 211 -> 207 us.  Every column
// sums the rows in the order gather_slice does, so the results are bitwise
// those of the two slices done separately.
template <int VT, bool NT, int UN = UNROLL / 2>
__device__ __forceinline__ void gather_two_slices(const uint8_t *__restrict__ values, const float *__restrict__ scale,
                                                  int D, int N, int R, const int32_t *ib, const float *wb,
                                                  float *__restrict__ out_row, int lane)
{
    constexpr int EPL = Fmt<VT>::EPL;
    constexpr bool SCALED = VT >= 2;
    const int c0 = lane * EPL, c1 = (64 + lane) * EPL;
    const bool act0 = c0 < D, act1 = c1 < D;
    const int64_t row_bytes = elem_bytes<VT>(D);
    const uint8_t *col0 = values + (act0 ? elem_bytes<VT>(c0) : 0);
    const uint8_t *col1 = values + (act1 ? elem_bytes<VT>(c1) : 0);

    float a0[EPL], a1[EPL], wsum = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        a0[e] = 0.0f;
        a1[e] = 0.0f;
    }
    for (int r0 = 0; r0 < R; r0 += 64) {
        const int nr = min(64, R - r0);
        const int my_row = lane < nr ? ib[r0 + lane] : 0;
        float my_w = lane < nr ? wb[r0 + lane] : 0.0f;
        if constexpr (SCALED) my_w *= lane < nr ? scale[min(max(my_row, 0), N - 1)] : 0.0f;
        int r = 0;
        for (; r + UN <= nr; r += UN) {
            uint4 v[UN][2];
            float wt[UN];
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                const int64_t off = (int64_t)min(max(__builtin_amdgcn_readlane(my_row, r + u), 0), N - 1) * row_bytes;
                wt[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), r + u));
                v[u][0] = act0 ? load_row_piece<NT>(col0 + off) : make_uint4(0, 0, 0, 0);
                v[u][1] = act1 ? load_row_piece<NT>(col1 + off) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                accumulate<VT>(a0, v[u][0], wt[u]);
                accumulate<VT>(a1, v[u][1], wt[u]);
                if constexpr (VT == 4) wsum += wt[u];
            }
        }
        for (; r < nr; ++r) {
            const int64_t off = (int64_t)min(max(__builtin_amdgcn_readlane(my_row, r), 0), N - 1) * row_bytes;
            const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), r));
            accumulate<VT>(a0, act0 ? load_row_piece<NT>(col0 + off) : make_uint4(0, 0, 0, 0), wt);
            accumulate<VT>(a1, act1 ? load_row_piece<NT>(col1 + off) : make_uint4(0, 0, 0, 0), wt);
            if constexpr (VT == 4) wsum += wt;
        }
    }
    int4_offset_sum<VT>(a0, wsum);
    int4_offset_sum<VT>(a1, wsum);
    if (act0) {
        float4 *o = reinterpret_cast<float4 *>(out_row + c0);
#pragma unroll
        for (int e = 0; e < EPL / 4; ++e) o[e] = make_float4(a0[4 * e], a0[4 * e + 1], a0[4 * e + 2], a0[4 * e + 3]);
    }
    if (act1) {
        float4 *o = reinterpret_cast<float4 *>(out_row + c1);
#pragma unroll
        for (int e = 0; e < EPL / 4; ++e) o[e] = make_float4(a1[4 * e], a1[4 * e + 1], a1[4 * e + 2], a1[4 * e + 3]);
    }
}

// Rows of at most 512 bytes fill only 32 lanes: SPLIT waves share a token,
// wave `wave` taking the contiguous share [wave * ceil(R / SPLIT), ...) of
// its rows, and within a wave lanes 0-31 take the even rows of the share,
// lanes 32-63 the odd ones.  On return lanes 0-31 hold the wave's sums
// (odd rows added onto even rows) for columns (lane & 31) EPL .. + EPL - 1;
// the caller adds the later waves' sums onto the first's, in wave order.
template <int VT, int SPLIT, bool NT, int UN = UNROLL>
__device__ __forceinline__ void gather_pair_share(const uint8_t *__restrict__ values, const float *__restrict__ scale,
                                                  int D, int N, int R, int wave, bool live, const int32_t *ib,
                                                  const float *wb, float (&acc)[Fmt<VT>::EPL], int lane)
{
    constexpr int EPL = Fmt<VT>::EPL;
    constexpr bool SCALED = VT >= 2;
    const int half = lane >> 5;
    const int c0 = (lane & 31) * EPL;
    const bool active = c0 < D;
    const int64_t row_bytes = elem_bytes<VT>(D);
    const uint8_t *col = values + (active ? elem_bytes<VT>(c0) : 0);

    float wsum = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;

    const int share = (R + SPLIT - 1) / SPLIT;
    const int rb = live ? min(R, wave * share) : 0, re = live ? min(R, rb + share) : 0;
    for (int r0 = rb; r0 < re; r0 += 64) {
        const int nr = min(64, re - r0);
        const int my_row = lane < nr ? ib[r0 + lane] : 0;
        // the weights, times the row scales, for up to 64 rows at once
        float my_w = lane < nr ? wb[r0 + lane] : 0.0f;
        if constexpr (SCALED) my_w *= lane < nr ? scale[min(max(my_row, 0), N - 1)] : 0.0f;
        const int pairs = (nr + 1) >> 1;
        for (int t0 = 0; t0 < pairs; t0 += UN) {
            uint4 v[UN];
            float wt[UN];
#pragma unroll
            for (int u = 0; u < UN; ++u) {
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
            for (int u = 0; u < UN; ++u) {
                accumulate<VT>(acc, v[u], wt[u]);
                if constexpr (VT == 4) wsum += wt[u];
            }
        }
    }
    int4_offset_sum<VT>(acc, wsum);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += __shfl_xor(acc[e], 32, 64);
}

}  // namespace gdev
}  // namespace pkm
