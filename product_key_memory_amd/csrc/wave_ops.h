// Cross-lane exchanges for one wave64 on gfx950, without the LDS crossbar:
// xor_lane<S>(v) returns v from lane (lane ^ S), S a power of two < 64.
//   S = 1, 2   one DPP quad permutation
//   S = 4      DPP quad reverse (lane ^ 3) then row half-mirror (lane ^ 7)
//   S = 8      DPP row rotate by 8 inside a 16-lane row
//   S = 16     v_permlane16_swap (swaps odd rows of one copy with even rows
//              of the other), pick the copy that holds the partner row
//   S = 32     v_permlane32_swap (swaps the upper half of one copy with the
//              lower half of the other), same pick
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkm {

template <int S>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v)
{
    static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16 || S == 32, "power of two below 64");
    if constexpr (S == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (S == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else if constexpr (S == 4) {
        const int r = __builtin_amdgcn_mov_dpp((int)v, 0x1B, 0xF, 0xF, false);    // quad_perm [3,2,1,0]
        return (uint32_t)__builtin_amdgcn_mov_dpp(r, 0x141, 0xF, 0xF, false);      // row_half_mirror
    } else if constexpr (S == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false); // row_ror:8
    } else if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (__lane_id() & 16) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (__lane_id() & 32) ? r[0] : r[1];
    }
}

template <int S>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v)
{
    const uint32_t lo = xor_lane<S>((uint32_t)v);
    const uint32_t hi = xor_lane<S>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

template <int S, typename T>
__device__ __forceinline__ T xor_any(T v)
{
    if constexpr (sizeof(T) == 8)
        return (T)xor_lane64<S>((uint64_t)v);
    else
        return (T)xor_lane<S>((uint32_t)v);
}

// One compare-exchange step of a bitonic network over the wave: partner is
// lane ^ S; the lane keeps the larger value when `keep_max`.
template <int S, typename T>
__device__ __forceinline__ T cmp_xchg(T v, bool keep_max)
{
    const T o = xor_any<S>(v);
    return ((v > o) == keep_max) ? v : o;
}

// Bitonic merge steps with strides S, S/2, ..., 1 inside blocks of 2*S lanes;
// `desc` selects the direction of this lane's block.
template <int S, typename T>
__device__ __forceinline__ T merge_steps(T v, bool desc)
{
    const int lane = __lane_id();
    v = cmp_xchg<S>(v, ((lane & S) == 0) == desc);
    if constexpr (S > 1) v = merge_steps<S / 2>(v, desc);
    return v;
}

// Sorts one value per lane over the whole wave, descending with lane.
template <typename T>
__device__ __forceinline__ T sort64_desc(T v)
{
    const int lane = __lane_id();
    v = merge_steps<1>(v, (lane & 2) == 0);
    v = merge_steps<2>(v, (lane & 4) == 0);
    v = merge_steps<4>(v, (lane & 8) == 0);
    v = merge_steps<8>(v, (lane & 16) == 0);
    v = merge_steps<16>(v, (lane & 32) == 0);
    v = merge_steps<32>(v, true);
    return v;
}

// A score's order key: an unsigned integer with the same order as the fp32
// score (-0 folded onto +0, so equal scores give equal keys), and back.
__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k)
{
    return __uint_as_float(k ^ ((uint32_t)((int32_t)~k >> 31) | 0x80000000u));
}

// Wave-wide sum; every lane receives the same value (pairwise xor tree, so
// the association is identical in all lanes).
__device__ __forceinline__ float wave_sum(float x)
{
    x += __uint_as_float(xor_lane<1>(__float_as_uint(x)));
    x += __uint_as_float(xor_lane<2>(__float_as_uint(x)));
    x += __uint_as_float(xor_lane<4>(__float_as_uint(x)));
    x += __uint_as_float(xor_lane<8>(__float_as_uint(x)));
    x += __uint_as_float(xor_lane<16>(__float_as_uint(x)));
    x += __uint_as_float(xor_lane<32>(__float_as_uint(x)));
    return x;
}

}  // namespace pkm
