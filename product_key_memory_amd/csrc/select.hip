// Steps a4-a6 of the lookup in one kernel, one wave64 per (token, head):
//   a4  exact top-k of each half's n subkey scores,
//   a5  the k*k candidate grid s0[i] + s1[j] (flat row i0[i]*n + i1[j]) and
//       its exact top-k,
//   a6  softmax over the k winners.
// ("Product-Key Memory", §Factorising the key space and the code listing's
// forward; "Memory Retrieval Mechanisms: From Soft to Efficient", top-k
// section.)
//
// Ordering.  Each element becomes a 64-bit key: the high word maps the fp32
// score to an unsigned integer with the same order (-0 folded onto +0), the
// low word is ~index, so comparing keys compares (score desc, index asc),
// the tie rule of the whole lookup, and no two keys are equal.
//
// Selection (no sort of all n elements).  Lane l holds elements l, l+64, ...
// 1. T = k-th largest of the 64 lane maxima (bitonic sort of 64 words): at
//    least k elements are >= T, so every winner is >= T.
// 2. The elements >= T are counted with ballots.  For random scores about
//    1.35 k of them survive; if they fit in 64 they are compacted into LDS
//    (ballot + mbcnt) and one bitonic sort of 64 keys orders them.
// 3. Otherwise (heavy ties, unusual inputs) the exact k-th key is found by
//    MSB-first bisection with ballot counts, then the last index kept among
//    elements tied at it, so exactly k elements are compacted and sorted.
// Lane j then holds the j-th best key, j < k.
#include "pkm_internal.h"

namespace pkm {
namespace {

constexpr int WAVES = 4;  // (token, head) pairs per 256-thread workgroup

__device__ __forceinline__ uint32_t order_key(float f)
{
    f = f + 0.0f;  // -0 -> +0: equal scores must give equal keys
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ uint64_t pack(uint32_t key, uint32_t id)
{
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

__device__ __forceinline__ uint32_t unpack_id(uint64_t c) { return 0xFFFFFFFFu - (uint32_t)c; }

__device__ __forceinline__ uint32_t shfl_xor32(uint32_t v, int m) { return (uint32_t)__shfl_xor((int)v, m, 64); }

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m)
{
    const uint32_t lo = shfl_xor32((uint32_t)v, m), hi = shfl_xor32((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t xchg(uint32_t v, int m) { return shfl_xor32(v, m); }
__device__ __forceinline__ uint64_t xchg(uint64_t v, int m) { return shfl_xor64(v, m); }

// Bitonic sort of one value per lane over the wave, descending by lane.
template <typename T>
__device__ __forceinline__ T sort64_desc(T v, int lane)
{
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const T o = xchg(v, stride);
            const bool desc = (lane & size) == 0;  // direction of this block
            const bool lower = (lane & stride) == 0;
            v = (lower == desc) ? (v > o ? v : o) : (v < o ? v : o);
        }
    }
    return v;
}

// Orders this wave's LDS writes before its later LDS reads by other lanes (a
// wave's LDS operations complete in order; this keeps the compiler from
// moving accesses across the point).
__device__ __forceinline__ void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Exact top-k (k <= 64) of the wave's elements: element t of lane l has order
// key key[t] (0 = absent) and index id[t].  Returns, in lane j < k, the j-th
// best packed key.  buf: 64 slots of this wave's LDS.
template <int MAXM>
__device__ uint64_t wave_topk(const uint32_t (&key)[MAXM], const uint32_t (&id)[MAXM], int k, uint64_t *buf,
                              int lane)
{
    uint32_t lane_max = 0;
#pragma unroll
    for (int t = 0; t < MAXM; ++t) lane_max = key[t] > lane_max ? key[t] : lane_max;
    // Kept: key > kth, or key == kth and id <= last.
    uint32_t kth = (uint32_t)__shfl((int)sort64_desc(lane_max, lane), k - 1, 64);
    uint32_t last = 0xFFFFFFFFu;

    int count = 0;
#pragma unroll
    for (int t = 0; t < MAXM; ++t) count += __popcll(__ballot(key[t] >= kth));

    if (count > 64) {
        // Too many survivors for one sort (ties or unusual inputs): find the
        // exact k-th key by MSB-first bisection over the score key, then the
        // last index to keep among the elements tied at it.  count(key >= x)
        // is non-increasing in x, so the largest x with count >= k is the
        // k-th best score key.
        kth = 0;
#pragma unroll 1
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = kth | (1u << bit);
            int c = 0;
#pragma unroll
            for (int t = 0; t < MAXM; ++t) c += __popcll(__ballot(key[t] >= cand));
            if (c >= k) kth = cand;
        }
        int gt = 0;
#pragma unroll
        for (int t = 0; t < MAXM; ++t) gt += __popcll(__ballot(key[t] > kth));
        const int need = k - gt;  // lowest indices to take among the ties
        last = 0;
#pragma unroll 1
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = last | (1u << bit);
            int c = 0;
#pragma unroll
            for (int t = 0; t < MAXM; ++t) c += __popcll(__ballot(key[t] == kth && id[t] < cand));
            if (c < need) last = cand;
        }
        count = k;
    }

    int base = 0;
#pragma unroll
    for (int t = 0; t < MAXM; ++t) {
        const bool keep = key[t] > kth || (key[t] == kth && id[t] <= last);
        const uint64_t mask = __ballot(keep);
        if (keep) {
            const int below =
                __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
            if (base + below < 64) buf[base + below] = pack(key[t], id[t]);  // never more than count <= 64
        }
        base += __popcll(mask);
    }
    wave_sync_lds();
    const uint64_t v = lane < count ? buf[lane] : 0ull;
    wave_sync_lds();
    return sort64_desc(v, lane);
}

template <int MAXM>
__global__ __launch_bounds__(64 * WAVES) void select_kernel(const float *__restrict__ scores, int64_t pairs, int n,
                                                            int k, int32_t *__restrict__ idx_out,
                                                            float *__restrict__ w_out)
{
    __shared__ uint64_t buf[WAVES][64];
    __shared__ float half_score[WAVES][2][64];
    __shared__ uint32_t half_index[WAVES][2][64];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t pair = (int64_t)blockIdx.x * WAVES + wv;  // b * H + h
    if (pair >= pairs) return;
    float *hs = &half_score[wv][0][0];
    uint32_t *hi = &half_index[wv][0][0];

    // a4: each half's top-k, kept in LDS as (score, subkey index), best first.
    const int m = (n + 63) >> 6;
#pragma unroll 1
    for (int p = 0; p < 2; ++p) {
        const float *row = scores + (pair * 2 + p) * (int64_t)n;
        uint32_t key[MAXM], id[MAXM];
#pragma unroll
        for (int t = 0; t < MAXM; ++t) {
            const int e = t * 64 + lane;
            const bool ok = t < m && e < n;
            key[t] = ok ? order_key(row[e]) : 0u;
            id[t] = (uint32_t)e;
        }
        const uint64_t c = wave_topk<MAXM>(key, id, k, &buf[wv][0], lane);
        if (lane < k) {
            hs[p * 64 + lane] = key_score((uint32_t)(c >> 32));
            hi[p * 64 + lane] = unpack_id(c);
        }
    }
    wave_sync_lds();

    // a5: candidate (i, j) lives in lane (i % R) * k + j, slot i / R, with
    // R = floor(64 / k) grid rows per slot.
    const int R = 64 / k;
    const int q = lane / k;
    const int j = lane - q * k;
    const bool lane_ok = q < R;
    const float s1 = lane_ok ? hs[64 + j] : 0.0f;
    const uint32_t i1 = lane_ok ? hi[64 + j] : 0u;
    const int slots = (k + R - 1) / R;
    uint32_t key[MAXM], id[MAXM];
#pragma unroll
    for (int t = 0; t < MAXM; ++t) {
        const int i = t * R + q;
        const bool ok = lane_ok && t < slots && i < k;
        const float s0 = ok ? hs[i] : 0.0f;
        const uint32_t i0 = ok ? hi[i] : 0u;
        key[t] = ok ? order_key(s0 + s1) : 0u;
        id[t] = i0 * (uint32_t)n + i1;
    }
    const uint64_t c = wave_topk<MAXM>(key, id, k, &buf[wv][0], lane);

    // a6: softmax over the k winners; lane 0 holds the largest score.
    const float top = key_score((uint32_t)(c >> 32));
    const float mx = __shfl(top, 0, 64);
    const float e = lane < k ? expf(top - mx) : 0.0f;
    float sum = e;
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) sum += __shfl_xor(sum, s, 64);
    if (lane < k) {
        idx_out[pair * k + lane] = (int32_t)unpack_id(c);
        w_out[pair * k + lane] = e / sum;
    }
}

template <int MAXM>
hipError_t launch(const float *scores, int64_t pairs, int n, int k, int32_t *idx, float *w, hipStream_t stream)
{
    const int64_t blocks = (pairs + WAVES - 1) / WAVES;
    hipLaunchKernelGGL(select_kernel<MAXM>, dim3((unsigned)blocks), dim3(64 * WAVES), 0, stream, scores, pairs, n, k,
                       idx, w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const float *scores, int64_t B, int H, int n, int k, int32_t *idx, float *w,
                         hipStream_t stream)
{
    const int64_t pairs = B * H;
    if (pairs <= 0) return hipSuccess;
    const int R = 64 / k;
    const int m_half = (n + 63) / 64;
    const int m_cand = (k + R - 1) / R;
    const int m = m_half > m_cand ? m_half : m_cand;
    if (m <= 4) return launch<4>(scores, pairs, n, k, idx, w, stream);
    if (m <= 16) return launch<16>(scores, pairs, n, k, idx, w, stream);
    if (m <= 32) return launch<32>(scores, pairs, n, k, idx, w, stream);
    return launch<64>(scores, pairs, n, k, idx, w, stream);
}

}  // namespace pkm
