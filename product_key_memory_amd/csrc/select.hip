// Steps a4-a6 of the lookup in one kernel, one wave64 per (token, head):
//   a4  exact top-k of each half's n subkey scores,
//   a5  the exact top-k of the k*k candidates s0[i] + s1[j] (flat row
//       i0[i]*n + i1[j]),
//   a6  softmax over the k winners.
// ("Product-Key Memory", §Factorising the key space and the code listing's
// forward; "Memory Retrieval Mechanisms: From Soft to Efficient", top-k
// section.)
//
// Ordering.  An element's order key maps its fp32 score to an unsigned
// integer with the same order (-0 folded onto +0); packed with ~index below
// it, comparing 64-bit keys compares (score desc, index asc), the tie rule of
// the whole lookup, and no two packed keys are equal.
//
// Per-half top-k (no sort of all n elements).  Lane l holds elements l,
// l + 64, ... of the half in registers.  T = the k-th largest of the 64 lane
// maxima, its low bits cleared (a ballot bisection): at least k elements are
// >= T, so every winner is.  The elements >= T (about 1.35 k for random
// scores) are compacted into LDS with ballot + mbcnt and one 64-lane bitonic
// sort of packed keys orders them (65 to 128 survivors: two sorts and one
// bitonic merge).  If more than 128 survive (heavy exact ties), the exact
// k-th key is found by MSB-first bisection with ballot counts, then the last
// index kept among the ties, and exactly k are compacted.  The halves are
// selected one after the other; every row load is issued before the first
// is consumed.
//
// Candidates.  With both halves sorted, s0[i] + s1[j] can only be beaten by
// the cells above and left of it, so a cell with (i+1)(j+1) > k has at
// least k cells of the "staircase" {(i+1)(j+1) <= k} at or above it: the
// k-th best score v_k of the full grid is the k-th best of the staircase
// (119 of 1024 cells at k = 32), and every cell scoring above v_k lies in
// it.  The staircase's top-k is therefore the answer unless a cell outside
// it ties v_k; the best outside cell of column j is (floor(k/(j+1)), j), so
// one comparison per column certifies the result.  Otherwise (ties) the full
// k*k grid is ranked.  All scores stay fp32; the candidate sums are the same
// fp32 additions whichever path runs.
#include "gather_dev.h"
#include "pkm_internal.h"
#include "wave_ops.h"

namespace pkm {
namespace {

constexpr int WAVES = 4;        // (token, head) pairs per 256-thread workgroup
constexpr int STAIR_SLOTS = 5;  // staircase cells per lane: 280 cells at k = 64

__device__ __forceinline__ uint64_t pack(uint32_t key, uint32_t id)
{
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

__device__ __forceinline__ uint32_t unpack_id(uint64_t c) { return 0xFFFFFFFFu - (uint32_t)c; }

__device__ __forceinline__ uint32_t read_lane(uint32_t v, int src)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, src);
}

__device__ __forceinline__ int below_me(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Orders this wave's LDS writes before its later LDS reads by other lanes (a
// wave's LDS operations complete in order; this keeps the compiler from
// moving accesses across the point).
__device__ __forceinline__ void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Per-wave LDS: 128 compaction slots plus one discard slot per lane, so the
// compaction stores unconditionally and never branches.
constexpr int kSlots = 128;
struct Stage {
    uint64_t slot[kSlots + 64];
};

// Appends the packed key of an element to the compaction when `keep`.
__device__ __forceinline__ void append(bool keep, uint32_t key, uint32_t id, int &base, Stage &st, int lane)
{
    const uint64_t mask = __ballot(keep);
    const int pos = base + below_me(mask);
    st.slot[keep && pos < kSlots ? pos : kSlots + lane] = pack(key, id);
    base += __popcll(mask);
}

__device__ __forceinline__ bool kept(uint32_t key, uint32_t id, uint32_t kth, uint32_t last)
{
    return key > kth || (key == kth && id <= last);
}

// Exact k-th largest key and, among elements tied at it, the largest index
// to keep so that exactly k elements are kept.  count(key >= x) does not
// increase with x, so the MSB-first greedy finds the largest x with at least
// k elements >= x: the k-th largest key.  Rolled loops over the m slots with
// keys recomputed by key_of: only inputs with more than 128 keys at or above
// the first threshold (heavy exact ties) come here, and it must not hold
// registers.
template <typename KeyOf, typename IdOf>
__device__ void exact_cut(KeyOf key_of, IdOf id_of, int m, int k, uint32_t &kth, uint32_t &last)
{
    kth = 0;
#pragma unroll 1
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = kth | (1u << bit);
        int c = 0;
#pragma unroll 1
        for (int t = 0; t < m; ++t) c += __popcll(__ballot(key_of(t) >= cand));
        if (c >= k) kth = cand;
    }
    int gt = 0;
#pragma unroll 1
    for (int t = 0; t < m; ++t) gt += __popcll(__ballot(key_of(t) > kth));
    const int need = k - gt;  // lowest indices to take among the ties
    last = 0;
#pragma unroll 1
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = last | (1u << bit);
        int c = 0;
#pragma unroll 1
        for (int t = 0; t < m; ++t) c += __popcll(__ballot(key_of(t) == kth && id_of(t) < cand));
        if (c < need) last = cand;
    }
}

// Rolled compaction with recomputed keys.
template <typename KeyOf, typename IdOf>
__device__ int compact_rolled(KeyOf key_of, IdOf id_of, int m, uint32_t kth, uint32_t last, Stage &st, int lane)
{
    int base = 0;
#pragma unroll 1
    for (int t = 0; t < m; ++t) {
        const uint32_t key = key_of(t), id = id_of(t);
        append(kept(key, id, kth, last), key, id, base, st, lane);
    }
    return base;
}

__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Sorts the count (<= 128) compacted keys; lane j receives the j-th best.
// Up to 64: one 64-lane bitonic sort.  Up to 128: both halves sorted, the
// second reversed and merged elementwise (a bitonic sequence holding the
// best 64 of both), then one bitonic clean.
__device__ __forceinline__ uint64_t sorted_survivors(int count, Stage &st, int lane)
{
    wave_sync_lds();
    uint64_t v = lane < count ? st.slot[lane] : 0ull;
    uint64_t u = count > 64 && lane + 64 < count ? st.slot[lane + 64] : 0ull;
    wave_sync_lds();
    v = sort64_desc(v);
    if (count > 64) {
        u = sort64_desc(u);
        const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)u, 63 - lane, 64);
        const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(u >> 32), 63 - lane, 64);
        v = merge_steps<32>(max64(v, ((uint64_t)hi << 32) | lo), true);
    }
    return v;
}

// Clustered scores (e.g. a few lanes holding most of the best) can leave
// more than kSlots elements at or above a first threshold kth.  The slots
// then hold kSlots of them, so the k-th best key among the slots is a
// higher threshold that still keeps at least k elements; it is raised that
// way while it rises and the survivors overflow.  Returns the new count
// (still above kSlots only for heavy exact ties, left to exact_cut).
template <int M, typename IdOf>
__device__ __forceinline__ int raise_threshold(const uint32_t (&key)[M], IdOf id_of, int k, uint32_t &kth, int count,
                                               Stage &st, int lane)
{
#pragma unroll 1
    for (int it = 0; it < 3 && count > kSlots; ++it) {
        const uint64_t s = sorted_survivors(kSlots, st, lane);
        const uint32_t t2 = read_lane((uint32_t)(s >> 32), k - 1);
        if (t2 <= kth) break;
        kth = t2;
        count = 0;
#pragma unroll
        for (int t = 0; t < M; ++t) append(key[t] >= kth, key[t], id_of(t), count, st, lane);
    }
    return count;
}

// A first threshold from the lanes' largest keys v: the largest T whose low
// 12 bits are clear such that at least k lanes hold v >= T, by MSB-first
// bisection with ballot counts (one compare per step instead of sorting the
// 64 maxima).  T is at most the k-th largest v, so at least k elements are
// >= T, and within 2^-11 of it relative to the score, so hardly more survive.
constexpr int kBisectLowBits = 12;
__device__ __forceinline__ uint32_t kth_lane_bound(uint32_t v, int k)
{
    uint32_t t = 0;
#pragma unroll
    for (int bit = 31; bit >= kBisectLowBits; --bit) {
        const uint32_t cand = t | (1u << bit);
        if (__popcll(__ballot(v >= cand)) >= k) t = cand;
    }
    return t;
}

// Exact top-k (k <= 64) of the wave's elements, keys in registers key[M]
// (0 = absent) and recomputed by slow_key for the rare heavy-tie path: lane
// j < k receives the j-th best packed key.  RAISE: try raise_threshold
// before that path (the flat search's rows, whose scores cluster; the
// lookup's subkey scores keep the smaller register footprint).
template <int M, bool RAISE = false, typename SlowKey, typename IdOf>
__device__ uint64_t wave_topk(const uint32_t (&key)[M], SlowKey slow_key, IdOf id_of, int m, int k, Stage &st,
                              int lane)
{
    uint32_t lane_max = 0;
#pragma unroll
    for (int t = 0; t < M; ++t) lane_max = key[t] > lane_max ? key[t] : lane_max;
    uint32_t kth = kth_lane_bound(lane_max, k);
    uint32_t last = 0xFFFFFFFFu;
    int count = 0;
#pragma unroll
    for (int t = 0; t < M; ++t) append(kept(key[t], id_of(t), kth, last), key[t], id_of(t), count, st, lane);
    if constexpr (RAISE) count = raise_threshold(key, id_of, k, kth, count, st, lane);
    if (count > kSlots) {
        exact_cut(slow_key, id_of, m, k, kth, last);
        count = compact_rolled(slow_key, id_of, m, kth, last, st, lane);
    }
    return sorted_survivors(count, st, lane);
}

// Exact top-k with every key recomputed by key_of in rolled loops (the rare
// full-grid path).
template <typename KeyOf, typename IdOf>
__device__ uint64_t wave_topk_rolled(KeyOf key_of, IdOf id_of, int m, int k, Stage &st, int lane)
{
    uint32_t lane_max = 0;
#pragma unroll 1
    for (int t = 0; t < m; ++t) {
        const uint32_t key = key_of(t);
        lane_max = key > lane_max ? key : lane_max;
    }
    uint32_t kth = kth_lane_bound(lane_max, k);
    uint32_t last = 0xFFFFFFFFu;
    int count = compact_rolled(key_of, id_of, m, kth, last, st, lane);
    if (count > kSlots) {
        exact_cut(key_of, id_of, m, k, kth, last);
        count = compact_rolled(key_of, id_of, m, kth, last, st, lane);
    }
    return sorted_survivors(count, st, lane);
}

// Element held in slot t of a lane.  With VEC4 (rows of a multiple of 256
// scores) slot t holds element (t/4)*256 + 4*lane + t%4, so each lane reads
// float4s; otherwise element t*64 + lane.
template <bool VEC4>
__device__ __forceinline__ int slot_element(int t, int lane)
{
    return VEC4 ? ((t >> 2) << 8) + (lane << 2) + (t & 3) : t * 64 + lane;
}

typedef float fx4v __attribute__((ext_vector_type(4)));

// Loads the order keys of one half row (0 past the end of the row).  The
// loads are unconditional (clamped index), so all of them are in flight
// together instead of one exec-masked load at a time.  NTS: non-temporal
// loads (VEC4 rows), for a kernel whose later row reads rely on the caches.
template <int MH, bool VEC4, bool NTS = false>
__device__ __forceinline__ void load_keys(const float *row, int n, int lane, uint32_t (&key)[MH])
{
    float v[MH];
    if constexpr (VEC4) {
        static_assert(MH % 4 == 0, "whole float4s");
#pragma unroll
        for (int q = 0; q < MH / 4; ++q) {
            const fx4v *src = reinterpret_cast<const fx4v *>(row + min(q * 256 + lane * 4, n - 4));
            const fx4v f = NTS ? __builtin_nontemporal_load(src) : *src;
            v[4 * q] = f[0];
            v[4 * q + 1] = f[1];
            v[4 * q + 2] = f[2];
            v[4 * q + 3] = f[3];
        }
    } else {
#pragma unroll
        for (int t = 0; t < MH; ++t) v[t] = row[min(t * 64 + lane, n - 1)];
    }
#pragma unroll
    for (int t = 0; t < MH; ++t) key[t] = slot_element<VEC4>(t, lane) < n ? order_key(v[t]) : 0u;
}

// Top-k of one half from keys already in registers; writes the sorted result
// to (hs[p][j], hi[p][j]), j < k.
template <int MH, bool VEC4>
__device__ __forceinline__ void half_select(const uint32_t (&key)[MH], const float *row, int p, int n, int k,
                                            Stage &st, float (*hs)[64], uint32_t (*hi)[64], int lane)
{
    const auto id_of = [lane](int t) { return (uint32_t)slot_element<VEC4>(t, lane); };
    const auto reread = [=](int t) {
        const int e = slot_element<VEC4>(t, lane);
        return e < n ? order_key(row[e]) : 0u;
    };
    const uint64_t v = wave_topk(key, reread, id_of, VEC4 ? MH : (n + 63) >> 6, k, st, lane);
    if (lane < k) {
        hs[p][lane] = key_score((uint32_t)(v >> 32));
        hi[p][lane] = unpack_id(v);
    }
}

// a4 for both halves of one (token, head), one after the other.  Short rows
// (MH <= 16 slots) load both halves before selecting, so the second row's
// loads overlap the first selection; longer rows load each half in turn to
// bound the live registers.
template <int MH, bool VEC4, bool NTS = false>
__device__ void half_topk(const float *row0, int n, int k, Stage &st, float (*hs)[64], uint32_t (*hi)[64], int lane)
{
    const float *row1 = row0 + n;
    if constexpr (MH <= 16) {
        uint32_t key0[MH], key1[MH];
        load_keys<MH, VEC4, NTS>(row0, n, lane, key0);
        load_keys<MH, VEC4, NTS>(row1, n, lane, key1);
        half_select<MH, VEC4>(key0, row0, 0, n, k, st, hs, hi, lane);
        half_select<MH, VEC4>(key1, row1, 1, n, k, st, hs, hi, lane);
    } else {
#pragma unroll 1
        for (int p = 0; p < 2; ++p) {
            uint32_t key[MH];
            const float *row = p ? row1 : row0;
            load_keys<MH, VEC4, NTS>(row, n, lane, key);
            half_select<MH, VEC4>(key, row, p, n, k, st, hs, hi, lane);
        }
    }
}

// a5 over the whole k*k grid (when the staircase cannot be certified): cell
// (i, j) lives in lane (i % R) * k + j, slot i / R, R = floor(64 / k); keys
// are recomputed from the LDS half lists.
__device__ uint64_t full_grid_topk(int n, int k, float (*hs)[64], uint32_t (*hi)[64], Stage &st, int lane)
{
    const int R = 64 / k;
    const int q = lane / k;
    const int j = lane - q * k;
    const bool lane_ok = q < R;
    const int jj = lane_ok ? j : 0;
    const int slots = (k + R - 1) / R;
    const auto key_of = [=](int t) {
        const int i = t * R + q;
        const bool ok = lane_ok && i < k;
        return ok ? order_key(hs[0][ok ? i : 0] + hs[1][jj]) : 0u;
    };
    const auto id_of = [=](int t) {
        const int i = min(t * R + q, k - 1);
        return hi[0][i] * (uint32_t)n + hi[1][jj];
    };
    return wave_topk_rolled(key_of, id_of, slots, k, st, lane);
}

// The staircase cells of every k <= 64, fixed at compile time: row k - 1
// holds the cells (i, j) with (i+1)(j+1) <= k, packed (i << 16) | j in
// row-major order, then 0xFFFFFFFF up to kMaxStaircaseCells.
struct StairTables {
    uint32_t cell[64][kMaxStaircaseCells];
};

constexpr StairTables make_stair_tables()
{
    StairTables t{};
    for (int k = 1; k <= 64; ++k) {
        for (int c = 0; c < kMaxStaircaseCells; ++c) t.cell[k - 1][c] = 0xFFFFFFFFu;
        int c = 0;
        for (int i = 0; i < k; ++i)
            for (int j = 0; (i + 1) * (j + 1) <= k; ++j) t.cell[k - 1][c++] = ((uint32_t)i << 16) | (uint32_t)j;
    }
    return t;
}

__device__ const StairTables kStairTables = make_stair_tables();

// a4-a6 for one (token, head) whose half scores start at row0 (half 1 at
// row0 + n): lane j < k receives the j-th winner's flat row and softmax
// weight (winners by score desc, flat row asc).  hs / hi: the wave's LDS
// lists of the two halves' top-k.
template <int MH, bool VEC4, bool NTS = false>
__device__ __forceinline__ void select_pair(const float *row0, int n, int k, Stage &st, float (*hs)[64],
                                            uint32_t (*hi)[64], int lane, int32_t &id_out, float &w_out)
{
    // a4
    half_topk<MH, VEC4, NTS>(row0, n, k, st, hs, hi, lane);
    wave_sync_lds();

    // a5 on the staircase: stair[c] = (i << 16) | j for the staircase's
    // cells, 0xFFFFFFFF up to STAIR_SLOTS * 64 (loaded unconditionally)
    const uint32_t *stair = kStairTables.cell[k - 1];
    const auto cell_of = [=](int t) { return stair[t * 64 + lane]; };
    uint32_t cell[STAIR_SLOTS], key[STAIR_SLOTS], id[STAIR_SLOTS];
#pragma unroll
    for (int t = 0; t < STAIR_SLOTS; ++t) cell[t] = cell_of(t);
#pragma unroll
    for (int t = 0; t < STAIR_SLOTS; ++t) {
        const bool ok = cell[t] != 0xFFFFFFFFu;
        const uint32_t i = ok ? cell[t] >> 16 : 0u, j = ok ? cell[t] & 0xFFFFu : 0u;
        key[t] = ok ? order_key(hs[0][i] + hs[1][j]) : 0u;
        id[t] = hi[0][i] * (uint32_t)n + hi[1][j];
    }
    const auto stair_key = [=](int t) {
        const uint32_t ij = cell_of(t);
        return ij != 0xFFFFFFFFu ? order_key(hs[0][ij >> 16] + hs[1][ij & 0xFFFFu]) : 0u;
    };
    uint64_t c = wave_topk(key, stair_key, [&](int t) { return id[t]; }, STAIR_SLOTS, k, st, lane);

    // certificate: no cell outside the staircase reaches the k-th score
    const uint32_t vk = read_lane((uint32_t)(c >> 32), k - 1);
    bool reach = false;
    if (lane < k) {
        const int i_out = k / (lane + 1);  // first row of column `lane` outside the staircase
        if (i_out < k) reach = order_key(hs[0][i_out] + hs[1][lane]) >= vk;
    }
    if (__ballot(reach) != 0ull) c = full_grid_topk(n, k, hs, hi, st, lane);

    // a6: softmax over the k winners; lane 0 holds the largest score.
    const float top = key_score((uint32_t)(c >> 32));
    const float mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(top), 0));
    const float e = lane < k ? expf(top - mx) : 0.0f;
    const float sum = wave_sum(e);
    id_out = (int32_t)unpack_id(c);
    w_out = e / sum;
}

template <int MH, bool VEC4>
__global__ __launch_bounds__(64 * WAVES) void select_kernel(const float *__restrict__ scores, int64_t pairs, int n,
                                                            int k, int32_t *__restrict__ idx_out,
                                                            float *__restrict__ w_out)
{
    __shared__ Stage stage[WAVES];
    __shared__ float half_score[WAVES][2][64];
    __shared__ uint32_t half_index[WAVES][2][64];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t pair = (int64_t)blockIdx.x * WAVES + wv;  // b * H + h
    if (pair >= pairs) return;
    int32_t id;
    float wt;
    select_pair<MH, VEC4>(scores + pair * 2 * (int64_t)n, n, k, stage[wv], half_score[wv], half_index[wv], lane, id,
                          wt);
    if (lane < k) {
        idx_out[pair * k + lane] = id;
        w_out[pair * k + lane] = wt;
    }
}

// a4-a7 fused: one workgroup per token.  Its waves first select the
// token's heads (wave w takes heads w, w + kFusedWaves, ...), keeping the H k
// (row, weight) pairs in LDS (and writing them out when idx_out is given),
// then gather the token's output from those pairs with exactly the share
// and order of the stand-alone gather (a 1 KiB column slice per wave, or
// whole rows in wave 0 when they are two slices long; every row in order),
// so the result is bitwise the same as select followed by gather.  The selection is ALU-bound and the gather HBM-bound; with
// several tokens' workgroups on a CU, one token's selection runs while
// another token's row loads are in flight.  Rows of at most 512 bytes are
// not fused: their gather takes two waves per token, and the fused kernel's
// occupancy would leave half the stand-alone kernel's loads in flight.
constexpr int kFusedMaxRows = 512;  // H * k held in LDS
constexpr int kFusedWaves = 4;      // waves per token

template <int MH, int VT, bool NT>
__global__ __launch_bounds__(64 * kFusedWaves) void select_gather_kernel(const float *__restrict__ scores, int H, int n,
                                                                   int k, const uint8_t *__restrict__ values,
                                                                   const float *__restrict__ scale, int D, int N,
                                                                   int32_t *__restrict__ idx_out,
                                                                   float *__restrict__ w_out, float *__restrict__ out)
{
    constexpr int EPL = gdev::Fmt<VT>::EPL;
    __shared__ Stage stage[kFusedWaves];
    __shared__ float half_score[kFusedWaves][2][64];
    __shared__ uint32_t half_index[kFusedWaves][2][64];
    __shared__ int32_t sel_row[kFusedMaxRows];
    __shared__ float sel_w[kFusedMaxRows];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t b = blockIdx.x;
    for (int h = wv; h < H; h += kFusedWaves) {
        const int64_t pair = b * H + h;
        int32_t id;
        float wt;
        // scores read non-temporally when the gather's row reads go through
        // the caches (rows repeat), so the scores do not displace them
        select_pair<MH, true, !NT>(scores + pair * 2 * (int64_t)n, n, k, stage[wv], half_score[wv], half_index[wv],
                                   lane, id, wt);
        if (lane < k) {
            sel_row[h * k + lane] = id;
            sel_w[h * k + lane] = wt;
            if (idx_out) {
                idx_out[pair * k + lane] = id;
                w_out[pair * k + lane] = wt;
            }
        }
    }
    __syncthreads();
    const int slices = (D + 64 * EPL - 1) / (64 * EPL);
    if (slices == 2) {  // as the stand-alone gather: one wave reads the rows whole
        if (wv == 0) gdev::gather_two_slices<VT, NT>(values, scale, D, N, H * k, sel_row, sel_w, out + b * D, lane);
        return;
    }
    for (int sl = wv; sl < slices; sl += kFusedWaves)
        gdev::gather_slice<VT, NT>(values, scale, D, N, H * k, sl, sel_row, sel_w, out + b * D, lane);
}

// Flat exact search: top-k over rows of up to n^2 scores, in passes.  Pass 1
// reads scores: one wave per (row, segment of 4096), the segment's k best
// as packed keys (0 where a short segment has fewer than k elements).
// Later passes read those packed keys, 2048 per wave.  Packed keys are
// unique, so the k best of a row are among the k best of its segments; the
// pass with one segment per row writes the flat indices and scores.
constexpr int kFlatScoreSeg = 4096;
constexpr int kFlatKeySeg = 2048;

template <bool FROM_SCORES, bool VEC4>
__global__ __launch_bounds__(64 * WAVES) void flat_topk_kernel(const void *__restrict__ in, int64_t rows, int64_t len,
                                                               int segs, int k, uint64_t *__restrict__ out_keys,
                                                               int32_t *__restrict__ idx_out,
                                                               float *__restrict__ top_out)
{
    constexpr int SEG = FROM_SCORES ? kFlatScoreSeg : kFlatKeySeg;
    constexpr int MH = SEG / 64;
    __shared__ Stage stage[WAVES];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t item = (int64_t)blockIdx.x * WAVES + wv;  // row * segs + segment
    if (item >= rows * segs) return;
    const int64_t row = item / segs;
    const int seg = (int)(item - row * segs);
    const int64_t base = (int64_t)seg * SEG;
    const int m = (int)min((int64_t)SEG, len - base);  // elements in this segment, >= 1

    uint64_t c;
    if constexpr (FROM_SCORES) {
        const float *seg_row = static_cast<const float *>(in) + row * len + base;
        uint32_t key[MH];
        load_keys<MH, VEC4>(seg_row, m, lane, key);
        const auto id_of = [=](int t) { return (uint32_t)(base + slot_element<VEC4>(t, lane)); };
        const auto reread = [=](int t) {
            const int e = slot_element<VEC4>(t, lane);
            return e < m ? order_key(seg_row[e]) : 0u;
        };
        c = wave_topk<MH, true>(key, reread, id_of, VEC4 ? MH : (m + 63) >> 6, k, stage[wv], lane);
    } else {
        const uint64_t *seg_row = static_cast<const uint64_t *>(in) + row * len + base;
        uint64_t v[MH];
#pragma unroll
        for (int t = 0; t < MH; ++t) v[t] = seg_row[min(t * 64 + lane, m - 1)];
        uint32_t key[MH], id[MH];
#pragma unroll
        for (int t = 0; t < MH; ++t) {
            const bool ok = t * 64 + lane < m;
            key[t] = ok ? (uint32_t)(v[t] >> 32) : 0u;
            id[t] = ok ? unpack_id(v[t]) : 0xFFFFFFFFu;
        }
        const auto reread = [=](int t) {
            const int e = t * 64 + lane;
            return e < m ? (uint32_t)(seg_row[e] >> 32) : 0u;
        };
        const auto id_again = [=](int t) {
            const int e = t * 64 + lane;
            return e < m ? unpack_id(seg_row[e]) : 0xFFFFFFFFu;
        };
        // registers for the common path, re-reads for the heavy-tie path
        uint32_t lane_max = 0;
#pragma unroll
        for (int t = 0; t < MH; ++t) lane_max = key[t] > lane_max ? key[t] : lane_max;
        uint32_t kth = kth_lane_bound(lane_max, k);
        uint32_t last = 0xFFFFFFFFu;
        int count = 0;
#pragma unroll
        for (int t = 0; t < MH; ++t) append(kept(key[t], id[t], kth, last), key[t], id[t], count, stage[wv], lane);
        count = raise_threshold(key, [&](int t) { return id[t]; }, k, kth, count, stage[wv], lane);
        if (count > kSlots) {
            exact_cut(reread, id_again, (m + 63) >> 6, k, kth, last);
            count = compact_rolled(reread, id_again, (m + 63) >> 6, kth, last, stage[wv], lane);
        }
        c = sorted_survivors(count, stage[wv], lane);
    }
    if (lane < k) {
        if (out_keys) {
            out_keys[item * k + lane] = (c >> 32) != 0u ? c : 0ull;
        } else {
            idx_out[row * k + lane] = (int32_t)unpack_id(c);
            top_out[row * k + lane] = key_score((uint32_t)(c >> 32));
        }
    }
}

template <bool FROM_SCORES, bool VEC4>
hipError_t launch_flat_pass(const void *in, int64_t rows, int64_t len, int k, uint64_t *out_keys, int32_t *idx,
                            float *top, hipStream_t stream)
{
    const int seg = FROM_SCORES ? kFlatScoreSeg : kFlatKeySeg;
    const int64_t segs = (len + seg - 1) / seg;
    const int64_t blocks = (rows * segs + WAVES - 1) / WAVES;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((flat_topk_kernel<FROM_SCORES, VEC4>), dim3((unsigned)blocks), dim3(64 * WAVES), 0, stream, in,
                       rows, len, (int)segs, k, out_keys, idx, top);
    return hipGetLastError();
}

// Flat top-k with a threshold (rows longer than one 4096-score segment).
// theta = the k-th largest of a row's group maxima (groups of 64 scores): k
// distinct groups hold an element >= theta, so the row's k-th best score is
// >= theta and every winner scores >= theta.  For untied scores only a few
// more than k elements do.  A group whose maximum is below theta holds no
// such element, so only the groups whose maximum reaches theta (about k of
// the row's n^2 / 64) are read: a wave scans kGroupSeg group maxima of its
// row and, for each group that qualifies, reads its 64 scores and appends
// those >= theta to the row's list at positions from an atomic add (the
// list's order varies between runs; its top-k, over unique packed keys,
// does not).  The maxima are the scores' own values (order-key maxima), so
// the test is exact.
constexpr int kGroupSeg = 1024;

__global__ __launch_bounds__(64 * WAVES) void flat_filter_kernel(const float *__restrict__ scores,
                                                                 const float *__restrict__ gmax, int64_t rows,
                                                                 int64_t len, int64_t groups, int segs, int k,
                                                                 const float *__restrict__ ttop,
                                                                 uint32_t *__restrict__ count,
                                                                 uint64_t *__restrict__ list)
{
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);  // row * segs + segment
    if (item >= rows * segs) return;
    const int64_t row = item / segs;
    const int seg = (int)(item - row * segs);
    const uint32_t tkey = order_key(ttop[row * k + k - 1]);
    const float *grow = gmax + row * groups;
    const float *srow = scores + row * len;
    uint64_t *lst = list + row * kFlatListCap;
    const int64_t g0 = (int64_t)seg * kGroupSeg;
    float gm[kGroupSeg / 64];
#pragma unroll
    for (int t = 0; t < kGroupSeg / 64; ++t) {
        const int64_t g = g0 + t * 64 + lane;
        gm[t] = g < groups ? grow[g] : 0.0f;
    }
#pragma unroll
    for (int t = 0; t < kGroupSeg / 64; ++t) {
        uint64_t hits = __ballot(g0 + t * 64 + lane < groups && order_key(gm[t]) >= tkey);
        while (hits) {
            const int l = __builtin_ctzll(hits);
            hits &= hits - 1;
            const int64_t base = (g0 + t * 64 + l) * 64;
            const int m = (int)min((int64_t)64, len - base);
            const float v = lane < m ? srow[base + lane] : 0.0f;
            const uint32_t key = order_key(v);
            const bool keep = lane < m && key >= tkey;
            const uint64_t mask = __ballot(keep);
            if (mask == 0) continue;
            uint32_t pos = 0;
            if (lane == 0) pos = atomicAdd(count + row, (uint32_t)__popcll(mask));
            const uint32_t p = read_lane(pos, 0) + (uint32_t)below_me(mask);
            if (keep && p < (uint32_t)kFlatListCap) lst[p] = pack(key, (uint32_t)(base + lane));
        }
    }
}

// A row whose list overflowed (more than kFlatListCap scores >= theta: heavy
// exact ties) is ranked in full by one wave.
template <bool VEC4>
__global__ __launch_bounds__(64 * WAVES) void flat_rescan_kernel(const float *__restrict__ scores, int64_t rows,
                                                                 int64_t len, int k, const uint32_t *__restrict__ count,
                                                                 int32_t *__restrict__ idx_out,
                                                                 float *__restrict__ top_out)
{
    constexpr int MH = kFlatScoreSeg / 64;
    __shared__ Stage stage[WAVES];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * WAVES + wv;
    if (row >= rows || count[row] <= (uint32_t)kFlatListCap) return;
    const float *srow = scores + row * len;
    uint64_t best = 0;
#pragma unroll 1
    for (int64_t base = 0; base < len; base += kFlatScoreSeg) {
        const int m = (int)min((int64_t)kFlatScoreSeg, len - base);
        const float *brow = srow + base;
        uint32_t key[MH];
        load_keys<MH, VEC4>(brow, m, lane, key);
        const auto id_of = [=](int t) { return (uint32_t)(base + slot_element<VEC4>(t, lane)); };
        const auto reread = [=](int t) {
            const int e = slot_element<VEC4>(t, lane);
            return e < m ? order_key(brow[e]) : 0u;
        };
        const uint64_t c = wave_topk<MH, true>(key, reread, id_of, VEC4 ? MH : (m + 63) >> 6, k, stage[wv], lane);
        if (lane < k) {
            stage[wv].slot[lane] = best;
            stage[wv].slot[k + lane] = c;
        }
        best = sorted_survivors(2 * k, stage[wv], lane);
    }
    if (lane < k) {
        idx_out[row * k + lane] = (int32_t)unpack_id(best);
        top_out[row * k + lane] = key_score((uint32_t)(best >> 32));
    }
}

template <int MH>
hipError_t launch(const float *scores, int64_t pairs, int n, int k, int32_t *idx, float *w, hipStream_t stream)
{
    const int64_t blocks = (pairs + WAVES - 1) / WAVES;
    const dim3 grid((unsigned)blocks), block(64 * WAVES);
    if (n % 256 == 0 && n == MH * 64)
        hipLaunchKernelGGL((select_kernel<MH, true>), grid, block, 0, stream, scores, pairs, n, k, idx, w);
    else
        hipLaunchKernelGGL((select_kernel<MH, false>), grid, block, 0, stream, scores, pairs, n, k, idx, w);
    return hipGetLastError();
}

}  // namespace

int64_t flat_topk_keys_per_row(int64_t len, int k)
{
    return (len + kFlatScoreSeg - 1) / kFlatScoreSeg * k;
}

hipError_t launch_flat_topk(const float *scores, int64_t rows, int64_t len, int k, uint64_t *buf0, uint64_t *buf1,
                            int32_t *idx, float *top, hipStream_t stream)
{
    if (rows <= 0) return hipSuccess;
    if (k < 1 || k > 64 || len < k) return hipErrorInvalidValue;
    const bool vec4 = len % 4 == 0;
    if (len <= kFlatScoreSeg)
        return vec4 ? launch_flat_pass<true, true>(scores, rows, len, k, nullptr, idx, top, stream)
                    : launch_flat_pass<true, false>(scores, rows, len, k, nullptr, idx, top, stream);
    hipError_t e = vec4 ? launch_flat_pass<true, true>(scores, rows, len, k, buf0, nullptr, nullptr, stream)
                        : launch_flat_pass<true, false>(scores, rows, len, k, buf0, nullptr, nullptr, stream);
    int64_t klen = flat_topk_keys_per_row(len, k);
    uint64_t *src = buf0, *dst = buf1;
    while (e == hipSuccess) {
        if (klen <= kFlatKeySeg) return launch_flat_pass<false, false>(src, rows, klen, k, nullptr, idx, top, stream);
        e = launch_flat_pass<false, false>(src, rows, klen, k, dst, nullptr, nullptr, stream);
        klen = (klen + kFlatKeySeg - 1) / kFlatKeySeg * k;
        uint64_t *t = src;
        src = dst;
        dst = t;
    }
    return e;
}

hipError_t launch_flat_topk_threshold(const float *scores, const float *gmax, int64_t rows, int64_t len, int k,
                                      uint64_t *buf0, uint64_t *buf1, int32_t *tidx, float *ttop, uint32_t *count,
                                      uint64_t *list, int32_t *idx, float *top, hipStream_t stream)
{
    if (rows <= 0) return hipSuccess;
    if (k < 1 || k > 64 || len <= kFlatScoreSeg) return hipErrorInvalidValue;
    const int64_t groups = (len + 63) / 64;  // >= 65 > k
    hipError_t e = launch_flat_topk(gmax, rows, groups, k, buf0, buf1, tidx, ttop, stream);
    if (e != hipSuccess) return e;
    if ((e = launch_fill(count, rows, 0u, stream)) != hipSuccess) return e;
    if ((e = launch_fill(reinterpret_cast<uint32_t *>(list), rows * kFlatListCap * 2, 0u, stream)) != hipSuccess)
        return e;
    const bool vec4 = len % 4 == 0;
    const int64_t segs = (groups + kGroupSeg - 1) / kGroupSeg;
    const int64_t blocks = (rows * segs + WAVES - 1) / WAVES;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(flat_filter_kernel, dim3((unsigned)blocks), dim3(64 * WAVES), 0, stream, scores, gmax, rows,
                       len, groups, (int)segs, k, ttop, count, list);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the lists' top-k (unused slots hold 0, the absent key), then the rows
    // whose list overflowed
    if ((e = launch_flat_pass<false, false>(list, rows, kFlatListCap, k, nullptr, idx, top, stream)) != hipSuccess)
        return e;
    const unsigned rblocks = (unsigned)((rows + WAVES - 1) / WAVES);
    if (vec4)
        hipLaunchKernelGGL((flat_rescan_kernel<true>), dim3(rblocks), dim3(64 * WAVES), 0, stream, scores, rows, len,
                           k, count, idx, top);
    else
        hipLaunchKernelGGL((flat_rescan_kernel<false>), dim3(rblocks), dim3(64 * WAVES), 0, stream, scores, rows, len,
                           k, count, idx, top);
    return hipGetLastError();
}

int staircase_cells(int k)
{
    int c = 0;
    for (int j = 0; j < k; ++j) c += k / (j + 1);
    return c;
}

namespace {

template <int MH, int VT>
hipError_t launch_fused(const float *scores, int64_t B, int H, int n, int k, const void *values, const float *scale,
                        int D, int N, int32_t *idx, float *w, float *out, hipStream_t stream)
{
    const bool nt = B * H * k < N;  // as the stand-alone gather: rows seldom repeat
    const uint8_t *v = static_cast<const uint8_t *>(values);
    const dim3 grid((unsigned)B), block(64 * kFusedWaves);
    if (nt)
        hipLaunchKernelGGL((select_gather_kernel<MH, VT, true>), grid, block, 0, stream, scores, H, n, k, v, scale, D,
                           N, idx, w, out);
    else
        hipLaunchKernelGGL((select_gather_kernel<MH, VT, false>), grid, block, 0, stream, scores, H, n, k, v, scale, D,
                           N, idx, w, out);
    return hipGetLastError();
}

template <int MH>
hipError_t launch_fused_vt(const float *scores, int64_t B, int H, int n, int k, const void *values,
                           const float *scale, int value_type, int D, int N, int32_t *idx, float *w, float *out,
                           hipStream_t stream)
{
    switch (value_type) {
    case 0: return launch_fused<MH, 0>(scores, B, H, n, k, values, scale, D, N, idx, w, out, stream);
    case 1: return launch_fused<MH, 1>(scores, B, H, n, k, values, scale, D, N, idx, w, out, stream);
    case 2: return launch_fused<MH, 2>(scores, B, H, n, k, values, scale, D, N, idx, w, out, stream);
    case 3: return launch_fused<MH, 3>(scores, B, H, n, k, values, scale, D, N, idx, w, out, stream);
    default: return launch_fused<MH, 4>(scores, B, H, n, k, values, scale, D, N, idx, w, out, stream);
    }
}

}  // namespace

bool select_gather_fusable(int H, int n, int k, int value_type, int D)
{
    const int64_t row_bytes = value_type == 0 ? 4 * (int64_t)D : value_type == 1 ? 2 * (int64_t)D
                            : value_type == 4 ? D / 2 : D;
    return (n == 1024 || n == 2048) && H * k <= kFusedMaxRows && row_bytes > 512;
}

hipError_t launch_select_gather(const float *scores, int64_t B, int H, int n, int k, const void *values,
                                const float *scale, int value_type, int D, int N, int32_t *idx, float *w, float *out,
                                hipStream_t stream)
{
    if (B <= 0) return hipSuccess;
    if (k < 1 || k > 64 || k > n || !select_gather_fusable(H, n, k, value_type, D) || (idx == nullptr) != (w == nullptr) ||
        B > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    if (n == 1024) return launch_fused_vt<16>(scores, B, H, n, k, values, scale, value_type, D, N, idx, w, out, stream);
    return launch_fused_vt<32>(scores, B, H, n, k, values, scale, value_type, D, N, idx, w, out, stream);
}

hipError_t launch_select(const float *scores, int64_t B, int H, int n, int k, int32_t *idx, float *w,
                         hipStream_t stream)
{
    const int64_t pairs = B * H;
    if (pairs <= 0) return hipSuccess;
    if (k < 1 || k > 64 || k > n) return hipErrorInvalidValue;
    static_assert(STAIR_SLOTS * 64 <= kMaxStaircaseCells, "the kernel reads the whole padded table");
    if (staircase_cells(k) > STAIR_SLOTS * 64) return hipErrorInvalidValue;
    const int mh = (n + 63) / 64;
    if (mh <= 4) return launch<4>(scores, pairs, n, k, idx, w, stream);
    if (mh <= 16) return launch<16>(scores, pairs, n, k, idx, w, stream);
    if (mh <= 32) return launch<32>(scores, pairs, n, k, idx, w, stream);
    return launch<64>(scores, pairs, n, k, idx, w, stream);
}

}  // namespace pkm
