// The backward direction of the lookup: gradients of a loss L given
// dout = dL/dout, through steps a7 -> a1 for the winners the forward chose
// (the top-k selections pass gradient only to the winning scores; "Product-
// Key Memory", the code listing's forward, read backwards).  For token b,
// head h and winner j (flat row r_j = i0_j * n + i1_j, weight w_j):
//   g_j   = dout_b . V[r_j]                      value_backward_kernel
//   dt_j  = w_j (g_j - sum_l w_l g_l)            (softmax)
//   ds_p[i_p(j)] += dt_j                          dqhat_kernel: the dense
//                                                 [2H][n][tokens] matrix G
//   dq^_p = sum_j dt_j C[h,p,i_p(j)]              dqhat_kernel
//   dq    = dq^ gamma / sqrt(var + eps)           dqhat_kernel
//   dgamma += dq^ xhat, dbeta += dq^              colsum kernels (token order)
//   dWq[h] += dq^T x, dx = dq Wq                  fp32-accurate MFMA GEMMs
//   dC[h,p,i] += sum_b G[h,p][i][b] q^_p[b]       dsub_kernel (G is ~k/n
//                                                 dense: a scan per subkey
//                                                 row, not a GEMM)
//   dV[r] += sum over the occurrences of r of w dout_b
//                                                 counting sort by row, then
//                                                 one owner per row
// Every sum runs in a fixed order (no floating-point atomics), so the
// gradients are bitwise reproducible.
#include "pkm_internal.h"
#include "wave_ops.h"

namespace pkm {
namespace {

constexpr int WAVES = 4;  // waves per 256-thread workgroup

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
struct Fmt<4> {  // int4, two per byte (even element low) + row scale
    static constexpr int EPL = 32;
    static constexpr int BYTES = 0;  // half a byte per element: see elem_bytes
};

template <int VT>
__host__ __device__ __forceinline__ int64_t elem_bytes(int64_t c)
{
    return VT == 4 ? c / 2 : c * Fmt<VT>::BYTES;
}

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));

// Loads of data read once per call (table rows, the old value-gradient
// rows), non-temporal so they do not displace what the caches hold for the
// rest of the pass (measured: the backward 1.81 -> 1.72 ms, same results).
__device__ __forceinline__ uint4 load_once(const uint8_t *p)
{
    const u4v t = __builtin_nontemporal_load(reinterpret_cast<const u4v *>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ float4 load_once(const float *p)
{
    const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
}

// dot of EPL decoded values with EPL fp32 values
template <int VT>
__device__ __forceinline__ float dot_row(const uint4 &v, const float *d)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float s = 0.0f;
    if constexpr (VT == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s = fmaf(__uint_as_float(w[i]), d[i], s);
    } else if constexpr (VT == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s = fmaf(__uint_as_float(w[i] << 16), d[2 * i], s);
            s = fmaf(__uint_as_float(w[i] & 0xFFFF0000u), d[2 * i + 1], s);
        }
    } else if constexpr (VT == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const floatx2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
            const floatx2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
            s = fmaf(lo.x, d[4 * i], s);
            s = fmaf(lo.y, d[4 * i + 1], s);
            s = fmaf(hi.x, d[4 * i + 2], s);
            s = fmaf(hi.y, d[4 * i + 3], s);
        }
    } else if constexpr (VT == 3) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) s = fmaf((float)(int32_t)__builtin_amdgcn_sbfe((int)w[i], 8 * j, 8), d[4 * i + j], s);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) s = fmaf((float)(int32_t)__builtin_amdgcn_sbfe((int)w[i], 4 * j, 4), d[8 * i + j], s);
    }
    return s;
}

__global__ __launch_bounds__(256) void fill_kernel(uint32_t *__restrict__ p, int64_t count, uint32_t v)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) p[i] = v;
}

// out[c][r] = f(in[r][c]) for r < R, c < C; out[c][r] = 0 for R <= r < Rp.
// With AFFINE, f is inference BN of column c: (v - mean) gamma / sqrt(var +
// eps) + beta.  64 x 64 tiles through LDS (65-float rows: conflict-free
// column reads).
template <bool AFFINE>
__global__ __launch_bounds__(256) void transpose_kernel(const float *__restrict__ in, int64_t ld_in, int R, int C,
                                                        float *__restrict__ out, int64_t ld_out, int Rp,
                                                        const float *__restrict__ mean, const float *__restrict__ var,
                                                        const float *__restrict__ gamma,
                                                        const float *__restrict__ beta, float eps)
{
    __shared__ float tile[64][65];
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
    const int c = c0 + tx;
    float mul = 1.0f, mu = 0.0f, be = 0.0f;
    if (AFFINE && c < C) {
        mu = mean[c];
        mul = gamma[c] / sqrtf(var[c] + eps);
        be = beta[c];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = r0 + ty + 4 * i;
        float v = 0.0f;
        if (r < R && c < C) {
            v = in[(int64_t)r * ld_in + c];
            if (AFFINE) v = (v - mu) * mul + be;
        }
        tile[ty + 4 * i][tx] = v;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int oc = c0 + ty + 4 * i, orow = r0 + tx;
        if (oc < C && orow < Rp) out[(int64_t)oc * ld_out + orow] = tile[tx][ty + 4 * i];
    }
}

// One wave per (token, head): g_j = dout_b . V[r_j] for the k winners, then
// the softmax backward dt_j = w_j (g_j - sum_l w_l g_l).  Each lane reads
// 16-byte pieces of a row (one coalesced 1 KiB request per row slice), U
// rows in flight; the row's partial dots are summed across the wave.
template <int VT>
__global__ __launch_bounds__(64 * WAVES) void value_backward_kernel(const uint8_t *__restrict__ values,
                                                                     const float *__restrict__ scale, int D, int N,
                                                                     int64_t pairs, int H, int k, int slices,
                                                                     const int32_t *__restrict__ idx,
                                                                     const float *__restrict__ w,
                                                                     const float *__restrict__ dout,
                                                                     float *__restrict__ dt)
{
    constexpr int EPL = Fmt<VT>::EPL, U = 8;
    const int lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
    if (pair >= pairs) return;
    const int64_t b = pair / H;
    const int64_t row_bytes = elem_bytes<VT>(D);
    const int my_row = lane < k ? min(max(idx[pair * k + lane], 0), N - 1) : 0;
    const float my_w = lane < k ? w[pair * k + lane] : 0.0f;
    float my_g = 0.0f;
    for (int j0 = 0; j0 < k; j0 += U) {
        float part[U];
#pragma unroll
        for (int u = 0; u < U; ++u) part[u] = 0.0f;
        for (int s = 0; s < slices; ++s) {
            const int c0 = (s * 64 + lane) * EPL;
            const bool active = c0 < D;
            float dv[EPL];
#pragma unroll
            for (int e = 0; e < EPL / 4; ++e) {
                const float4 f = active ? *reinterpret_cast<const float4 *>(dout + b * D + c0 + 4 * e)
                                        : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                dv[4 * e] = f.x;
                dv[4 * e + 1] = f.y;
                dv[4 * e + 2] = f.z;
                dv[4 * e + 3] = f.w;
            }
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = __builtin_amdgcn_readlane(my_row, min(j0 + u, k - 1));
                v[u] = active ? load_once(values + (int64_t)r * row_bytes + elem_bytes<VT>(c0)) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) part[u] += dot_row<VT>(v[u], dv);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (j0 + u >= k) break;
            float g = wave_sum(part[u]);
            if constexpr (VT >= 2) g *= scale[__builtin_amdgcn_readlane(my_row, j0 + u)];
            if (lane == j0 + u) my_g = g;
        }
    }
    const float wg = wave_sum(lane < k ? my_w * my_g : 0.0f);
    if (lane < k) dt[pair * k + lane] = my_w * (my_g - wg);
}

// One wave per (token b, head h) of the chunk.  First the half-score
// gradients: for half p the winners sharing a subkey index i add up,
//   ds_p[i] = sum of dt_j over the winners j with i_p(j) = i  (j in order),
// kept by the winner that first uses i (G[2h+p][i][b] = ds_p[i]; G is zero
// elsewhere).  Then, over the distinct subkeys only (in order of first use),
//   dq^[d] = sum_i ds_p(d)[i] C[h, p(d), i, d - p(d) D/2]
//   dq[d]  = dq^[d] gamma / sqrt(var + eps).
// Lane l owns columns 4 l + 256 t (float4 loads and stores).
__global__ __launch_bounds__(64 * WAVES) void dqhat_kernel(const float *__restrict__ subkeys,
                                                          const float *__restrict__ var,
                                                          const float *__restrict__ gamma, float eps, int D, int n,
                                                          int64_t pairs, int H, int k,
                                                          const int32_t *__restrict__ idx,
                                                          const float *__restrict__ dt, float *__restrict__ dqhat,
                                                          float *__restrict__ dq, float *__restrict__ G,
                                                          int64_t ldG)
{
    const int lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
    if (pair >= pairs) return;
    const int64_t b = pair / H;
    const int h = (int)(pair - b * H);
    const int half = D / 2;
    const int N = n * n;
    const int my_row = lane < k ? min(max(idx[pair * k + lane], 0), N - 1) : 0;
    const float my_dt = lane < k ? dt[pair * k + lane] : 0.0f;
    const int my_a = my_row / n, my_c = my_row - (my_row / n) * n;

    float s0 = 0.0f, s1 = 0.0f;
    bool first0 = lane < k, first1 = lane < k;
    for (int l = 0; l < k; ++l) {
        const int al = __builtin_amdgcn_readlane(my_a, l), cl = __builtin_amdgcn_readlane(my_c, l);
        const float dl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_dt), l));
        if (al == my_a) {
            s0 += dl;
            if (l < lane) first0 = false;
        }
        if (cl == my_c) {
            s1 += dl;
            if (l < lane) first1 = false;
        }
    }
    if (first0) G[(((int64_t)h * 2 + 0) * n + my_a) * ldG + b] = s0;
    if (first1) G[(((int64_t)h * 2 + 1) * n + my_c) * ldG + b] = s1;
    const uint64_t distinct0 = __ballot(first0), distinct1 = __ballot(first1);

    const float *c0base = subkeys + ((int64_t)h * 2 + 0) * n * half;
    const float *c1base = subkeys + ((int64_t)h * 2 + 1) * n * half;
    for (int col0 = 0; col0 < D; col0 += 256) {
        const int col = col0 + 4 * lane;
        const bool active = col < D;
        const int p = col >= half;
        const int sub_col = active ? col - p * half : 0;
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        // both halves' lists; a lane takes the entries of its own half
        for (int q = 0; q < 2; ++q) {
            uint64_t m = q ? distinct1 : distinct0;
            const float *base = q ? c1base : c0base;
            const bool mine = active && p == q;
            while (m) {
                const int l = __builtin_ctzll(m);
                m &= m - 1;
                const int i = __builtin_amdgcn_readlane(q ? my_c : my_a, l);
                const float sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(q ? s1 : s0), l));
                if (mine) {
                    const float4 cv = *reinterpret_cast<const float4 *>(base + (int64_t)i * half + sub_col);
                    acc.x = fmaf(sv, cv.x, acc.x);
                    acc.y = fmaf(sv, cv.y, acc.y);
                    acc.z = fmaf(sv, cv.z, acc.z);
                    acc.w = fmaf(sv, cv.w, acc.w);
                }
            }
        }
        if (active) {
            const int64_t hd = (int64_t)h * D + col;
            const float4 vv = *reinterpret_cast<const float4 *>(var + hd);
            const float4 gg = *reinterpret_cast<const float4 *>(gamma + hd);
            *reinterpret_cast<float4 *>(dqhat + pair * D + col) = acc;
            *reinterpret_cast<float4 *>(dq + pair * D + col) =
                make_float4(acc.x * (gg.x / sqrtf(vv.x + eps)), acc.y * (gg.y / sqrtf(vv.y + eps)),
                            acc.z * (gg.z / sqrtf(vv.z + eps)), acc.w * (gg.w / sqrtf(vv.w + eps)));
        }
    }
}

// dC[h,p,i] += sum over tokens b (in order) of G[2h+p][i][b] * q^_p[b]:
// one wave per subkey row (g = 2h + p, i).  The wave scans its row of G
// (one token per lane, four 64-token chunks in flight) and, for each
// non-zero entry, adds ds * q^ with q^ = BN(q) of that token's half p
// computed on the fly from q.  Columns: lane l owns 4 l + 256 t of the
// D/2, in passes of 1024.
__global__ __launch_bounds__(64 * WAVES) void dsub_kernel(const float *__restrict__ G, int64_t ldG, int64_t B,
                                                         const float *__restrict__ q, int H, int D, int n,
                                                         const float *__restrict__ mean,
                                                         const float *__restrict__ var,
                                                         const float *__restrict__ gamma,
                                                         const float *__restrict__ beta, float eps,
                                                         float *__restrict__ dsub)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);  // g * n + i
    if (row >= (int64_t)2 * H * n) return;
    const int g = (int)(row / n);
    const int h = g >> 1, p = g & 1;
    const int half = D / 2;
    const int64_t qcol0 = (int64_t)h * D + (int64_t)p * half;  // this half's first column in q's rows
    const int64_t ldq = (int64_t)H * D;
    const float *grow = G + row * ldG;
    float *out = dsub + row * half;
    for (int c1 = 0; c1 < half; c1 += 1024) {
        int col[4];
        bool act[4];
        float4 mu[4], sc[4], be[4], acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c = c1 + 256 * t + 4 * lane;
            act[t] = c < half;
            col[t] = act[t] ? c : 0;
            const int64_t hd = qcol0 + col[t];
            const float4 m4 = *reinterpret_cast<const float4 *>(mean + hd);
            const float4 v4 = *reinterpret_cast<const float4 *>(var + hd);
            const float4 g4 = *reinterpret_cast<const float4 *>(gamma + hd);
            mu[t] = m4;
            sc[t] = make_float4(g4.x / sqrtf(v4.x + eps), g4.y / sqrtf(v4.y + eps), g4.z / sqrtf(v4.z + eps),
                                g4.w / sqrtf(v4.w + eps));
            be[t] = *reinterpret_cast<const float4 *>(beta + hd);
            acc[t] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        for (int64_t b0 = 0; b0 < B; b0 += 256) {
            float gv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t b = b0 + 64 * c + lane;
                gv[c] = b < B ? grow[b] : 0.0f;
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                uint64_t nz = __ballot(gv[c] != 0.0f);
                while (nz) {
                    const int l = __builtin_ctzll(nz);
                    nz &= nz - 1;
                    const float ds = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv[c]), l));
                    const float *qrow = q + (b0 + 64 * c + l) * ldq + qcol0;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float4 v = act[t] ? *reinterpret_cast<const float4 *>(qrow + col[t])
                                                : make_float4(0, 0, 0, 0);
                        acc[t].x = fmaf(ds, (v.x - mu[t].x) * sc[t].x + be[t].x, acc[t].x);
                        acc[t].y = fmaf(ds, (v.y - mu[t].y) * sc[t].y + be[t].y, acc[t].y);
                        acc[t].z = fmaf(ds, (v.z - mu[t].z) * sc[t].z + be[t].z, acc[t].z);
                        acc[t].w = fmaf(ds, (v.w - mu[t].w) * sc[t].w + be[t].w, acc[t].w);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (act[t]) {
                const float4 o = *reinterpret_cast<const float4 *>(out + col[t]);
                *reinterpret_cast<float4 *>(out + col[t]) =
                    make_float4(o.x + acc[t].x, o.y + acc[t].y, o.z + acc[t].z, o.w + acc[t].w);
            }
    }
}

// dgamma / dbeta, pass 1: partial sums over 64-token chunks, in token
// order: part[chunk][col] for col = h * D + d.
constexpr int kColChunk = 64;
__global__ __launch_bounds__(256) void colsum_partial_kernel(const float *__restrict__ dqhat,
                                                             const float *__restrict__ q,
                                                             const float *__restrict__ mean,
                                                             const float *__restrict__ var, float eps, int64_t B,
                                                             int cols, float *__restrict__ part_g,
                                                             float *__restrict__ part_b)
{
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= cols) return;
    const int64_t t0 = (int64_t)blockIdx.y * kColChunk;
    const int n = (int)min((int64_t)kColChunk, B - t0);
    const float mu = mean[col], inv = 1.0f / sqrtf(var[col] + eps);
    // the chunk's rows loaded together (rows past B repeat the last one and
    // are not added), then summed in row order
    float g[kColChunk], x[kColChunk];
#pragma unroll
    for (int i = 0; i < kColChunk; ++i) {
        const int64_t t = t0 + min(i, n - 1);
        g[i] = dqhat[t * cols + col];
        x[i] = q[t * cols + col];
    }
    float sg = 0.0f, sb = 0.0f;
#pragma unroll
    for (int i = 0; i < kColChunk; ++i)
        if (i < n) {
            sg = fmaf(g[i], (x[i] - mu) * inv, sg);
            sb += g[i];
        }
    part_g[(int64_t)blockIdx.y * cols + col] = sg;
    part_b[(int64_t)blockIdx.y * cols + col] = sb;
}

// pass 2: the sums of the partials in chunk order, added to dgamma / dbeta
// and stored to sum_g / sum_b (each pair optional).
__global__ __launch_bounds__(256) void colsum_final_kernel(const float *__restrict__ part_g,
                                                           const float *__restrict__ part_b, int chunks, int cols,
                                                           float *__restrict__ dgamma, float *__restrict__ dbeta,
                                                           float *__restrict__ sum_g, float *__restrict__ sum_b)
{
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= cols) return;
    float sg = 0.0f, sb = 0.0f;
#pragma unroll 8
    for (int c = 0; c < chunks; ++c) {
        sg += part_g[(int64_t)c * cols + col];
        sb += part_b[(int64_t)c * cols + col];
    }
    if (dgamma) {
        dgamma[col] += sg;
        dbeta[col] += sb;
    }
    if (sum_g) {
        sum_g[col] = sg;
        sum_b[col] = sb;
    }
}

// ---- value gradient: counting sort of the occurrences by row.

__global__ __launch_bounds__(256) void count_rows_kernel(const int32_t *__restrict__ idx, int64_t M, int N,
                                                         uint32_t *__restrict__ count)
{
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o < M) atomicAdd(&count[min(max(idx[o], 0), N - 1)], 1u);
}

// Exclusive scan of count[0, N) into offs, in blocks of kScanBlock.
constexpr int kScanBlock = 4096;  // 256 threads x 16

__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *lds, uint32_t &total)
{
    // 256 threads: inclusive scan in LDS (Hillis-Steele), then shift
    const int t = threadIdx.x;
    lds[t] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const uint32_t add = t >= off ? lds[t - off] : 0u;
        __syncthreads();
        lds[t] += add;
        __syncthreads();
    }
    total = lds[255];
    const uint32_t excl = lds[t] - v;
    __syncthreads();
    return excl;
}

// FLAGS: scan (count > 0) instead of count (the positions of the touched
// rows among themselves)
template <bool FLAGS>
__global__ __launch_bounds__(256) void scan_sums_kernel(const uint32_t *__restrict__ count, int N,
                                                        uint32_t *__restrict__ block_sum)
{
    __shared__ uint32_t lds[256];
    const int64_t base = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * 16;
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t c = base + i < N ? count[base + i] : 0u;
        s += FLAGS ? (c != 0u) : c;
    }
    uint32_t total;
    block_exclusive_scan(s, lds, total);
    if (threadIdx.x == 0) block_sum[blockIdx.x] = total;
}

// One workgroup: exclusive scan of the block sums in place (nb <= 256 * 64);
// the grand total to *total when given.
__global__ __launch_bounds__(256) void scan_top_kernel(uint32_t *__restrict__ block_sum, int nb,
                                                       int64_t *__restrict__ total_out)
{
    __shared__ uint32_t lds[256];
    uint32_t carry = 0;
    for (int b0 = 0; b0 < nb; b0 += 256) {
        const int i = b0 + threadIdx.x;
        const uint32_t v = i < nb ? block_sum[i] : 0u;
        uint32_t total;
        const uint32_t excl = block_exclusive_scan(v, lds, total);
        if (i < nb) block_sum[i] = carry + excl;
        carry += total;
    }
    if (total_out && threadIdx.x == 0) *total_out = (int64_t)carry;
}

template <bool FLAGS>
__global__ __launch_bounds__(256) void scan_apply_kernel(const uint32_t *__restrict__ count, int N,
                                                         const uint32_t *__restrict__ block_off,
                                                         uint32_t *__restrict__ offs)
{
    __shared__ uint32_t lds[256];
    const int64_t base = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * 16;
    uint32_t v[16], s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t c = base + i < N ? count[base + i] : 0u;
        v[i] = FLAGS ? (c != 0u) : c;
        s += v[i];
    }
    uint32_t total;
    uint32_t run = block_off[blockIdx.x] + block_exclusive_scan(s, lds, total);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (base + i < N) offs[base + i] = run;
        run += v[i];
    }
}

__global__ __launch_bounds__(256) void fill_lists_kernel(const int32_t *__restrict__ idx, int64_t M, int N,
                                                         const uint32_t *__restrict__ offs,
                                                         uint32_t *__restrict__ cursor, uint32_t *__restrict__ list)
{
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= M) return;
    const int r = min(max(idx[o], 0), N - 1);
    list[offs[r] + atomicAdd(&cursor[r], 1u)] = (uint32_t)o;
}

// dV[r] += sum over the occurrences o of r, in increasing o (token, head,
// winner), of w[o] * dout[token(o)].  SPARSE: the sum alone goes to row
// pos[r] of a compact [U][D] array and r to rows[pos[r]] (no old row read).
// One wave per ROWS rows (8 dense, 2 sparse: measured best); the wave
// takes its non-empty rows in turn.  Up to 64 occurrences are put in order
// by a 64-lane bitonic sort (lane t holds the t-th) and summed over passes
// of 1024 columns (lane l: columns 4 l + 256 q, q < 4; the old row and two
// occurrences' dout rows in flight), then added to the row; more are
// walked by repeated minimum search, each added into the row in turn.
constexpr int kGradRowsDense = 8, kGradRowsSparse = 2;
template <bool SPARSE, int ROWS>
__global__ __launch_bounds__(64 * WAVES) void value_grad_kernel(const uint32_t *__restrict__ count,
                                                               const uint32_t *__restrict__ offs,
                                                               const uint32_t *__restrict__ list, int N, int D,
                                                               int per_token, const float *__restrict__ w,
                                                               const float *__restrict__ dout,
                                                               float *__restrict__ dval,
                                                               const uint32_t *__restrict__ pos,
                                                               int32_t *__restrict__ rows)
{
    const int lane = threadIdx.x & 63;
    const int64_t group = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
    if (group * ROWS >= N) return;
    const int64_t r_lane = group * ROWS + lane;
    const bool mine = lane < ROWS && r_lane < N;
    const uint32_t my_count = mine ? count[r_lane] : 0u;
    const uint32_t my_start = mine ? offs[r_lane] : 0u;
    uint64_t pending = __ballot(my_count > 0);
    while (pending) {
        const int src = __builtin_ctzll(pending);
        pending &= pending - 1;
        const int64_t r = group * ROWS + src;
        const uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)my_count, src);
        const uint32_t start = (uint32_t)__builtin_amdgcn_readlane((int)my_start, src);
        float *out = dval + (SPARSE ? (int64_t)pos[r] : r) * D;
        if (SPARSE && lane == 0) rows[pos[r]] = (int32_t)r;
        if (m <= 64) {
            const uint32_t id = lane < (int)m ? list[start + lane] : 0xFFFFFFFFu;
            const uint32_t asc = m == 1 ? id : ~sort64_desc(~id);  // lane t: the t-th smallest id
            const float wt = lane < (int)m ? w[asc] : 0.0f;
            const uint32_t tok = lane < (int)m ? asc / (uint32_t)per_token : 0u;
            for (int c1 = 0; c1 < D; c1 += 1024) {
                int col[4];
                bool act[4];
                float4 old[4], acc[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = c1 + 256 * q + 4 * lane;
                    act[q] = c < D;
                    col[q] = act[q] ? c : 0;
                    old[q] = act[q] && !SPARSE ? load_once(out + col[q]) : make_float4(0, 0, 0, 0);
                    acc[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                }
                for (uint32_t t0 = 0; t0 < m; t0 += 2) {
                    float4 v[2][4];
                    float wv[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int t = (int)min(t0 + u, m - 1);
                        const float *src_row = dout + (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)tok, t) * D;
                        wv[u] = t0 + u < m ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), t)) : 0.0f;
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            v[u][q] = act[q] ? *reinterpret_cast<const float4 *>(src_row + col[q])
                                             : make_float4(0, 0, 0, 0);
                    }
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            acc[q].x = fmaf(wv[u], v[u][q].x, acc[q].x);
                            acc[q].y = fmaf(wv[u], v[u][q].y, acc[q].y);
                            acc[q].z = fmaf(wv[u], v[u][q].z, acc[q].z);
                            acc[q].w = fmaf(wv[u], v[u][q].w, acc[q].w);
                        }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (act[q]) {
                        const float4 nv = make_float4(old[q].x + acc[q].x, old[q].y + acc[q].y, old[q].z + acc[q].z,
                                                      old[q].w + acc[q].w);
                        // written once per call: stream it out of the caches
                        const f4v nvv = {nv.x, nv.y, nv.z, nv.w};
                        __builtin_nontemporal_store(nvv, reinterpret_cast<f4v *>(out + col[q]));
                    }
            }
        } else {
            // more than 64: walk the occurrences in increasing id (one wave
            // minimum per step), adding each into the row
            if (SPARSE)
                for (int d = lane; d < D; d += 64) out[d] = 0.0f;
            int64_t last = -1;
            for (uint32_t t = 0; t < m; ++t) {
                uint32_t best = 0xFFFFFFFFu;
                for (uint32_t e = lane; e < m; e += 64) {
                    const uint32_t v = list[start + e];
                    if ((int64_t)v > last && v < best) best = v;
                }
                const uint32_t o = ~(uint32_t)__builtin_amdgcn_readlane((int)sort64_desc(~best), 0);
                last = o;
                const float wo = w[o];
                const float *src_row = dout + (int64_t)(o / per_token) * D;
                for (int d = lane; d < D; d += 64) out[d] = fmaf(wo, src_row[d], out[d]);
            }
        }
    }
}

template <int VT>
hipError_t launch_value_backward(const void *values, const float *scale, int D, int N, int64_t pairs, int H, int k,
                                 const int32_t *idx, const float *w, const float *dout, float *dt, hipStream_t st)
{
    const int slices = (int)((elem_bytes<VT>(D) + 1023) / 1024);
    const int64_t blocks = (pairs + WAVES - 1) / WAVES;
    hipLaunchKernelGGL(value_backward_kernel<VT>, dim3((unsigned)blocks), dim3(64 * WAVES), 0, st,
                       static_cast<const uint8_t *>(values), scale, D, N, pairs, H, k, slices, idx, w, dout, dt);
    return hipGetLastError();
}

unsigned grid_of(int64_t items, int per_block) { return (unsigned)((items + per_block - 1) / per_block); }

}  // namespace

hipError_t launch_fill(uint32_t *p, int64_t count, uint32_t value, hipStream_t st)
{
    if (count <= 0) return hipSuccess;
    const int64_t blocks = (count + 255) / 256;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, st, p, count,
                       value);
    return hipGetLastError();
}

hipError_t launch_transpose(const float *in, int64_t ld_in, int R, int C, float *out, int64_t ld_out, int Rp,
                            const float *mean, const float *var, const float *gamma, const float *beta, float eps,
                            hipStream_t st)
{
    if (R < 0 || C <= 0 || Rp < R || Rp <= 0) return Rp == 0 ? hipSuccess : hipErrorInvalidValue;
    const dim3 grid(grid_of(Rp, 64), grid_of(C, 64));
    if (grid.y > 65535) return hipErrorInvalidConfiguration;
    if (mean)
        hipLaunchKernelGGL(transpose_kernel<true>, grid, dim3(256), 0, st, in, ld_in, R, C, out, ld_out, Rp, mean, var,
                           gamma, beta, eps);
    else
        hipLaunchKernelGGL(transpose_kernel<false>, grid, dim3(256), 0, st, in, ld_in, R, C, out, ld_out, Rp, nullptr,
                           nullptr, nullptr, nullptr, eps);
    return hipGetLastError();
}

hipError_t launch_value_backward(const void *values, const float *scale, int value_type, int D, int N, int64_t B,
                                 int H, int k, const int32_t *idx, const float *w, const float *dout, float *dt,
                                 hipStream_t st)
{
    if (B <= 0) return hipSuccess;
    const int64_t pairs = B * H;
    switch (value_type) {
    case 0: return launch_value_backward<0>(values, scale, D, N, pairs, H, k, idx, w, dout, dt, st);
    case 1: return launch_value_backward<1>(values, scale, D, N, pairs, H, k, idx, w, dout, dt, st);
    case 2: return launch_value_backward<2>(values, scale, D, N, pairs, H, k, idx, w, dout, dt, st);
    case 3: return launch_value_backward<3>(values, scale, D, N, pairs, H, k, idx, w, dout, dt, st);
    default: return launch_value_backward<4>(values, scale, D, N, pairs, H, k, idx, w, dout, dt, st);
    }
}

hipError_t launch_dqhat(const float *subkeys, const float *var, const float *gamma, float eps, int D, int n, int64_t B,
                        int H, int k, const int32_t *idx, const float *dt, float *dqhat, float *dq, float *G,
                        int64_t ldG, hipStream_t st)
{
    if (B <= 0) return hipSuccess;
    const int64_t pairs = B * H;
    hipLaunchKernelGGL(dqhat_kernel, dim3(grid_of(pairs, WAVES)), dim3(64 * WAVES), 0, st, subkeys, var, gamma, eps, D,
                       n, pairs, H, k, idx, dt, dqhat, dq, G, ldG);
    return hipGetLastError();
}

hipError_t launch_dsub(const float *G, int64_t ldG, int64_t B, const float *q, int H, int D, int n, const float *mean,
                       const float *var, const float *gamma, const float *beta, float eps, float *dsub,
                       hipStream_t st)
{
    if (B <= 0) return hipSuccess;
    hipLaunchKernelGGL(dsub_kernel, dim3(grid_of((int64_t)2 * H * n, WAVES)), dim3(64 * WAVES), 0, st, G, ldG, B, q, H,
                       D, n, mean, var, gamma, beta, eps, dsub);
    return hipGetLastError();
}

int colsum_chunks(int64_t B) { return (int)((B + kColChunk - 1) / kColChunk); }

hipError_t launch_bn_grads(const float *dqhat, const float *q, const float *mean, const float *var, float eps,
                           int64_t B, int cols, float *part_g, float *part_b, float *dgamma, float *dbeta,
                           float *sum_g, float *sum_b, hipStream_t st)
{
    if (B <= 0) return hipSuccess;
    const int chunks = colsum_chunks(B);
    if (chunks > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(colsum_partial_kernel, dim3(grid_of(cols, 256), chunks), dim3(256), 0, st, dqhat, q, mean, var,
                       eps, B, cols, part_g, part_b);
    hipLaunchKernelGGL(colsum_final_kernel, dim3(grid_of(cols, 256)), dim3(256), 0, st, part_g, part_b, chunks, cols,
                       dgamma, dbeta, sum_g, sum_b);
    return hipGetLastError();
}

int64_t scan_blocks(int N) { return (N + kScanBlock - 1) / kScanBlock; }

hipError_t launch_usage(const int32_t *idx, int64_t M, int N, uint32_t *counts, hipStream_t st)
{
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(count_rows_kernel, dim3(grid_of(M, 256)), dim3(256), 0, st, idx, M, N, counts);
    return hipGetLastError();
}

hipError_t launch_value_grad(const int32_t *idx, int64_t M, int N, int D, int per_token, const float *w,
                             const float *dout, uint32_t *count, uint32_t *cursor, uint32_t *offs,
                             uint32_t *block_sum, uint32_t *list, float *dval, int32_t *rows, int64_t *row_count,
                             hipStream_t st)
{
    if (M <= 0) return hipSuccess;
    const int64_t nb = scan_blocks(N);
    if (nb > 256 * 64) return hipErrorInvalidValue;
    hipError_t e;
    if ((e = launch_fill(count, N, 0u, st)) != hipSuccess || (e = launch_fill(cursor, N, 0u, st)) != hipSuccess)
        return e;
    hipLaunchKernelGGL(count_rows_kernel, dim3(grid_of(M, 256)), dim3(256), 0, st, idx, M, N, count);
    hipLaunchKernelGGL(scan_sums_kernel<false>, dim3((unsigned)nb), dim3(256), 0, st, count, N, block_sum);
    hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(256), 0, st, block_sum, (int)nb, nullptr);
    hipLaunchKernelGGL(scan_apply_kernel<false>, dim3((unsigned)nb), dim3(256), 0, st, count, N, block_sum, offs);
    hipLaunchKernelGGL(fill_lists_kernel, dim3(grid_of(M, 256)), dim3(256), 0, st, idx, M, N, offs, cursor, list);
    const dim3 block(64 * WAVES);
    if (rows) {
        // the touched rows' positions among themselves, into cursor (free
        // once the lists are filled), and their number
        hipLaunchKernelGGL(scan_sums_kernel<true>, dim3((unsigned)nb), dim3(256), 0, st, count, N, block_sum);
        hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(256), 0, st, block_sum, (int)nb, row_count);
        hipLaunchKernelGGL(scan_apply_kernel<true>, dim3((unsigned)nb), dim3(256), 0, st, count, N, block_sum,
                           cursor);
        const dim3 grid(grid_of((N + kGradRowsSparse - 1) / kGradRowsSparse, WAVES));
        hipLaunchKernelGGL((value_grad_kernel<true, kGradRowsSparse>), grid, block, 0, st, count, offs, list, N, D,
                           per_token, w, dout, dval, cursor, rows);
    } else {
        const dim3 grid(grid_of((N + kGradRowsDense - 1) / kGradRowsDense, WAVES));
        hipLaunchKernelGGL((value_grad_kernel<false, kGradRowsDense>), grid, block, 0, st, count, offs, list, N, D,
                           per_token, w, dout, dval, nullptr, nullptr);
    }
    return hipGetLastError();
}

}  // namespace pkm
