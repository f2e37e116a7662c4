// fp32 MFMA GEMM for the two dense contractions of the lookup:
//   a1+a2  qhat = BN(x . Wq^T)         M = tokens, N = H*D,     K = D
//   a3     s_g  = qhat_g . C_g^T       M = tokens, N = n_keys,  K = D/2,
//                                      one batch entry g = 2h + p per half
// ("Product-Key Memory", code listing: the Linear + BatchNorm1d query and the
// two subkey products; §Factorising the key space for the split).
//
// Both operands are K-contiguous (x rows, Wq rows, qhat rows, subkey rows),
// so C = A . B^T with no transposes.  Scores decide the winners, so the
// contraction stays in fp32: v_mfma_f32_32x32x2_f32, fp32 accumulate.
//
// Tiling for CDNA4: a 256-thread workgroup owns a 128x128 tile of C; its four
// wave64s each own 64x64 (2x2 MFMA blocks of 32x32, 64 accumulators per
// lane).  K advances 32 at a time through one LDS stage per operand
// (128 rows x 32 floats, rows padded to 36 floats so the 16-byte fragment
// reads of consecutive rows fall on distinct banks); the next stage is
// prefetched into registers while the MFMAs run.  Within a 32-wide K chunk
// MFMA step t pairs k = t (lanes 0-31) with k = 16 + t (lanes 32-63), which
// makes every lane's fragments 16 contiguous floats (four ds_read_b128).
#include "pkm_internal.h"

namespace pkm {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 32;
constexpr int LDS_STRIDE = BK + 4;  // floats per LDS row
constexpr int THREADS = 256;

typedef float floatx16 __attribute__((ext_vector_type(16)));

template <bool BN_EPILOGUE>
__global__ __launch_bounds__(THREADS, 2) void gemm_nt_f32_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) float As[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) float Bs[BN * LDS_STRIDE];

    const int tiles_n = (a.N + BN - 1) / BN;
    const int tm = blockIdx.x / tiles_n;
    const int tn = blockIdx.x - tm * tiles_n;
    const int g = blockIdx.y;
    const float *A = a.A + (int64_t)g * a.strideA;
    const float *Bmat = a.B + (int64_t)g * a.strideB;
    float *C = a.C + (int64_t)g * a.strideC;
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // Global -> register mapping: thread t moves float4 column (t & 7) of
    // rows (t >> 3) + 32 i, i < 4, of both operand tiles.  Rows past the
    // matrix edge re-read the last row; their results are never stored.
    const int lc4 = tid & 7;
    const int lr = tid >> 3;
    const float *ap[4];
    const float *bp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int am = min(m0 + lr + 32 * i, a.M - 1);
        int bn = min(n0 + lr + 32 * i, a.N - 1);
        ap[i] = A + (int64_t)am * a.lda + lc4 * 4;
        bp[i] = Bmat + (int64_t)bn * a.ldb + lc4 * 4;
    }
    float4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define PKM_GLOAD(k0)                                                  \
    do {                                                               \
        ra0 = *reinterpret_cast<const float4 *>(ap[0] + (k0));         \
        ra1 = *reinterpret_cast<const float4 *>(ap[1] + (k0));         \
        ra2 = *reinterpret_cast<const float4 *>(ap[2] + (k0));         \
        ra3 = *reinterpret_cast<const float4 *>(ap[3] + (k0));         \
        rb0 = *reinterpret_cast<const float4 *>(bp[0] + (k0));         \
        rb1 = *reinterpret_cast<const float4 *>(bp[1] + (k0));         \
        rb2 = *reinterpret_cast<const float4 *>(bp[2] + (k0));         \
        rb3 = *reinterpret_cast<const float4 *>(bp[3] + (k0));         \
    } while (0)
    float *as_w = &As[lr * LDS_STRIDE + lc4 * 4];
    float *bs_w = &Bs[lr * LDS_STRIDE + lc4 * 4];
#define PKM_SSTORE()                                                                   \
    do {                                                                               \
        *reinterpret_cast<float4 *>(as_w + 0 * 32 * LDS_STRIDE) = ra0;                 \
        *reinterpret_cast<float4 *>(as_w + 1 * 32 * LDS_STRIDE) = ra1;                 \
        *reinterpret_cast<float4 *>(as_w + 2 * 32 * LDS_STRIDE) = ra2;                 \
        *reinterpret_cast<float4 *>(as_w + 3 * 32 * LDS_STRIDE) = ra3;                 \
        *reinterpret_cast<float4 *>(bs_w + 0 * 32 * LDS_STRIDE) = rb0;                 \
        *reinterpret_cast<float4 *>(bs_w + 1 * 32 * LDS_STRIDE) = rb1;                 \
        *reinterpret_cast<float4 *>(bs_w + 2 * 32 * LDS_STRIDE) = rb2;                 \
        *reinterpret_cast<float4 *>(bs_w + 3 * 32 * LDS_STRIDE) = rb3;                 \
    } while (0)

    floatx16 acc[2][2];
#pragma unroll
    for (int si = 0; si < 2; ++si)
#pragma unroll
        for (int sj = 0; sj < 2; ++sj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[si][sj][v] = 0.0f;

    const int il = lane & 31;  // row (A) / column (B) inside a 32x32 block
    const int kk = lane >> 5;  // which k of the MFMA's pair this lane feeds

    PKM_GLOAD(0);
    PKM_SSTORE();
    __syncthreads();
    const int KT = a.K / BK;
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) PKM_GLOAD((kt + 1) * BK);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float4 af[2], bf[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                af[s] = *reinterpret_cast<const float4 *>(&As[(wm * 64 + s * 32 + il) * LDS_STRIDE + kk * 16 + q * 4]);
                bf[s] = *reinterpret_cast<const float4 *>(&Bs[(wn * 64 + s * 32 + il) * LDS_STRIDE + kk * 16 + q * 4]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int si = 0; si < 2; ++si)
#pragma unroll
                    for (int sj = 0; sj < 2; ++sj)
                        acc[si][sj] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[si][e], bf[sj][e], acc[si][sj], 0, 0, 0);
        }
        __syncthreads();
        if (kt + 1 < KT) {
            PKM_SSTORE();
            __syncthreads();
        }
    }
#undef PKM_GLOAD
#undef PKM_SSTORE

    // 32x32 accumulator layout: register v of lane l holds row
    // 8*(v/4) + 4*(l/32) + v%4, column l%32.
#pragma unroll
    for (int sj = 0; sj < 2; ++sj) {
        const int col = n0 + wn * 64 + sj * 32 + il;
        if (col >= a.N) continue;
        float mean = 0.0f, mul = 1.0f, beta = 0.0f;
        if (BN_EPILOGUE) {
            mean = a.bn_mean[col];
            mul = a.bn_gamma[col] / sqrtf(a.bn_var[col] + a.bn_eps);
            beta = a.bn_beta[col];
        }
#pragma unroll
        for (int si = 0; si < 2; ++si) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * 64 + si * 32 + (v >> 2) * 8 + kk * 4 + (v & 3);
                if (row < a.M) {
                    float c = acc[si][sj][v];
                    if (BN_EPILOGUE) c = (c - mean) * mul + beta;
                    C[(int64_t)row * a.ldc + col] = c;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_nt_f32(const GemmArgs &a, hipStream_t stream)
{
    if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
    const int64_t tiles = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (tiles > 0x7FFFFFFF || a.batch > 65535) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)tiles, a.batch);
    if (a.bn_mean)
        hipLaunchKernelGGL(gemm_nt_f32_kernel<true>, grid, dim3(THREADS), 0, stream, a);
    else
        hipLaunchKernelGGL(gemm_nt_f32_kernel<false>, grid, dim3(THREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkm
