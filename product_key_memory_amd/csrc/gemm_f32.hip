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
// Tiling for CDNA4.  A workgroup owns a BM x BN tile of C; each of its
// WM x WN wave64s owns (BM/WM) x (BN/WN) as 32x32 MFMA blocks.  K advances
// BK at a time through LDS stages (rows padded by 4 floats so the 16-byte
// fragment reads of consecutive rows land on distinct banks); the next chunk
// is loaded into registers while the MFMAs run, and with two stages one
// barrier per chunk suffices.  Within a chunk, MFMA step t pairs k = t
// (lanes 0-31) with k = BK/2 + t (lanes 32-63), so each lane's fragment is
// BK/2 contiguous floats (ds_read_b128 only).
//   Large grids: 256x256 tiles, 8 waves of 64x128, BK 32, two stages
//   (147 KB of LDS, one workgroup per CU: operand traffic per flop halves
//   against 128x128).
//   Small grids (fewer tiles than CUs at 256x256): 128x128, 4 waves of
//   64x64, BK 32, one stage.
// A result that the next kernel reads once (the subkey scores) is stored
// non-temporally: it reaches HBM during this compute-bound kernel rather than
// being written back from the caches while the memory-bound gather runs.
//
// Flat exact search (the comparator for the product search of
// §Factorising the key space: every one of the n^2 concatenated keys
// scored by one full-length dot product).  The B operand is the virtual
// key matrix: row j = (a, c) is [C0[a]; C1[c]], read from the two subkey
// sets as K advances (a chunk never straddles the halves).  M is a few
// dozen tokens, so this uses 32 x 256 tiles: 4 waves of 32 x 64, one LDS
// stage (41 KiB, three workgroups per CU).
#include "pkm_internal.h"

#include <atomic>

namespace pkm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float fx4 __attribute__((ext_vector_type(4)));

constexpr int kCUs = 256;  // MI355X compute units

template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, STAGES = STAGES_;
    static constexpr int THREADS = 64 * WM * WN;
    static constexpr int LDS = BK + 4;                          // floats per LDS row
    static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;  // 32x32 blocks per wave
    static constexpr int HK = BK / 2;                           // k per lane half within a chunk
    static constexpr int C4 = BK / 4;                           // float4 per row chunk
    static constexpr int RPP = THREADS / C4;                    // rows moved per pass
    static constexpr int PA = BM / RPP, PB = BN / RPP;          // passes per operand
    static constexpr size_t LDS_BYTES = (size_t)STAGES * (BM + BN) * LDS * sizeof(float);
    static_assert(BM % RPP == 0 && BN % RPP == 0 && BK % 8 == 0, "tile shape");
};

using BigTile = Tile<256, 256, 32, 4, 2, 2>;
using SmallTile = Tile<128, 128, 32, 2, 2, 1>;
using KeyTile = Tile<32, 256, 32, 1, 4, 1>;

// B row pointers of a thread: plain rows, or the two halves of product keys
// (k < split reads the first half's row at k, else the second's at k - split).
template <typename T, bool PRODUCT_B>
struct BRows {
    const float *p0[T::PB];
    const float *p1[PRODUCT_B ? T::PB : 1];
    __device__ __forceinline__ const float *at(int i, int k, int split) const
    {
        if constexpr (PRODUCT_B) return k < split ? p0[i] + k : p1[i] + (k - split);
        return p0[i] + k;
    }
};

template <typename T, bool PRODUCT_B>
__device__ __forceinline__ void load_chunk(fx4 (&ra)[T::PA], fx4 (&rb)[T::PB], const float *const (&ap)[T::PA],
                                           const BRows<T, PRODUCT_B> &bp, int kt, int split)
{
#pragma unroll
    for (int i = 0; i < T::PA; ++i) ra[i] = *reinterpret_cast<const fx4 *>(ap[i] + kt * T::BK);
#pragma unroll
    for (int i = 0; i < T::PB; ++i) rb[i] = *reinterpret_cast<const fx4 *>(bp.at(i, kt * T::BK, split));
}

template <typename T>
__device__ __forceinline__ void store_chunk(const fx4 (&ra)[T::PA], const fx4 (&rb)[T::PB], float *as, float *bs,
                                            int lr, int lc4)
{
#pragma unroll
    for (int i = 0; i < T::PA; ++i) *reinterpret_cast<fx4 *>(&as[(lr + T::RPP * i) * T::LDS + lc4 * 4]) = ra[i];
#pragma unroll
    for (int i = 0; i < T::PB; ++i) *reinterpret_cast<fx4 *>(&bs[(lr + T::RPP * i) * T::LDS + lc4 * 4]) = rb[i];
}

template <typename T>
__device__ __forceinline__ void mfma_chunk(floatx16 (&acc)[T::TM][T::TN], const float *as, const float *bs, int wm,
                                           int wn, int il, int kk)
{
#pragma unroll
    for (int q = 0; q < T::HK / 4; ++q) {
        fx4 af[T::TM], bf[T::TN];
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
            af[i] = *reinterpret_cast<const fx4 *>(&as[(wm * T::TM * 32 + i * 32 + il) * T::LDS + kk * T::HK + q * 4]);
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
            bf[j] = *reinterpret_cast<const fx4 *>(&bs[(wn * T::TN * 32 + j * 32 + il) * T::LDS + kk * T::HK + q * 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][e], bf[j][e], acc[i][j], 0, 0, 0);
    }
}

template <typename T, bool BN_EPILOGUE, bool STREAM_OUT, bool PRODUCT_B = false, bool ACCUMULATE = false>
__global__ __launch_bounds__(T::THREADS) void gemm_nt_f32_kernel(GemmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float smem[];
    float *As = smem;
    float *Bs = smem + T::STAGES * T::BM * T::LDS;

    const int tiles_n = (a.N + T::BN - 1) / T::BN;
    const int tm = blockIdx.x / tiles_n;
    const int tn = blockIdx.x - tm * tiles_n;
    const int g = blockIdx.y;
    const float *A = a.A + (int64_t)g * a.strideA;
    const float *Bmat = a.B + (int64_t)g * a.strideB;
    float *C = a.C + (int64_t)g * a.strideC;
    const int m0 = tm * T::BM, n0 = tn * T::BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / T::WN, wn = wave % T::WN;

    // Global -> register mapping: thread t moves float4 column (t % C4) of
    // rows t / C4 + RPP * i of both operand tiles.  Rows past the matrix
    // edge re-read the last row; their results are never stored.
    const int lc4 = tid % T::C4;
    const int lr = tid / T::C4;
    const float *ap[T::PA];
    BRows<T, PRODUCT_B> bp;
#pragma unroll
    for (int i = 0; i < T::PA; ++i) ap[i] = A + (int64_t)min(m0 + lr + T::RPP * i, a.M - 1) * a.lda + lc4 * 4;
#pragma unroll
    for (int i = 0; i < T::PB; ++i) {
        const int j = min(n0 + lr + T::RPP * i, a.N - 1);
        if constexpr (PRODUCT_B) {
            const int ka = j / a.key_n, kc = j - ka * a.key_n;
            bp.p0[i] = Bmat + (int64_t)ka * a.ldb + lc4 * 4;
            bp.p1[i] = a.B2 + (int64_t)g * a.strideB + (int64_t)kc * a.ldb + lc4 * 4;
        } else {
            bp.p0[i] = Bmat + (int64_t)j * a.ldb + lc4 * 4;
        }
    }
    fx4 ra[T::PA], rb[T::PB];

    floatx16 acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int il = lane & 31;  // row (A) / column (B) inside a 32x32 block
    const int kk = lane >> 5;  // which k of the MFMA's pair this lane feeds
    const int KT = a.K / T::BK;

    load_chunk<T, PRODUCT_B>(ra, rb, ap, bp, 0, a.split_k);
    store_chunk<T>(ra, rb, As, Bs, lr, lc4);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int s = T::STAGES == 1 ? 0 : (kt & 1);
        if (kt + 1 < KT) load_chunk<T, PRODUCT_B>(ra, rb, ap, bp, kt + 1, a.split_k);
        mfma_chunk<T>(acc, As + s * T::BM * T::LDS, Bs + s * T::BN * T::LDS, wm, wn, il, kk);
        if constexpr (T::STAGES == 1) {
            __syncthreads();
            if (kt + 1 < KT) {
                store_chunk<T>(ra, rb, As, Bs, lr, lc4);
                __syncthreads();
            }
        } else {
            // stage s ^ 1 was last read in the previous chunk, before the
            // barrier that closed it
            if (kt + 1 < KT)
                store_chunk<T>(ra, rb, As + (s ^ 1) * T::BM * T::LDS, Bs + (s ^ 1) * T::BN * T::LDS, lr, lc4);
            __syncthreads();
        }
    }

    // 32x32 accumulator layout: register v of lane l holds row
    // 8*(v/4) + 4*(l/32) + v%4, column l%32.
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
        const int col = n0 + wn * T::TN * 32 + j * 32 + il;
        if (col >= a.N) continue;
        float mean = 0.0f, mul = 1.0f, beta = 0.0f;
        if (BN_EPILOGUE) {
            mean = a.bn_mean[col];
            mul = a.bn_gamma[col] / sqrtf(a.bn_var[col] + a.bn_eps);
            beta = a.bn_beta[col];
        }
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * T::TM * 32 + i * 32 + (v >> 2) * 8 + kk * 4 + (v & 3);
                if (row < a.M) {
                    float c = acc[i][j][v];
                    if (BN_EPILOGUE) c = (c - mean) * mul + beta;
                    if (ACCUMULATE) c += C[(int64_t)row * a.ldc + col];
                    if (STREAM_OUT)
                        __builtin_nontemporal_store(c, &C[(int64_t)row * a.ldc + col]);
                    else
                        C[(int64_t)row * a.ldc + col] = c;
                }
            }
        }
    }
}

template <typename T>
int64_t tile_count(const GemmArgs &a)
{
    return (int64_t)((a.M + T::BM - 1) / T::BM) * ((a.N + T::BN - 1) / T::BN);
}

template <typename T, bool BN_EPILOGUE, bool STREAM_OUT, bool PRODUCT_B = false, bool ACCUMULATE = false>
hipError_t launch_variant(const GemmArgs &a, hipStream_t stream)
{
    const auto kernel = &gemm_nt_f32_kernel<T, BN_EPILOGUE, STREAM_OUT, PRODUCT_B, ACCUMULATE>;
    if (T::LDS_BYTES > 65536) {
        // Dynamic LDS above 64 KiB must be allowed per kernel (gfx950 has
        // 160 KiB per CU); done once per kernel and device.
        static std::atomic<uint64_t> allowed_on{0};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
        if (!bit || !(allowed_on.load(std::memory_order_acquire) & bit)) {
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)T::LDS_BYTES);
            if (e != hipSuccess) return e;
            allowed_on.fetch_or(bit, std::memory_order_acq_rel);
        }
    }
    const dim3 grid((unsigned)tile_count<T>(a), a.batch);
    hipLaunchKernelGGL(kernel, grid, dim3(T::THREADS), T::LDS_BYTES, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_tile(const GemmArgs &a, hipStream_t stream)
{
    if (tile_count<T>(a) > 0x7FFFFFFF || a.batch > 65535) return hipErrorInvalidConfiguration;
    if (a.accumulate) {
        if (a.bn_mean || a.stream_out) return hipErrorInvalidValue;
        return launch_variant<T, false, false, false, true>(a, stream);
    }
    if (a.bn_mean) {
        if (a.stream_out) return launch_variant<T, true, true>(a, stream);
        return launch_variant<T, true, false>(a, stream);
    }
    if (a.stream_out) return launch_variant<T, false, true>(a, stream);
    return launch_variant<T, false, false>(a, stream);
}

}  // namespace

hipError_t launch_gemm_nt_f32(const GemmArgs &a, hipStream_t stream)
{
    if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
    if (a.K % 32 != 0) return hipErrorInvalidValue;
    if (tile_count<BigTile>(a) * a.batch >= kCUs) return launch_tile<BigTile>(a, stream);
    return launch_tile<SmallTile>(a, stream);
}

hipError_t launch_gemm_nt_f32_product(const GemmArgs &a, hipStream_t stream)
{
    if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
    if (a.K % 32 != 0 || a.split_k % 32 != 0 || a.split_k <= 0 || a.split_k >= a.K || !a.B2 || a.key_n <= 0 ||
        (int64_t)a.key_n * a.key_n < a.N || a.bn_mean)
        return hipErrorInvalidValue;
    if (tile_count<KeyTile>(a) > 0x7FFFFFFF || a.batch > 65535) return hipErrorInvalidConfiguration;
    return launch_variant<KeyTile, false, false, true>(a, stream);
}

}  // namespace pkm
