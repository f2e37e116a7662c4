// fp32-accurate GEMM on the matrix cores for the dense contractions of the
// lookup:
//   a1+a2  qhat = BN(x . Wq^T)         M = tokens, N = H*D,     K = D
//   a3     s_g  = qhat_g . C_g^T       M = tokens, N = n_keys,  K = D/2,
//                                      one batch entry g = 2h + p per half
// ("Product-Key Memory", code listing: the Linear + BatchNorm1d query and the
// two subkey products; §Factorising the key space for the split), and of the
// backward (dWq, dx) and the flat exact search.
//
// Both operands are K-contiguous (x rows, Wq rows, qhat rows, subkey rows),
// so C = A . B^T with no transposes.  Scores decide the winners, so the
// contraction must be as accurate as fp32.
//
// Engine: two-piece fp16 splitting with three products (the method of
// Ootomo and Yokota, "Recovering single precision accuracy from Tensor Cores
// while surpassing the FP32 theoretical peak performance", IJHPCA 2022,
// here without their scaling of the low piece, so that one fp32 accumulator
// takes all three products).  Every row of A and of B is first scaled by a
// power of two that brings its largest magnitude into [2^14, 2^15) (exact;
// computed per call by row_exponent_kernel), so fp16's range holds every
// row whatever its size.  Each scaled value is split while it is staged into
// LDS: hi = fp16(a), lo = fp16(a - hi), round to nearest; a - hi is exact and
// a = hi + lo + e with |e| <= 2^-22 |a| (+ 2^-25 absolute where lo falls
// below fp16's normal range, i.e. for entries below 2^-17 of the row's
// largest).  a.b is accumulated in fp32 from lo*hi, hi*lo and hi*hi, each
// exact in the accumulator; what is left out (lo*lo and the two e terms) is
// at most about 3 * 2^-22 |a||b| per product and random in sign.  The
// epilogue multiplies by 2^-(e_row + e_col).  v_mfma_f32_32x32x16_f16 runs
// at the bf16 rate, 16x the fp32 MFMA's, so the three products cost 3/16 of
// the fp32 instruction's time, with fewer accumulator roundings per k than
// that instruction.
//
// Tiling for CDNA4.  A workgroup owns a BM x BN tile of C; each of its
// WM x WN wave64s owns (BM/WM) x (BN/WN) as 32x32 MFMA blocks.  K advances
// 16 at a time (one MFMA step) through two LDS stages; chunk t + 1 is split
// and stored while chunk t is multiplied, and chunk t + 2 is loaded into
// registers.  An LDS row holds the two pieces' 16 fp16 each (64 bytes) plus
// 16 bytes of padding, so 16-byte accesses to consecutive rows fall on
// distinct banks.  Lane l of an MFMA step feeds row (or column) l % 32 with
// k = 8 (l / 32) .. 8 (l / 32) + 7 of the chunk (one ds_read_b128 per
// piece); A and B use the same k order, which is all a dot product needs.
// Staging uses the same lane -> (row, k) pattern, so its 16-byte LDS stores
// are conflict-free as well.
//   Large grids: 256x256 tiles, 8 waves of 64x128 (80 KiB of LDS, one
//   workgroup per CU, two waves per SIMD), run ping-pong: the second half
//   of the waves starts one barrier later, so on each SIMD one wave issues
//   MFMAs (at raised priority) while the other does the LDS and VALU work.
//   Small grids (fewer tiles than CUs at 256x256): 128x128, 4 waves of
//   64x64; plain or accumulated products with a workspace split K instead.
// Epilogue: BN (a1) and accumulated results are staged through LDS a few
// dozen rows at a time so each store instruction writes whole rows of C in
// 16-byte runs.  A result that the next kernel reads once (the subkey
// scores) is stored non-temporally, straight from the accumulators: it
// reaches HBM during this compute-bound kernel rather than being written
// back from the caches while the memory-bound gather runs.
//
// Operands split ahead of the call.  Weights that stay fixed between calls
// can be split once (launch_presplit: row exponents, then the pieces in the
// order a staging lane copies them), and so can the tokens (launch_exp_split:
// exponents and pieces in one pass); a tile then copies pieces instead of
// splitting, with the same bits.  With both operands split (the folded
// lookup: x against the folded projection, batch-norm and subkeys, summed
// in fp64 by fold_kernel) the staging is a pure copy and two chunks ride in
// registers ahead of the one being staged.
//
// Flat exact search (the comparator for the product search of
// §Factorising the key space: every one of the n^2 concatenated keys
// scored by one full-length dot product).  The B operand is the virtual
// key matrix: row j = (a, c) is [C0[a]; C1[c]].  The subkey rows are split
// into their fp16 pieces once per call (split_rows_kernel, each row with
// its own power of two) in the order a staging lane copies them, so a tile
// stages its 256 virtual rows by copying pieces.  The two halves of K carry
// different key-row exponents: after the first half the accumulators of
// each key are multiplied by the power of two between them (exact) and the
// second half adds on in the same registers.  M is a few dozen tokens:
// 64 x 256 tiles of 4 waves of 64 x 64 (32 x 256, waves of 32 x 64, for at
// most 32 tokens), so each staged key row serves up to 64 tokens.  The
// epilogue can record each row's largest score per group of 64 keys, from
// which the top-k derives a threshold.
#include "pkm_internal.h"
#include "wave_ops.h"

#include <atomic>

namespace pkm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float fx4 __attribute__((ext_vector_type(4)));
typedef float fx2 __attribute__((ext_vector_type(2)));
typedef _Float16 hx2 __attribute__((ext_vector_type(2)));
typedef _Float16 hx8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef int32_t i4 __attribute__((ext_vector_type(4)));

constexpr int kCUs = 256;     // MI355X compute units
constexpr int kXcds = 8;      // its accelerator dies, each with its own L2
constexpr int kBK = 16;       // k per chunk: one v_mfma_f32_32x32x16_f16 step
constexpr int kPieces = 2;    // fp16 pieces per fp32 operand
constexpr int kPieceDw = 8;   // dwords per piece in an LDS row (16 fp16)
constexpr int kRowDw = kPieces * kPieceDw + 4;  // + 16 bytes of padding
constexpr int kRowTop = 14;   // a row's largest magnitude is scaled into [2^14, 2^15)

template <int BM_, int BN_, int WM_, int WN_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = 2;
    static constexpr int WAVES = WM * WN, THREADS = 64 * WAVES;
    static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;  // 32x32 blocks per wave
    // Operand rows are staged in groups of 32: lane l of a wave moves row
    // l % 32 of its group, k = 8 (l / 32) .. + 7 of the chunk (the same
    // row/k assignment as an MFMA fragment read).  Group g of a chunk is
    // moved by wave g % WAVES.
    static constexpr int GROUPS = (BM + BN) / 32;
    static constexpr int UNITS = (GROUPS + WAVES - 1) / WAVES;  // groups per wave
    static constexpr size_t LDS_BYTES = (size_t)STAGES * (BM + BN) * kRowDw * sizeof(uint32_t);
    // Ping-pong when two waves share each SIMD: the second half of the waves
    // runs one phase behind the first, so on every SIMD one wave issues MFMAs
    // while the other reads fragments and splits, stores and loads chunks.
    static constexpr bool PING_PONG = WAVES == 8;
    // rows of C staged through LDS per epilogue pass: 64, or 32 where 64
    // rows and the exponents would not fit in the stages' LDS
    static constexpr int EPI_ROWS =
        BM < 64 ? BM : ((size_t)(64 * (BN + 8) + BM + BN) * sizeof(float) <= LDS_BYTES ? 64 : 32);
    static_assert(BM % 32 == 0 && BN % 32 == 0 && BM % EPI_ROWS == 0, "tile shape");
    // epilogue LDS: the staged rows, then the tile's row and column exponents
    static constexpr int EX_OFF = EPI_ROWS * (BN + 8);
    static_assert((size_t)(EX_OFF + BM + BN) * sizeof(float) <= LDS_BYTES, "epilogue staging fits");
    static_assert(EPI_ROWS * BN / 4 % THREADS == 0 && THREADS % (BN / 4) == 0, "epilogue work divides");
};

// The power of two that scales a row whose largest magnitude is m into
// [2^14, 2^15); 0 for m = 0 or not finite.
__device__ __forceinline__ int row_exponent(float m)
{
    int ex = 0;
    if (m > 0.0f && m <= 3.402823466e38f) {
        int p;
        (void)__builtin_frexpf(m, &p);  // m = f 2^p, f in [0.5, 1)
        ex = kRowTop + 1 - p;
    }
    return ex;
}

using BigTile = Tile<256, 256, 4, 2>;
using SmallTile = Tile<128, 128, 2, 2>;
using KeyTile = Tile<32, 256, 1, 4>;    // up to 32 rows of A
using KeyTile64 = Tile<64, 256, 1, 4>;  // more: each staged key row serves 64

// Eight consecutive k-values of one row, scaled by 2^ex and split into their
// hi and lo fp16 pieces (a - hi is exact: one mixed fp32/fp16 FMA per value
// with `one` a 1.0 the compiler cannot fold away).
__device__ __forceinline__ void split8(const fx4 (&v)[2], int ex, float one, u4 &hi, u4 &lo)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const fx2 e = {__builtin_ldexpf(v[q >> 1][2 * (q & 1)], ex), __builtin_ldexpf(v[q >> 1][2 * (q & 1) + 1], ex)};
        const hx2 h = __builtin_convertvector(e, hx2);
        const fx2 r = {__builtin_fmaf(e[0], one, -(float)h[0]), __builtin_fmaf(e[1], one, -(float)h[1])};
        hi[q] = __builtin_bit_cast(uint32_t, h);
        lo[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, hx2));
    }
}

// The staging work of one thread: UNITS groups; for each, the global source
// of its 8 k-values, the row's exponent, and its LDS destination in stage 0
// (dwords) with the stride between stages.  Product-key B rows come already
// split (split_rows_kernel): a B unit copies its lane's two 16-byte pieces
// of each chunk, from the first subkey set's row (src) and from chunk kch
// on from the second set's (src2), both pointing at pieces.  SPLIT >= 1: a
// plain B operand split ahead of the call (weights split once, when they are
// prepared), copied the same way from src alone; SPLIT == 2: the A operand
// as well (rows split by the pass that takes their exponents).
template <typename T, bool PRODUCT_B, int SPLIT = 0>
struct Stager {
    static constexpr bool PIECES_B = PRODUCT_B || SPLIT >= 1;
    static constexpr bool PIECES_A = SPLIT == 2;
    // When the A rows and the B rows each fill whole rounds of the waves'
    // groups (both 256x256 and 128x128 tiles), unit u of every wave is an
    // A group for u < BM / 32 / WAVES and a B group after, and every unit
    // is in range: known at compile time, no flags in registers.
    static constexpr bool STATIC_UNITS = (T::BM / 32) % T::WAVES == 0 && (T::BN / 32) % T::WAVES == 0;
    const float *src[T::UNITS];
    const float *src2[PRODUCT_B ? T::UNITS : 1];
    bool is_b[(PIECES_A || PIECES_B) && !STATIC_UNITS ? T::UNITS : 1];
    int kch;
    int lds[T::UNITS], stage_stride[T::UNITS], ex[T::UNITS];
    bool valid[STATIC_UNITS ? 1 : T::UNITS];
    fx4 v[T::UNITS][2];
    // a second chunk in flight, where the contraction fetches two ahead
    fx4 v2[SPLIT == 2 && T::PING_PONG ? T::UNITS : 1][2];

    __device__ __forceinline__ bool b_unit(int u) const
    {
        if constexpr (STATIC_UNITS) return u >= T::BM / 32 / T::WAVES;
        else return is_b[u];
    }
    __device__ __forceinline__ bool in_range(int u) const
    {
        if constexpr (STATIC_UNITS) return true;
        else return valid[u];
    }
    // unit u copies pieces (its operand was split beforehand)
    __device__ __forceinline__ bool copies(int u) const
    {
        if constexpr (PIECES_A && PIECES_B) return true;
        else if constexpr (PIECES_B) return b_unit(u);
        else if constexpr (PIECES_A) return !b_unit(u);
        else return false;
    }

    __device__ __forceinline__ void load(int kt) { load_into(v, kt); }
    __device__ __forceinline__ void store(uint32_t *smem, int s) const { store_from(v, smem, s); }

    template <typename Buf>
    __device__ __forceinline__ void load_into(Buf &v, int kt)
    {
#pragma unroll
        for (int u = 0; u < T::UNITS; ++u) {
            if (!in_range(u)) continue;
            if constexpr (PIECES_A || PIECES_B) {
                if (copies(u)) {
                    const u4 *q;
                    if constexpr (PRODUCT_B)
                        q = kt < kch ? reinterpret_cast<const u4 *>(src[u]) + (int64_t)kt * 128
                                     : reinterpret_cast<const u4 *>(src2[u]) + (int64_t)(kt - kch) * 128;
                    else
                        q = reinterpret_cast<const u4 *>(src[u]) + (int64_t)kt * 128;
                    v[u][0] = __builtin_bit_cast(fx4, q[0]);
                    v[u][1] = __builtin_bit_cast(fx4, q[64]);
                    continue;
                }
            }
            const float *q = src[u] + kt * kBK;
            v[u][0] = *reinterpret_cast<const fx4 *>(q);
            v[u][1] = *reinterpret_cast<const fx4 *>(q + 4);
        }
    }

    // Scale the 8 values by the row's power of two and split them into
    // their two fp16 pieces; each piece's 16 bytes go to that piece's part of
    // the LDS row.
    template <typename Buf>
    __device__ __forceinline__ void store_from(const Buf &v, uint32_t *smem, int s) const
    {
        float one = 1.0f;
        asm volatile("" : "+v"(one));
#pragma unroll
        for (int u = 0; u < T::UNITS; ++u) {
            if (!in_range(u)) continue;
            if constexpr (PIECES_A || PIECES_B) {
                if (copies(u)) {  // pieces as loaded
                    uint32_t *dst = smem + lds[u] + s * stage_stride[u];
#pragma unroll
                    for (int p = 0; p < kPieces; ++p)
                        *reinterpret_cast<u4 *>(dst + p * kPieceDw) = __builtin_bit_cast(u4, v[u][p]);
                    continue;
                }
            }
            u4 w[kPieces];
            split8(v[u], ex[u], one, w[0], w[1]);
            uint32_t *dst = smem + lds[u] + s * stage_stride[u];
#pragma unroll
            for (int p = 0; p < kPieces; ++p) *reinterpret_cast<u4 *>(dst + p * kPieceDw) = w[p];
        }
    }
};

template <typename T>
__device__ __forceinline__ void read_frags(hx8 (&af)[T::TM][kPieces], hx8 (&bf)[T::TN][kPieces], const uint32_t *as,
                                           const uint32_t *bs, int wm, int wn, int il, int kk)
{
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int p = 0; p < kPieces; ++p)
            af[i][p] = __builtin_bit_cast(hx8, *reinterpret_cast<const u4 *>(
                                                   &as[(wm * T::TM * 32 + i * 32 + il) * kRowDw + p * kPieceDw + kk * 4]));
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
        for (int p = 0; p < kPieces; ++p)
            bf[j][p] = __builtin_bit_cast(hx8, *reinterpret_cast<const u4 *>(
                                                   &bs[(wn * T::TN * 32 + j * 32 + il) * kRowDw + p * kPieceDw + kk * 4]));
}

// The three products of one chunk, the small ones first: (lo,hi) (hi,lo)
// (hi,hi); piece 0 is hi, piece 1 lo.
template <typename T>
__device__ __forceinline__ void mfma_frags(floatx16 (&acc)[T::TM][T::TN], const hx8 (&af)[T::TM][kPieces],
                                           const hx8 (&bf)[T::TN][kPieces])
{
    constexpr int pa[3] = {1, 0, 0};
    constexpr int pb[3] = {0, 1, 0};
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i][pa[t]], bf[j][pb[t]], acc[i][j], 0, 0, 0);
}

// One BM x BN tile (tm, tn) of batch entry g and K range z.  KEEP_PRE: the
// BN epilogue also stores the values before BN (a.C_pre).
// SPLIT >= 1: B's rows come split into fp16 pieces (a.b_presplit, scaled by
// a.b_exp_given), and the tile copies them; SPLIT == 2: A's rows as well
// (a.a_presplit, scaled by the exponents in the row-exponent workspace).
template <typename T, bool BN_EPILOGUE, bool STREAM_OUT, bool PRODUCT_B, bool ACCUMULATE, bool KEEP_PRE = false,
          int SPLIT = 0>
__device__ __forceinline__ void gemm_tile(const GemmArgs &a, int tm, int tn, int g, int z, uint32_t *smem)
{
    static_assert(!KEEP_PRE || (BN_EPILOGUE && !STREAM_OUT), "values before BN: the staged BN epilogue");
    static_assert(!PRODUCT_B || (!STREAM_OUT && !BN_EPILOGUE && !ACCUMULATE), "product-key B: plain staged epilogue");
    static_assert(!(PRODUCT_B && SPLIT), "one form of pre-split B");
    constexpr bool SPLIT_B = SPLIT >= 1;
    uint32_t *As = smem;
    uint32_t *Bs = smem + T::STAGES * T::BM * kRowDw;
    // split-K: this block's range of K (the operands are K-contiguous)
    const int kbeg = a.k_chunk ? z * a.k_chunk : 0;
    const int klen = a.k_chunk ? min(a.k_chunk, a.K - kbeg) : a.K;
    const float *A = a.A + (int64_t)g * a.strideA + kbeg;
    const float *Bmat = a.B + (int64_t)g * a.strideB + kbeg;
    float *C = a.C + (int64_t)g * a.strideC + (int64_t)z * a.batch * a.strideC;
    const int32_t *a_exp = a.a_rowmax ? nullptr : a.a_exp + (int64_t)g * a.M;
    // exponent of A row m (its maxima given, or computed by the pre-pass)
    const auto row_exp = [&](int m) {
        return a.a_rowmax ? row_exponent(__uint_as_float(a.a_rowmax[(int64_t)m * a.a_rowmax_ld + g])) : a_exp[m];
    };
    const int32_t *b_exp = a.b_exp + (int64_t)g * (PRODUCT_B ? a.key_n : a.N);
    const int32_t *b2_exp = PRODUCT_B ? a.b2_exp + (int64_t)g * a.key_n : nullptr;
    const int m0 = tm * T::BM, n0 = tn * T::BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / T::WN, wn = wave % T::WN;
    const int il = lane & 31;  // row (A) / column (B) inside a 32x32 block
    const int kk = lane >> 5;  // which half of the chunk's k this lane feeds

    // Rows past the matrix edge re-read the last row; their results are
    // never stored.
    Stager<T, PRODUCT_B, SPLIT> st;
    st.kch = a.split_k / kBK;
    // pre-split plain B: this batch entry's rows, from this K range's first
    // chunk (pieces of rows past N are zero)
    const int kt_all = a.K / kBK;
    const u4 *bsplit = SPLIT_B ? reinterpret_cast<const u4 *>(a.b_presplit) +
                                     ((int64_t)g * ((a.N + 31) / 32) * kt_all + kbeg / kBK) * 128
                               : nullptr;
    const u4 *asplit = SPLIT == 2 ? reinterpret_cast<const u4 *>(a.a_presplit) +
                                        ((int64_t)g * ((a.M + 31) / 32) * kt_all + kbeg / kBK) * 128
                                  : nullptr;
    // product-key B: the split rows of this batch entry's two subkey sets
    const int kgroups = (a.key_n + 31) / 32;
    const u4 *set0 =
        PRODUCT_B ? reinterpret_cast<const u4 *>(a.b_split) + (int64_t)g * 2 * kgroups * st.kch * 128 : nullptr;
    const u4 *set1 = PRODUCT_B ? set0 + (int64_t)kgroups * st.kch * 128 : nullptr;
#pragma unroll
    for (int u = 0; u < T::UNITS; ++u) {
        const int grp = wave + T::WAVES * u;
        if constexpr (!decltype(st)::STATIC_UNITS) st.valid[u] = grp < T::GROUPS;
        const int r = min(grp, T::GROUPS - 1) * 32 + il;  // row of the A tile, then of the B tile
        if constexpr ((PRODUCT_B || SPLIT) && !decltype(st)::STATIC_UNITS) st.is_b[u] = r >= T::BM;
        if (decltype(st)::STATIC_UNITS ? !st.b_unit(u) : r < T::BM) {
            const int m = min(m0 + r, a.M - 1);
            if constexpr (SPLIT == 2)  // lane (kk, m % 32) of row m's group
                st.src[u] = reinterpret_cast<const float *>(asplit + (int64_t)(m / 32) * kt_all * 128 + kk * 32 + m % 32);
            else
                st.src[u] = A + (int64_t)m * a.lda + kk * 8;
            if constexpr (PRODUCT_B) st.src2[u] = nullptr;
            st.ex[u] = row_exp(m);
            st.lds[u] = r * kRowDw + kk * 4;
            st.stage_stride[u] = T::BM * kRowDw;
        } else {
            const int j = min(n0 + r - T::BM, a.N - 1);
            if constexpr (PRODUCT_B) {
                // lane (kk, row % 32) of the subkey row's group, chunk 0
                const int ka = j / a.key_n, kc = j - ka * a.key_n;
                st.src[u] = reinterpret_cast<const float *>(set0 + (int64_t)(ka / 32) * st.kch * 128 + kk * 32 + ka % 32);
                st.src2[u] = reinterpret_cast<const float *>(set1 + (int64_t)(kc / 32) * st.kch * 128 + kk * 32 + kc % 32);
                st.ex[u] = 0;
            } else if constexpr (SPLIT_B) {
                // lane (kk, j % 32) of row j's group
                st.src[u] = reinterpret_cast<const float *>(bsplit + (int64_t)(j / 32) * kt_all * 128 + kk * 32 + j % 32);
                st.ex[u] = 0;
            } else {
                st.src[u] = Bmat + (int64_t)j * a.ldb + kk * 8;
                st.ex[u] = b_exp[j];
            }
            st.lds[u] = (T::STAGES * T::BM + r - T::BM) * kRowDw + kk * 4;
            st.stage_stride[u] = T::BN * kRowDw;
        }
    }
    // exponent of output column n (its B row's; product-key columns are
    // scaled in the epilogue's combination below instead)
    const auto col_exp = [&](int n) { return PRODUCT_B ? 0 : b_exp[n]; };

    floatx16 acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // Both operands split beforehand (pure copies): two chunks ride in
    // registers ahead of the one being staged, so a fetch has two chunks'
    // time to arrive (the register budget allows the second buffer here).
    constexpr bool DEEP = SPLIT == 2 && T::PING_PONG;
    const int KT = klen / kBK;
    st.load(0);
    st.store(smem, 0);
    if constexpr (DEEP) {
        // unconditional fetches (past the end: the last chunk again), in a
        // fixed order, so the count of loads behind each buffer's is the
        // same on every path and a stage waits only for its own chunk
        st.load(min(1, KT - 1));
        asm volatile("" ::: "memory");
        st.load_into(st.v2, min(2, KT - 1));
    } else if (KT > 1) {
        st.load(1);
    }
    __syncthreads();
    const bool late = T::PING_PONG && wave >= T::WAVES / 2;
    if (late) __builtin_amdgcn_s_barrier();
    const auto run = [&](auto &accx, int kt0, int kt1) {
        for (int kt = kt0; kt < kt1; ++kt) {
            const int s = kt & 1;
            hx8 af[T::TM][kPieces], bf[T::TN][kPieces];
            read_frags<T>(af, bf, As + s * T::BM * kRowDw, Bs + s * T::BN * kRowDw, wm, wn, il, kk);
            // chunk kt + 1 into the other stage (last read in chunk kt - 1,
            // before the barrier that closed it), then fetch chunk kt + 2
            if (kt + 1 < KT) {
                st.store(smem, s ^ 1);
                if (kt + 2 < KT) st.load(kt + 2);
            }
            if constexpr (T::PING_PONG) {
                __syncthreads();
                __builtin_amdgcn_s_setprio(1);
                mfma_frags<T>(accx, af, bf);
                __builtin_amdgcn_s_setprio(0);
                __syncthreads();
            } else {
                mfma_frags<T>(accx, af, bf);
                __syncthreads();
            }
        }
    };
    if constexpr (DEEP) {
        // chunk kt + 1 is staged from v (kt even) or v2 (kt odd), which then
        // fetches chunk kt + 3
        // (the last step's store goes to a stage no one reads again, and
        // fetches past the end re-read the last chunk)
        const auto step = [&](int kt, auto &buf) {
            const int s = kt & 1;
            hx8 af[T::TM][kPieces], bf[T::TN][kPieces];
            read_frags<T>(af, bf, As + s * T::BM * kRowDw, Bs + s * T::BN * kRowDw, wm, wn, il, kk);
            st.store_from(buf, smem, s ^ 1);
            st.load_into(buf, min(kt + 3, KT - 1));
            __syncthreads();
            __builtin_amdgcn_s_setprio(1);
            mfma_frags<T>(acc, af, bf);
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();
        };
        // K is a multiple of 32, so the chunks come in pairs (and the loop
        // body is straight-line code)
        for (int kt = 0; kt < KT; kt += 2) {
            step(kt, st.v);
            step(kt + 1, st.v2);
        }
    } else if constexpr (PRODUCT_B) {
        // Product-key B: the two halves of K carry their own key-row
        // exponents e0 (first subkey) and e1 (second).  After the first
        // half the sums of column n are moved from scale 2^e0 to 2^e1
        // (exact: a power of two), then the second half adds on in the same
        // accumulators.  32x32 layout: lane l holds column l % 32 of each
        // block.
        run(acc, 0, st.kch);
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int col = min(n0 + wn * T::TN * 32 + j * 32 + il, a.N - 1);
            const int ka = col / a.key_n;
            const int shift = b2_exp[col - ka * a.key_n] - b_exp[ka];
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_ldexpf(acc[i][j][v], shift);
        }
        run(acc, st.kch, KT);
    } else {
        run(acc, 0, KT);
    }
    if (T::PING_PONG && !late) __builtin_amdgcn_s_barrier();

    // The exponents of the tile's rows and columns, once, into LDS (every
    // wave is past its last fragment read).
    int32_t *ex_lds = reinterpret_cast<int32_t *>(smem) + T::EX_OFF;
    for (int t = tid; t < T::BM + T::BN; t += T::THREADS)
        ex_lds[t] = t < T::BM ? row_exp(min(m0 + t, a.M - 1)) : col_exp(min(n0 + t - T::BM, a.N - 1));
    __syncthreads();
    if constexpr (PRODUCT_B) {
        // to true scale, 2^-(e_row + e1) (32x32 layout: register v of lane l
        // is row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32 of its
        // block); the staged epilogue below then scales nothing
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int col = min(n0 + wn * T::TN * 32 + j * 32 + il, a.N - 1);
            const int ka = col / a.key_n;
            const int e1 = b2_exp[col - ka * a.key_n];
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const i4 er = *reinterpret_cast<const i4 *>(&ex_lds[wm * T::TM * 32 + i * 32 + v4 * 8 + kk * 4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i][j][v4 * 4 + e] = __builtin_ldexpf(acc[i][j][v4 * 4 + e], -(er[e] + e1));
                }
        }
    }

    if constexpr (STREAM_OUT) {
        // A streamed result (read once by the next kernel) is stored straight
        // from the accumulators, non-temporally.  32x32 accumulator layout:
        // register v of lane l holds row 8*(v/4) + 4*(l/32) + v%4, column
        // l%32 of its block.
        // The columns' parameters are all loaded first and made ready once:
        // vmcnt counts stores as well as loads, so a wait for a load issued
        // after some stores (or one the compiler cannot place exactly, behind
        // the per-row branches) would also wait for those stores to land.
        int ecol[T::TN];
        float mean[T::TN], mul[T::TN], beta[T::TN], bias[T::TN];
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int col = min(n0 + wn * T::TN * 32 + j * 32 + il, a.N - 1);
            ecol[j] = ex_lds[T::BM + col - n0];
            mean[j] = 0.0f, mul[j] = 1.0f, beta[j] = 0.0f;
            if (BN_EPILOGUE) {
                mean[j] = a.bn_mean[col];
                mul[j] = a.bn_gamma[col] / sqrtf(a.bn_var[col] + a.bn_eps);
                beta[j] = a.bn_beta[col];
            }
            bias[j] = a.col_bias ? a.col_bias[(int64_t)g * a.N + col] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < T::TN; ++j) asm volatile("" : "+v"(mean[j]), "+v"(mul[j]), "+v"(beta[j]), "+v"(bias[j]));
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int col = n0 + wn * T::TN * 32 + j * 32 + il;
            if (col >= a.N) continue;
#pragma unroll
            for (int i = 0; i < T::TM; ++i) {
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    // rows 8 v4 + 4 kk .. + 3 of the block: four row exponents
                    const int rb = m0 + wm * T::TM * 32 + i * 32 + v4 * 8 + kk * 4;
                    const i4 er = *reinterpret_cast<const i4 *>(&ex_lds[rb - m0]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = rb + e;
                        if (row < a.M) {
                            float c = __builtin_ldexpf(acc[i][j][v4 * 4 + e], -(er[e] + ecol[j]));
                            if (BN_EPILOGUE) c = (c - mean[j]) * mul[j] + beta[j];
                            if (a.col_bias) c += bias[j];
                            __builtin_nontemporal_store(c, &C[(int64_t)row * a.ldc + col]);
                        }
                    }
                }
            }
        }
        return;
    }
    // Otherwise the epilogue goes through LDS (free after the last chunk's
    // barrier): PR rows of the tile at a time, the waves holding them write
    // their accumulators row-major, then every thread stores whole 16-byte
    // runs of columns, so each store instruction covers contiguous kilobytes
    // of C.
    constexpr int CS = T::BN + 8;  // floats per staged row (rows 4 apart on other banks)
    constexpr int PR = T::EPI_ROWS;
    float *stage = reinterpret_cast<float *>(smem);
    const bool vec = a.ldc % 4 == 0 && (reinterpret_cast<uintptr_t>(C) & 15) == 0;
    // every pass gives a thread the same four columns: c0 .. c0 + 3
    const int c0 = (tid % (T::BN / 4)) * 4;
    const int ncol = min(4, a.N - (n0 + c0));
    fx4 bn_mean = {0.0f, 0.0f, 0.0f, 0.0f}, bn_mul = {1.0f, 1.0f, 1.0f, 1.0f}, bn_beta = {0.0f, 0.0f, 0.0f, 0.0f};
    i4 ecol = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e < ncol) {
            const int cc = n0 + c0 + e;
            ecol[e] = ex_lds[T::BM + c0 + e];
            if (BN_EPILOGUE) {
                bn_mean[e] = a.bn_mean[cc];
                bn_mul[e] = a.bn_gamma[cc] / sqrtf(a.bn_var[cc] + a.bn_eps);
                bn_beta[e] = a.bn_beta[cc];
            }
        }
    }
#pragma unroll
    for (int pass = 0; pass < T::BM / PR; ++pass) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const int rb = wm * T::TM * 32 + i * 32 - pass * PR;  // block's first row in the pass
            if (rb < 0 || rb >= PR) continue;
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    stage[(rb + (v >> 2) * 8 + kk * 4 + (v & 3)) * CS + wn * T::TN * 32 + j * 32 + il] = acc[i][j][v];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < PR * T::BN / 4 / T::THREADS; ++q) {
            const int f = tid + T::THREADS * q;
            const int r = f / (T::BN / 4);
            const int row = m0 + pass * PR + r, col = n0 + c0;
            const bool live = row < a.M && ncol > 0;
            fx4 x = *reinterpret_cast<const fx4 *>(&stage[r * CS + c0]);
            const int erow = ex_lds[pass * PR + r];
            if constexpr (!PRODUCT_B)
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = __builtin_ldexpf(x[e], -(erow + ecol[e]));
            if constexpr (BN_EPILOGUE) {
                if (KEEP_PRE && live) {  // the values before BN as well
                    float *pre = &a.C_pre[(int64_t)g * a.strideC + (int64_t)row * a.ldc + col];
                    if (vec && ncol == 4) *reinterpret_cast<fx4 *>(pre) = x;
                    else
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (e < ncol) pre[e] = x[e];
                }
                x = (x - bn_mean) * bn_mul + bn_beta;
            }
            if constexpr (PRODUCT_B) {
                static_assert(T::BN % 64 == 0, "a group of 64 columns is 16 lanes of one row");
                if (a.group_max) {
                    uint32_t mk = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (live && e < ncol) mk = max(mk, order_key(x[e]));
                    mk = max(mk, xor_lane<1>(mk));
                    mk = max(mk, xor_lane<2>(mk));
                    mk = max(mk, xor_lane<4>(mk));
                    mk = max(mk, xor_lane<8>(mk));
                    if (live && lane % 16 == 0)
                        a.group_max[(int64_t)row * a.group_ld + (int64_t)g * a.group_stride + col / 64] =
                            key_score(mk);
                }
            }
            if (a.row_seg_max) {
                // the row's largest |C| per segment: lanes of one row hold
                // consecutive columns, 4 each; a segment spans whole groups
                // of 8 lanes, or all of the row's lanes
                float m4 = 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (live && e < ncol) m4 = fmaxf(m4, fabsf(x[e]));
                m4 = fmaxf(m4, __uint_as_float(xor_lane<1>(__float_as_uint(m4))));
                m4 = fmaxf(m4, __uint_as_float(xor_lane<2>(__float_as_uint(m4))));
                m4 = fmaxf(m4, __uint_as_float(xor_lane<4>(__float_as_uint(m4))));
                constexpr int RL = T::BN / 4 < 64 ? T::BN / 4 : 64;  // lanes of one row
                int group = 8;
                if (a.seg_cols % (4 * RL) == 0) {
                    if constexpr (RL > 8) m4 = fmaxf(m4, __uint_as_float(xor_lane<8>(__float_as_uint(m4))));
                    if constexpr (RL > 16) m4 = fmaxf(m4, __uint_as_float(xor_lane<16>(__float_as_uint(m4))));
                    if constexpr (RL > 32) m4 = fmaxf(m4, __uint_as_float(xor_lane<32>(__float_as_uint(m4))));
                    group = RL;
                }
                if (live && lane % group == 0)
                    atomicMax(&a.row_seg_max[(int64_t)row * (a.N / a.seg_cols) + col / a.seg_cols],
                              __float_as_uint(m4));
            }
            if (live) {
                float *dst = &C[(int64_t)row * a.ldc + col];
                if (vec && ncol == 4) {
                    if (ACCUMULATE) x += *reinterpret_cast<const fx4 *>(dst);
                    // the flat search's key scores are read back only where
                    // a group can hold a winner: stream them past the caches
                    if constexpr (PRODUCT_B) __builtin_nontemporal_store(x, reinterpret_cast<fx4 *>(dst));
                    else *reinterpret_cast<fx4 *>(dst) = x;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (e >= ncol) break;
                        float y = x[e];
                        if (ACCUMULATE) y += dst[e];
                        dst[e] = y;
                    }
                }
            }
        }
        if (pass + 1 < T::BM / PR) __syncthreads();
    }
}

// PERSIST: a grid of at most one workgroup per CU walks all tiles (batch
// entry major), a barrier between tiles; otherwise one tile per workgroup,
// grid (tiles, batch, K ranges).
template <typename T, bool BN_EPILOGUE, bool STREAM_OUT, bool PRODUCT_B = false, bool ACCUMULATE = false,
          bool PERSIST = false, bool KEEP_PRE = false, int SPLIT = 0>
__global__ __launch_bounds__(T::THREADS) void gemm_nt_f32_kernel(GemmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
    const int tiles_n = (a.N + T::BN - 1) / T::BN;
    if constexpr (PERSIST) {
        // Workgroups are dealt to the XCDs in turn (workgroup w on XCD w %
        // kXcds, each XCD with its own L2).  Each XCD takes whole rows of
        // tiles -- (batch entry, row tile) pairs r with r % kXcds its own --
        // so a block of A rows is fetched into one L2 for all its column
        // tiles instead of into every XCD's: each XCD streams all of B and
        // an eighth of A.  That is the better split while B has no more rows
        // than A (per batch entry); with a wider B (the folded lookup's
        // 2H n keys against a few thousand tokens) and where whole rows
        // would leave XCDs short of work, the tiles go round-robin instead,
        // which deals the column tiles to the XCDs in turn (with a multiple
        // of 8 column tiles each XCD keeps its eighth of B in its L2 and
        // streams A).  Every tile is computed once, the same way, whichever
        // workgroup takes it.
        const int tiles_m = (a.M + T::BM - 1) / T::BM;
        const int rows = tiles_m * a.batch;
        const int64_t total = (int64_t)rows * tiles_n;
        const int xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;
        const int64_t rows_rounds = ((int64_t)((rows + kXcds - 1) / kXcds) * tiles_n + per_xcd - 1) / per_xcd;
        const bool by_rows = a.N <= a.M && rows_rounds <= (total + gridDim.x - 1) / gridDim.x;
        const int64_t count = by_rows ? (int64_t)((rows - xcd + kXcds - 1) / kXcds) * tiles_n : total;
        const int64_t step = by_rows ? per_xcd : gridDim.x;
        for (int64_t e = by_rows ? blockIdx.x / kXcds : blockIdx.x; e < count; e += step) {
            const int j = (int)(e / tiles_n), tn = (int)(e - (int64_t)j * tiles_n);
            const int r = by_rows ? xcd + kXcds * j : j;  // (batch entry, row tile) pair
            const int g = r / tiles_m;
            gemm_tile<T, BN_EPILOGUE, STREAM_OUT, PRODUCT_B, ACCUMULATE, KEEP_PRE, SPLIT>(a, r - g * tiles_m, tn, g, 0,
                                                                                          smem);
            __syncthreads();
        }
    } else {
        gemm_tile<T, BN_EPILOGUE, STREAM_OUT, PRODUCT_B, ACCUMULATE, KEEP_PRE, SPLIT>(
            a, blockIdx.x / tiles_n, blockIdx.x % tiles_n, blockIdx.y, blockIdx.z, smem);
    }
}

// Row exponents: for each row of a K-long fp32 matrix, the power of two that
// scales the row's largest magnitude into [2^14, 2^15); 0 for a row of
// zeros (or a non-finite largest magnitude, which no scaling helps).  One
// launch covers up to three such matrices (A, B and a product key's second
// half); a wave takes kExpRows consecutive rows of one of them, every load
// issued before the maxima are formed.
struct ExpJob {
    const float *base;
    int64_t stride, ld;
    uint32_t rows, per_batch;  // rows = per_batch * batch < 2^31
    int K;
    int32_t *out;
    // row maxima given instead (float bits): row m of batch entry g has
    // maxbits[m * ld + g]
    const uint32_t *maxbits;
};
struct ExpJobs {
    ExpJob job[3];
    int64_t first_wave[4];  // wave index where each job starts; [3] = rows' total
    uint32_t *zero_ptr;     // then zero_n uint32s to clear, 1024 per wave
    int64_t zero_n;
};
constexpr int kExpRows = 4;

__device__ __forceinline__ float wave_max(float x)
{
    x = fmaxf(x, __uint_as_float(xor_lane<1>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(xor_lane<2>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(xor_lane<4>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(xor_lane<8>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(xor_lane<16>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(xor_lane<32>(__float_as_uint(x))));
    return x;
}

__global__ __launch_bounds__(256) void row_exponent_kernel(ExpJobs jobs)
{
    const int lane = threadIdx.x & 63;
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wv >= jobs.first_wave[3]) {
        const int64_t z0 = (wv - jobs.first_wave[3]) * 1024 + lane * 16;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (z0 + i < jobs.zero_n) jobs.zero_ptr[z0 + i] = 0u;
        return;
    }
    const int j = wv >= jobs.first_wave[2] ? 2 : wv >= jobs.first_wave[1] ? 1 : 0;
    const ExpJob &jb = jobs.job[j];
    const uint32_t r0 = (uint32_t)(wv - jobs.first_wave[j]) * kExpRows;
    if (jb.maxbits) {  // one row per lane
        const uint32_t r = (uint32_t)(wv - jobs.first_wave[j]) * 64 + lane;
        if (r < jb.rows) {
            const uint32_t g = r / jb.per_batch;
            jb.out[r] = row_exponent(__uint_as_float(jb.maxbits[(int64_t)(r - g * jb.per_batch) * jb.ld + g]));
        }
        return;
    }
    const float *row[kExpRows];
#pragma unroll
    for (int i = 0; i < kExpRows; ++i) {
        const uint32_t r = min(r0 + i, jb.rows - 1), g = r / jb.per_batch;
        row[i] = jb.base + (int64_t)g * jb.stride + (int64_t)(r - g * jb.per_batch) * jb.ld;
    }
    float mx[kExpRows];
#pragma unroll
    for (int i = 0; i < kExpRows; ++i) mx[i] = 0.0f;
    const bool vec = jb.K % 4 == 0 && jb.ld % 4 == 0 && jb.stride % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(jb.base) & 15) == 0;
    if (vec) {
        // sixteen float4 loads in flight per lane
        for (int c0 = 4 * lane; c0 < jb.K; c0 += 1024) {
            fx4 v[kExpRows][4];
#pragma unroll
            for (int i = 0; i < kExpRows; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    v[i][q] = c0 + 256 * q < jb.K ? *reinterpret_cast<const fx4 *>(row[i] + c0 + 256 * q)
                                                  : fx4{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < kExpRows; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    mx[i] = fmaxf(fmaxf(mx[i], fmaxf(fabsf(v[i][q][0]), fabsf(v[i][q][1]))),
                                  fmaxf(fabsf(v[i][q][2]), fabsf(v[i][q][3])));
        }
    } else {
#pragma unroll
        for (int i = 0; i < kExpRows; ++i)
            for (int c = lane; c < jb.K; c += 64) mx[i] = fmaxf(mx[i], fabsf(row[i][c]));
    }
#pragma unroll
    for (int i = 0; i < kExpRows; ++i) {
        const float m = wave_max(mx[i]);
        if (lane == i && r0 + i < jb.rows) jb.out[r0 + i] = row_exponent(m);
    }
}

ExpJob exp_job(const float *base, int64_t rows_per_batch, int batch, int64_t stride, int64_t ld, int K, int32_t *out)
{
    return ExpJob{base, stride, ld, (uint32_t)(rows_per_batch * batch), (uint32_t)rows_per_batch, K, out, nullptr};
}

hipError_t launch_exponents(const ExpJob *jobs, int count, uint32_t *zero_ptr, int64_t zero_n, hipStream_t stream)
{
    ExpJobs j{};
    j.zero_ptr = zero_ptr;
    j.zero_n = zero_ptr ? zero_n : 0;
    int64_t w = 0;
    for (int i = 0; i < 3; ++i) {
        j.first_wave[i] = w;
        if (i < count) {
            j.job[i] = jobs[i];
            const int per_wave = jobs[i].maxbits ? 64 : kExpRows;
            w += ((int64_t)jobs[i].rows + per_wave - 1) / per_wave;
        } else {
            j.job[i] = count > 0 ? jobs[0] : ExpJob{};
        }
    }
    j.first_wave[3] = w;
    w += (j.zero_n + 1023) / 1024;
    if (w <= 0) return hipSuccess;
    const int64_t blocks = (w + 3) / 4;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(row_exponent_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, j);
    return hipGetLastError();
}

// The row exponents of both operands into the workspace, in one launch
// (with the extra set, if asked); sets a_exp, b_exp (and b2_exp for a
// product-key B operand).  Nothing to launch when both are known.
hipError_t prepare_exponents(GemmArgs &a, bool product_b, hipStream_t stream)
{
    if (a.a_rowmax && a.b_exp_given && !product_b && !a.extra_exp.base) {
        a.b_exp = a.b_exp_given;
        return a.zero_ptr && a.exp_phase != 2 ? launch_exponents(nullptr, 0, a.zero_ptr, a.zero_n, stream)
                                              : hipSuccess;
    }
    if (!a.exp_ws || a.exp_ws_ints < gemm_exp_ints(a)) return hipErrorInvalidValue;
    if (gemm_exp_ints(a) >= ((int64_t)1 << 31)) return hipErrorInvalidConfiguration;
    int32_t *w = a.exp_ws;
    ExpJob jobs[3];
    int n = 0;
    if (!a.a_rowmax) {
        a.a_exp = w;
        jobs[n++] = exp_job(a.A, a.M, a.batch, a.strideA, a.lda, a.K, w);
    }
    w += (int64_t)a.batch * a.M;
    if (product_b) {
        a.b_exp = w;
        jobs[n++] = exp_job(a.B, a.key_n, a.batch, a.strideB, a.ldb, a.split_k, w);
        w += (int64_t)a.batch * a.key_n;
        a.b2_exp = w;
        jobs[n++] = exp_job(a.B2, a.key_n, a.batch, a.strideB, a.ldb, a.K - a.split_k, w);
    } else if (a.b_exp_given) {
        a.b_exp = a.b_exp_given;
    } else {
        a.b_exp = w;
        jobs[n++] = exp_job(a.B, a.N, a.batch, a.strideB, a.ldb, a.K, w);
    }
    if (a.extra_exp.base) {
        if (n >= 3) return hipErrorInvalidValue;
        const auto &x = a.extra_exp;
        jobs[n++] = exp_job(x.base, x.rows_per_batch, x.batch, x.stride, x.ld, x.K, x.out);
    }
    if (a.exp_phase == 2) return hipSuccess;  // computed by an earlier launch with these arguments
    return launch_exponents(jobs, n, a.zero_ptr, a.zero_n, stream);
}

// Rows of a B operand split into fp16 pieces once: every row scaled by its
// own power of two and split as split8 does, stored in the order a staging
// lane copies them: per set of rows, [group of 32 rows][chunk of 16 k]
// [piece][lane][8 fp16] with lane l = 32 kh + row % 32 holding k = 16 chunk
// + 8 kh .. + 7.  Rows past `rows` are zero.  Product-key operand (B2
// non-null, the flat search, split per call): set s = 2 g + p is batch entry
// g's first (p = 0, at B, exponents b_exp) or second (at B2, b2_exp) subkey
// set.  Plain operand (B2 null, prepared weights): set s is batch entry s
// (b_exp).  One thread per (set, group, chunk, lane).
__global__ __launch_bounds__(256) void split_rows_kernel(const float *B, const float *B2, int64_t strideB, int64_t ldb,
                                                         int rows, int kch, const int32_t *b_exp,
                                                         const int32_t *b2_exp, u4 *out)
{
    const int set = blockIdx.y;
    const bool pairs = B2 != nullptr;
    const int g = pairs ? set >> 1 : set, half = pairs ? set & 1 : 0;
    const int64_t per_set = (int64_t)((rows + 31) / 32) * kch * 64;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= per_set) return;
    const int lane = (int)(t & 63);
    const int64_t blk = t >> 6;  // group * kch + chunk
    const int grp = (int)(blk / kch), c = (int)(blk - (int64_t)grp * kch);
    const int row = grp * 32 + (lane & 31);
    fx4 v[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    int ex = 0;
    if (row < rows) {
        const float *src = (half ? B2 : B) + (int64_t)g * strideB + (int64_t)row * ldb + c * kBK + (lane >> 5) * 8;
        v[0] = *reinterpret_cast<const fx4 *>(src);
        v[1] = *reinterpret_cast<const fx4 *>(src + 4);
        ex = (half ? b2_exp : b_exp)[(int64_t)g * rows + row];
    }
    float one = 1.0f;
    asm volatile("" : "+v"(one));
    u4 hi, lo;
    split8(v, ex, one, hi, lo);
    u4 *dst = out + (int64_t)set * per_set * 2 + blk * 128 + lane;
    dst[0] = hi;
    dst[64] = lo;
}

// The query projection, inference batch-norm and one subkey set folded
// into one matrix (all three are linear maps, the batch-norm's statistics
// fixed): for head h, half p and subkey j,
//   s[f] . qhat[f] summed over the half's features f = x . M[g][j] + bias[g][j]
// with g = 2h + p, m_f = gamma_f / sqrt(var_f + eps),
//   M[g][j][i] = sum_f C[g][j][f] m_f Wq[h][f][i],
//   bias[g][j] = sum_f C[g][j][f] (beta_f - mean_f m_f),
// f over the half's D/2 features (C = the half's subkeys).  Accumulated in
// fp64 from the fp32 parameters, f in order, and rounded once to fp32.
// 128 x 128 tiles of (j, i), 256 threads of 8 x 8 outputs (rows
// j0 + 16 r + ty, columns i0 + 16 c + tx, so the LDS reads of a wave are
// consecutive), f in steps of 16 through LDS with the step's m_f and
// beta_f - mean_f m_f computed once; the i = 0 tiles also sum the bias.
__global__ __launch_bounds__(256) void fold_kernel(const float *wq, const float *mean, const float *var,
                                                   const float *gamma, const float *beta, double eps,
                                                   const float *sub, int D, int n, float *M, float *bias)
{
    const int g = blockIdx.z, h = g >> 1, p = g & 1, half = D / 2;
    const int j0 = blockIdx.y * 128, i0 = blockIdx.x * 128;
    const int f_base = h * D + p * half;  // the half's first feature in [H][D]
    const float *C = sub + (int64_t)g * n * half;
    __shared__ double As[16][129];     // [f][j]: C[j][f] m_f
    __shared__ double Bs[16][129];     // [f][i]: Wq[h][f][i]
    __shared__ double ms[16], ts[16];  // m_f and beta_f - mean_f m_f of the step's features
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    const bool with_bias = blockIdx.x == 0 && threadIdx.x < 128 && j0 + (int)threadIdx.x < n;
    double acc[8][8], bsum = 0.0;
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] = 0.0;
    for (int f0 = 0; f0 < half; f0 += 16) {
        if (threadIdx.x < 16) {
            const int hf = f_base + f0 + threadIdx.x;
            const double m = (double)gamma[hf] / sqrt((double)var[hf] + eps);
            ms[threadIdx.x] = m;
            ts[threadIdx.x] = (double)beta[hf] - (double)mean[hf] * m;
        }
        __syncthreads();
        for (int e = threadIdx.x; e < 2048; e += 256) {
            const int jj = e / 16, ff = e % 16;  // C rows run along f
            const int j = j0 + jj;
            As[ff][jj] = j < n ? (double)C[(int64_t)j * half + f0 + ff] * ms[ff] : 0.0;
            const int ff2 = e / 128, ii = e % 128;  // Wq rows run along i
            Bs[ff2][ii] = i0 + ii < D ? (double)wq[((int64_t)f_base + f0 + ff2) * D + i0 + ii] : 0.0;
        }
        if (with_bias) {
            const float *crow = C + (int64_t)(j0 + threadIdx.x) * half + f0;
#pragma unroll
            for (int ff = 0; ff < 16; ++ff) bsum = fma((double)crow[ff], ts[ff], bsum);
        }
        __syncthreads();
#pragma unroll
        for (int ff = 0; ff < 16; ++ff) {
            double a[8], b[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) a[r] = As[ff][16 * r + ty];
#pragma unroll
            for (int c = 0; c < 8; ++c) b[c] = Bs[ff][16 * c + tx];
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[r][c] = fma(a[r], b[c], acc[r][c]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int j = j0 + 16 * r + ty;
        if (j >= n) continue;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int i = i0 + 16 * c + tx;
            if (i < D) M[((int64_t)g * n + j) * D + i] = (float)acc[r][c];
        }
    }
    if (with_bias) bias[(int64_t)g * n + j0 + threadIdx.x] = (float)bsum;
}

// A plain A operand's rows, exponents and fp16 pieces in one pass (the
// folded lookup's x): one workgroup of four waves per quarter group (8 rows,
// four workgroups per 32-row group, so a call of a few thousand rows still
// gives every CU several workgroups).  First each wave takes two rows'
// largest magnitudes (every load of a 1024-wide block in flight before the
// maxima) and their exponents (to exp_out and LDS); then it writes the
// quarter's share of the pieces as split_rows_kernel lays them out -- four
// chunks per wave at a time, lane l splitting row l % 8 of the quarter,
// k = 16 c + 8 ((l / 8) % 2) .. + 7 of chunk c = c0 + l / 16, into the lane
// slot that row and k half have in the 32-row group (8-lane runs of one
// 128-byte line).  Rows past M get exponent 0 and zero pieces.
__global__ __launch_bounds__(256) void exp_split_rows_kernel(const float *A, int64_t lda, int M, int K,
                                                             int32_t *exp_out, u4 *out)
{
    __shared__ int ex_lds[8];
    const int grp = blockIdx.x >> 2, quarter = blockIdx.x & 3;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = grp * 32 + quarter * 8;
    const int r0 = row0 + wave * 2;
    float mx[2] = {0.0f, 0.0f};
    for (int base = 0; base < K; base += 1024) {
        fx4 v[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = base + 256 * q + 4 * lane;
                v[i][q] = r0 + i < M && c < K ? *reinterpret_cast<const fx4 *>(A + (int64_t)(r0 + i) * lda + c)
                                              : fx4{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                mx[i] = fmaxf(fmaxf(mx[i], fmaxf(fabsf(v[i][q][0]), fabsf(v[i][q][1]))),
                              fmaxf(fabsf(v[i][q][2]), fabsf(v[i][q][3])));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float m = wave_max(mx[i]);
        if (lane == i) {
            const int e = r0 + i < M ? row_exponent(m) : 0;
            ex_lds[wave * 2 + i] = e;
            if (r0 + i < M) exp_out[r0 + i] = e;
        }
    }
    __syncthreads();
    const int kch = K / kBK, rr = lane & 7, kh = (lane >> 3) & 1, ci = lane >> 4;
    const int row = row0 + rr, slot = kh * 32 + quarter * 8 + rr;
    const int ex = ex_lds[rr];
    float one = 1.0f;
    asm volatile("" : "+v"(one));
    // the waves take quads of chunks in turn, four quads' loads in flight
    for (int p0 = wave; 4 * p0 < kch; p0 += 16) {
        fx4 v[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 4 * (p0 + 4 * i) + ci;
            v[i][0] = v[i][1] = fx4{0.0f, 0.0f, 0.0f, 0.0f};
            if (row < M && c < kch) {
                const float *src = A + (int64_t)row * lda + c * kBK + kh * 8;
                v[i][0] = *reinterpret_cast<const fx4 *>(src);
                v[i][1] = *reinterpret_cast<const fx4 *>(src + 4);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 4 * (p0 + 4 * i) + ci;
            if (c < kch) {
                u4 hi, lo;
                split8(v[i], ex, one, hi, lo);
                u4 *dst = out + ((int64_t)grp * kch + c) * 128 + slot;
                dst[0] = hi;
                dst[64] = lo;
            }
        }
    }
}

template <typename T>
int64_t tile_count(const GemmArgs &a)
{
    return (int64_t)((a.M + T::BM - 1) / T::BM) * ((a.N + T::BN - 1) / T::BN);
}

template <typename T, bool BN_EPILOGUE, bool STREAM_OUT, bool PRODUCT_B = false, bool ACCUMULATE = false,
          bool PERSIST = false, bool KEEP_PRE = false, int SPLIT = 0>
hipError_t launch_variant(const GemmArgs &a, hipStream_t stream)
{
    const auto kernel =
        &gemm_nt_f32_kernel<T, BN_EPILOGUE, STREAM_OUT, PRODUCT_B, ACCUMULATE, PERSIST, KEEP_PRE, SPLIT>;
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
    dim3 grid((unsigned)tile_count<T>(a), a.batch, a.k_chunk ? (a.K + a.k_chunk - 1) / a.k_chunk : 1);
    if constexpr (PERSIST) {
        // kCUs workgroups, kCUs / kXcds per XCD (the kernel's tile order
        // needs a whole number per XCD; launch_tile persists only with at
        // least kCUs tiles)
        static_assert(kCUs % kXcds == 0, "workgroups per XCD");
        const int64_t total = tile_count<T>(a) * a.batch;
        if (total < kCUs) return hipErrorInvalidConfiguration;
        grid = dim3((unsigned)kCUs, 1, 1);
    }
    hipLaunchKernelGGL(kernel, grid, dim3(T::THREADS), T::LDS_BYTES, stream, a);
    return hipGetLastError();
}

template <typename T, int SPLIT>
hipError_t launch_tile_form(const GemmArgs &a, hipStream_t stream)
{
    if (tile_count<T>(a) > 0x7FFFFFFF || a.batch > 65535) return hipErrorInvalidConfiguration;
    if (a.C_pre && (!a.bn_mean || a.stream_out || a.accumulate || a.k_chunk ||
                    (reinterpret_cast<uintptr_t>(a.C_pre) & 15) != 0 || (reinterpret_cast<uintptr_t>(a.C) & 15) != 0))
        return hipErrorInvalidValue;
    // At least as many 256x256 tiles as CUs: one workgroup per CU walks its
    // tiles in the XCD-aware order, and the stores of one tile drain while
    // the next one computes
    const bool persist = T::PING_PONG && !a.k_chunk && tile_count<T>(a) * a.batch >= kCUs;
    if constexpr (SPLIT == 2) {
        // both operands split beforehand: the streamed epilogue only (the
        // folded lookup's scores)
        if (!a.stream_out || a.bn_mean || a.accumulate || a.C_pre) return hipErrorInvalidValue;
        if (persist) return launch_variant<T, false, true, false, false, true, false, 2>(a, stream);
        return launch_variant<T, false, true, false, false, false, false, 2>(a, stream);
    } else {
        if (a.accumulate) {
            if (a.bn_mean || a.stream_out || SPLIT) return hipErrorInvalidValue;
            if constexpr (!SPLIT) return launch_variant<T, false, false, false, true>(a, stream);
        }
        if (a.C_pre) {  // the BN epilogue keeping the values before BN (checked above)
            if (persist) return launch_variant<T, true, false, false, false, true, true, SPLIT>(a, stream);
            return launch_variant<T, true, false, false, false, false, true, SPLIT>(a, stream);
        }
        if (a.bn_mean) {
            if (a.stream_out) return launch_variant<T, true, true, false, false, false, false, SPLIT>(a, stream);
            if (persist) return launch_variant<T, true, false, false, false, true, false, SPLIT>(a, stream);
            return launch_variant<T, true, false, false, false, false, false, SPLIT>(a, stream);
        }
        if (a.stream_out) {
            if (persist) return launch_variant<T, false, true, false, false, true, false, SPLIT>(a, stream);
            return launch_variant<T, false, true, false, false, false, false, SPLIT>(a, stream);
        }
        return launch_variant<T, false, false, false, false, false, false, SPLIT>(a, stream);
    }
}

// Operands split ahead of the call (a_presplit with b_presplit, or
// b_presplit alone) or in every tile
template <typename T>
hipError_t launch_tile(const GemmArgs &a, hipStream_t stream)
{
    if (a.a_presplit) return launch_tile_form<T, 2>(a, stream);
    if (a.b_presplit) return launch_tile_form<T, 1>(a, stream);
    return launch_tile_form<T, 0>(a, stream);
}

// C[g][m][n] (+)= sum over s of P[s][g][m][n], s in order: the split-K
// partial products (P has row stride N, batch stride M * N).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *P, int splits, int M, int N, int batch,
                                                            float *C, int64_t ldc, int64_t strideC, bool accumulate)
{
    const int64_t per = (int64_t)M * N, total = per * batch;
    const int64_t zs = total;  // stride between splits
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int g = (int)(e / per);
        const int64_t r = e - g * per;
        const int m = (int)(r / N), n = (int)(r - (int64_t)m * N);
        float sum = P[e];
        for (int s = 1; s < splits; ++s) sum += P[e + s * zs];
        float *c = &C[(int64_t)g * strideC + (int64_t)m * ldc + n];
        *c = accumulate ? *c + sum : sum;
    }
}

}  // namespace

int64_t gemm_split_bytes(const GemmArgs &a)
{
    return (int64_t)a.batch * 2 * ((a.key_n + 31) / 32) * 32 * (int64_t)a.split_k * 4;
}

int64_t gemm_exp_ints(const GemmArgs &a)
{
    const int64_t b_rows = a.B2 ? 2 * (int64_t)a.key_n : (int64_t)a.N;
    return (int64_t)a.batch * ((int64_t)a.M + b_rows);
}

int64_t gemm_presplit_bytes(int rows, int K, int batch)
{
    return (int64_t)batch * ((rows + 31) / 32) * 32 * (int64_t)K * 4;
}

hipError_t launch_presplit(const float *B, int64_t stride, int64_t ld, int rows, int K, int batch, int32_t *exp,
                           void *out, hipStream_t stream)
{
    if (rows <= 0 || batch <= 0) return hipSuccess;
    if (K % 32 != 0 || batch > 65535 || (reinterpret_cast<uintptr_t>(out) & 15) != 0) return hipErrorInvalidValue;
    const ExpJob job = exp_job(B, rows, batch, stride, ld, K, exp);
    hipError_t e = launch_exponents(&job, 1, nullptr, 0, stream);
    if (e != hipSuccess) return e;
    const int kch = K / kBK;
    const int64_t per_set = (int64_t)((rows + 31) / 32) * kch * 64;
    hipLaunchKernelGGL(split_rows_kernel, dim3((unsigned)((per_set + 255) / 256), batch), dim3(256), 0, stream, B,
                       nullptr, stride, ld, rows, kch, exp, nullptr, reinterpret_cast<u4 *>(out));
    return hipGetLastError();
}

hipError_t launch_exp_split(const float *A, int64_t lda, int M, int K, int32_t *exp_out, void *out,
                            hipStream_t stream)
{
    if (M <= 0) return hipSuccess;
    if (K % 32 != 0 || lda % 4 != 0 || (reinterpret_cast<uintptr_t>(A) & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(out) & 15) != 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(exp_split_rows_kernel, dim3((unsigned)((M + 31) / 32 * 4)), dim3(256), 0, stream, A, lda, M, K,
                       exp_out, reinterpret_cast<u4 *>(out));
    return hipGetLastError();
}

hipError_t launch_fold(const float *wq, const float *mean, const float *var, const float *gamma, const float *beta,
                       float eps, const float *subkeys, int D, int H, int n, float *M, float *bias, hipStream_t stream)
{
    if (D % 64 != 0 || D / 2 % 16 != 0 || H < 1 || n < 1 || 2 * H > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fold_kernel, dim3((D + 127) / 128, (n + 127) / 128, 2 * H), dim3(256), 0, stream, wq, mean, var,
                       gamma, beta, (double)eps, subkeys, D, n, M, bias);
    return hipGetLastError();
}

hipError_t launch_gemm_nt_f32(const GemmArgs &args, hipStream_t stream)
{
    if (args.M <= 0 || args.N <= 0 || args.batch <= 0) return hipSuccess;
    if (args.K % 32 != 0 || args.k_chunk != 0 || args.B2) return hipErrorInvalidValue;
    if (args.b_presplit && (!args.b_exp_given || args.accumulate || (reinterpret_cast<uintptr_t>(args.b_presplit) & 15)))
        return hipErrorInvalidValue;
    if (args.a_presplit && (!args.b_presplit || args.a_rowmax || args.batch != 1 || !args.stream_out ||
                            (reinterpret_cast<uintptr_t>(args.a_presplit) & 15)))
        return hipErrorInvalidValue;
    GemmArgs a = args;
    hipError_t e = prepare_exponents(a, false, stream);
    if (e != hipSuccess || a.exp_phase == 1) return e;
    const int64_t tiles = tile_count<BigTile>(a) * a.batch;
    if (tiles >= kCUs) return launch_tile<BigTile>(a, stream);
    // Split K when the contraction is long enough (at least 512 per split)
    // and a workspace for the partial products was given.
    int splits = (int)((kCUs + tiles - 1) / tiles);
    if (splits > kMaxKSplits) splits = kMaxKSplits;
    if (splits > a.K / 512) splits = a.K / 512;
    const int64_t need = (int64_t)splits * a.batch * a.M * a.N;
    if (splits >= 2 && a.partial && need <= a.partial_floats && !a.bn_mean && !a.stream_out) {
        GemmArgs p = a;
        p.k_chunk = (a.K / 32 + splits - 1) / splits * 32;
        p.C = a.partial;
        p.ldc = a.N;
        p.strideC = (int64_t)a.M * a.N;
        p.accumulate = false;
        e = launch_tile<BigTile>(p, stream);
        if (e != hipSuccess) return e;
        const int used = (a.K + p.k_chunk - 1) / p.k_chunk;
        const int64_t total = (int64_t)a.batch * a.M * a.N;
        const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, stream, a.partial, used, a.M, a.N,
                           a.batch, a.C, a.ldc, a.strideC, a.accumulate);
        return hipGetLastError();
    }
    return launch_tile<SmallTile>(a, stream);
}

hipError_t launch_gemm_nt_f32_product(const GemmArgs &args, hipStream_t stream)
{
    if (args.M <= 0 || args.N <= 0 || args.batch <= 0) return hipSuccess;
    if (args.K % 32 != 0 || args.split_k % 32 != 0 || 2 * args.split_k != args.K || !args.B2 || args.key_n <= 0 ||
        (int64_t)args.key_n * args.key_n < args.N || args.bn_mean || args.k_chunk != 0 || !args.b_split ||
        args.b_split_bytes < gemm_split_bytes(args) || (reinterpret_cast<uintptr_t>(args.b_split) & 15) != 0)
        return hipErrorInvalidValue;
    if (tile_count<KeyTile>(args) > 0x7FFFFFFF || args.batch > 32767) return hipErrorInvalidConfiguration;
    const bool wide = args.M > 32;
    GemmArgs a = args;
    hipError_t e = prepare_exponents(a, true, stream);
    if (e != hipSuccess || a.exp_phase == 1) return e;
    const int kch = a.split_k / kBK;
    const int64_t per_set = (int64_t)((a.key_n + 31) / 32) * kch * 64;
    hipLaunchKernelGGL(split_rows_kernel, dim3((unsigned)((per_set + 255) / 256), 2 * a.batch), dim3(256), 0, stream,
                       a.B, a.B2, a.strideB, a.ldb, a.key_n, kch, a.b_exp, a.b2_exp,
                       reinterpret_cast<u4 *>(a.b_split));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (wide) return launch_variant<KeyTile64, false, false, true>(a, stream);
    return launch_variant<KeyTile, false, false, true>(a, stream);
}

}  // namespace pkm
