// gemm.hip -- the projection of Eq. 1 (SRU++ paper, background section):
// the three gate matrices of all timesteps (and both directions) in one
// GEMM, U = X~ W^T, and its input gradient dX = dU W.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 (gfx950) with fp32 accumulation.  The
// A operand may arrive as fp32; it is rounded to bf16 (nearest even) while
// it is staged into LDS, so no separate conversion pass touches HBM.
// B (the weights) is bf16 and is used either as [N, K] (C = A B^T, both
// operands K-contiguous: the forward projection, and the backward-data
// product when W has been transposed once by sru_transpose_weight) or as
// [K, N] (C = A B, transposed while it is staged into LDS).
//
// Block tiles of the register-staged kernel (gemm_bf16_mfma): a grid of
// waves, each wave a tile of 32 x 32 MFMA blocks; the k-tile is staged
// global -> registers -> LDS (double-buffered in LDS) while the previous one
// is multiplied.  Large problems use 256 x 256 blocks of 8 waves (one block
// per CU, two waves per SIMD), small ones 128 x 128 blocks of 4 waves (two
// blocks per CU) to keep every CU busy.  C is fp32, or bf16 for the products
// whose consumers take bf16.
//
// When both operands are bf16, gemm_lds copies the k-tiles from memory
// straight into LDS (no registers, no LDS write instructions): A as [M, K]
// rows, B as [N, K] rows or as [K, N] k-rows (read back by transposing LDS
// reads, ds_read_b64_tr_b16).
//
// The weight gradient dW = dU^T X~ reads both operands K-major (the
// reduction index L*B is the slow one) and may split that reduction across
// blocks; split_reduce then adds the partial products in a fixed order.
// With bf16 operands (an fp32 X is rounded into the workspace first)
// gemm_lds_t copies both into LDS and reads both back transposed.
//
// fp32 path (W in fp32): LDS-tiled FMA kernel, fp32 products and sums.
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "internal.h"

namespace sru {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));


#ifndef SRU_GEMM_DB
#define SRU_GEMM_DB 1
#endif
#ifndef SRU_GEMM_HINTS
#define SRU_GEMM_HINTS 1
#endif

template <int BM_, int BN_, int BK_, int STAGES_, int MINB_, int WGM_ = 2, int WGN_ = 2,
          bool DB_ = true>
struct TileCfg {
    static constexpr bool DB = DB_ && SRU_GEMM_DB;   // two fragment buffers per wave
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int STAGES = STAGES_;   // register stages of prefetched k-tiles
    static constexpr int MINB = MINB_;       // blocks per CU the registers are sized for
    static constexpr int WGM = WGM_, WGN = WGN_;   // wave grid of the block
    static constexpr int NT = 64 * WGM * WGN;      // threads per block
    static constexpr int LDK = BK + 8;       // padded LDS row (bf16): 80 or 144 bytes
                                             // keeps 16-byte reads of 8 rows on distinct banks
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int TI = WM / 32, TJ = WN / 32;
    static constexpr int EPI_LD = WN + 4;    // fp32 epilogue staging row
    static constexpr int LDS_BYTES = 2 * (BM + BN) * LDK * 2;
    static_assert(LDS_BYTES >= WGM * WGN * 32 * EPI_LD * 4, "epilogue staging must fit in LDS");
};

// 128 x 128 blocks of 4 waves (two blocks per CU) for grids too small to
// fill the chip with larger tiles; 256 x 256 blocks of 8 waves (two waves per
// SIMD, 128 x 64 each) otherwise.  With 8 waves a k-tile costs each thread
// only a few staging registers, and the second wave of every SIMD issues its
// MFMAs while the first waits on LDS or on its loads.
typedef TileCfg<128, 128, 64, 1, 2> CfgSmall;
typedef TileCfg<256, 256, 64, 1, 1, 2, 4, false> CfgBig8;
// 256 x 192 blocks of 8 waves (4 x 2, 64 x 96 each): used where 256 x 256
// tiles would leave the last round of blocks part-empty and these fill whole
// rounds of the 256 CUs.
typedef TileCfg<256, 192, 64, 1, 1, 4, 2, false> CfgWide8;
#ifndef SRU_GEMM_WIDE
#define SRU_GEMM_WIDE 1
#endif
// Four register stages for bf16 A on small grids: with a long K and one
// block per CU the loads must be requested four k-tiles ahead to cover a
// round trip to HBM (the operand then comes from HBM, e.g. the bf16 dU the
// backward has just written).  fp32 A has no registers for that depth.
typedef TileCfg<128, 128, 64, 4, 2, 2, 2, false> CfgSmallDeep;


// ---- row-major operand tile (ROWS x BK) -> registers -> LDS (bf16) --------
// The operand is stored with its tile rows along the reduction (A as [M, K],
// or B as [N, K]), row stride ld elements.  FAST (whole k-tiles, 16-byte
// aligned rows): every thread's element offsets inside the k-tile window are
// loop invariant 32-bit byte offsets (rows past the end are clamped to the
// last row: they load valid memory whose results the epilogue never writes),
// and the window's base pointer is uniform.  Otherwise every element is
// bounds checked.  fp32 elements are rounded to bf16 (nearest even) as they
// are written to LDS.
template <class Cfg, int ROWS, typename T, bool FAST>
struct RowLoader {
    static constexpr int V = 16 / sizeof(T);             // elements per 16 bytes
    static constexpr int PER_ROW = Cfg::BK / V;
    static constexpr int N = ROWS * PER_ROW / Cfg::NT;   // 16-byte loads per thread
    struct Offsets {
        uint32_t v[N];
    };
    u32x4 reg[N];
    const Offsets *off = nullptr;                        // shared by the stages
    __device__ __forceinline__ static void init(Offsets &o, int64_t ld, int64_t rows,
                                                int64_t r0, int tid)
    {
        if (FAST) {
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int idx = tid + i * Cfg::NT;
                int64_t row = idx / PER_ROW;
                if (r0 + row > rows - 1) row = rows - 1 - r0;
                o.v[i] = (uint32_t)((row * ld + (idx % PER_ROW) * V) * (int64_t)sizeof(T));
            }
        }
    }
    __device__ __forceinline__ void load(const T *P, int64_t ld, int64_t rows, int64_t K,
                                         int64_t r0, int64_t k0, int tid)
    {
        if (FAST) {
            const char *base = (const char *)(P + r0 * ld + k0);   // uniform
#pragma unroll
            for (int i = 0; i < N; ++i) reg[i] = *(const u32x4 *)(base + off->v[i]);
            return;
        }
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * Cfg::NT;
            const int row = idx / PER_ROW, cv = idx % PER_ROW;
            const int64_t r = r0 + row, k = k0 + cv * V;
            u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const T a = (r < rows && k + e < K) ? P[r * ld + k + e] : T(0);
                if constexpr (sizeof(T) == 4)
                    v[e] = __builtin_bit_cast(uint32_t, a);
                else
                    v[e / 2] |= uint32_t(a) << (16 * (e % 2));
            }
            reg[i] = v;
        }
    }
    __device__ __forceinline__ void store(bf16_bits *S, int tid) const
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * Cfg::NT;
            const int row = idx / PER_ROW, cv = idx % PER_ROW;
            bf16_bits *dst = S + row * Cfg::LDK + cv * V;
            if constexpr (sizeof(T) == 4) {   // round fp32 -> bf16 (nearest even) here
                const u32x4 u = reg[i];
                u32x2 packed;
                packed.x = pack_bf16x2(__uint_as_float(u.x), __uint_as_float(u.y));
                packed.y = pack_bf16x2(__uint_as_float(u.z), __uint_as_float(u.w));
                *(u32x2 *)dst = packed;
            } else {
                *(u32x4 *)dst = reg[i];
            }
        }
    }
};

// ---- K-major operand -> LDS as S[r][k] (ROWS x BK) ------------------------
// The operand is stored [K, rows] with row stride ld >= rows (its tile rows
// contiguous): B given as [K, N], or A given as [K, M].  Each thread gathers KG k-values of
// two adjacent rows (one 4-byte load of a bf16 pair, or one 8-byte load of an
// fp32 pair, per k; a wave reads whole contiguous row segments) and writes
// them as 16-byte LDS rows (fp32 rounded to bf16, nearest even, here), so
// the tile is transposed without 2-byte LDS stores.
template <class Cfg, int ROWS, typename T, bool FAST>
struct KLoader {
    static constexpr int NP = ROWS / 2;                  // row pairs
    static constexpr int KQ = Cfg::NT / NP;              // k-groups
    static constexpr int KG = Cfg::BK / KQ;              // k-rows per thread
    static_assert(KG % 8 == 0 && KQ * NP == Cfg::NT, "whole 16-byte LDS rows");
    typedef typename std::conditional<sizeof(T) == 2, uint32_t, u32x2>::type Reg;
    struct Offsets {
        uint32_t v;                                      // byte offset
    };
    Reg reg[KG];
    const Offsets *off = nullptr;
    __device__ __forceinline__ static void init(Offsets &o, int64_t ld, int64_t rows,
                                                int64_t r0, int tid)
    {
        if (FAST) {   // ld and rows even: the pair (r, r+1) is one aligned load
            int64_t c = 2 * (tid % NP);
            if (r0 + c > rows - 2) c = rows - 2 - r0;    // rows past the end: any valid pair
            o.v = (uint32_t)(((tid / NP) * KG * ld + c) * (int64_t)sizeof(T));
        }
    }
    __device__ __forceinline__ void load(const T *P, int64_t ld, int64_t rows, int64_t K,
                                         int64_t r0, int64_t k0, int tid)
    {
        if (FAST) {
#pragma unroll
            for (int e = 0; e < KG; ++e) {
                const char *base = (const char *)(P + (k0 + e) * ld + r0);   // uniform
                reg[e] = *(const Reg *)(base + off->v);
            }
            return;
        }
        const int np = tid % NP, kq = tid / NP;
        const int64_t r = r0 + 2 * np;
#pragma unroll
        for (int e = 0; e < KG; ++e) {
            const int64_t k = k0 + kq * KG + e;
            const T lo = (k < K && r < rows) ? P[k * ld + r] : T(0);
            const T hi = (k < K && r + 1 < rows) ? P[k * ld + r + 1] : T(0);
            if constexpr (sizeof(T) == 2) {
                reg[e] = uint32_t(lo) | (uint32_t(hi) << 16);
            } else {
                reg[e].x = __builtin_bit_cast(uint32_t, lo);
                reg[e].y = __builtin_bit_cast(uint32_t, hi);
            }
        }
    }
    __device__ __forceinline__ void store(bf16_bits *S, int tid) const
    {
        const int np = tid % NP, kq = tid / NP;
        // row r takes the low halves (first elements), row r + 1 the high ones
#pragma unroll
        for (int h = 0; h < KG / 8; ++h) {
            const Reg *g = reg + h * 8;
            u32x4 lo, hi;
            if constexpr (sizeof(T) == 2) {
                auto lo2 = [](uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); };
                auto hi2 = [](uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); };
                lo = u32x4{lo2(g[0], g[1]), lo2(g[2], g[3]), lo2(g[4], g[5]), lo2(g[6], g[7])};
                hi = u32x4{hi2(g[0], g[1]), hi2(g[2], g[3]), hi2(g[4], g[5]), hi2(g[6], g[7])};
            } else {
                auto f = [](uint32_t u) { return __uint_as_float(u); };
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    lo[v] = pack_bf16x2(f(g[2 * v].x), f(g[2 * v + 1].x));
                    hi[v] = pack_bf16x2(f(g[2 * v].y), f(g[2 * v + 1].y));
                }
            }
            *(u32x4 *)(S + (2 * np) * Cfg::LDK + kq * KG + h * 8) = lo;
            *(u32x4 *)(S + (2 * np + 1) * Cfg::LDK + kq * KG + h * 8) = hi;
        }
    }
};

// f(integral_constant<0>) ... f(integral_constant<UNR - 1>) in order, until
// one returns true (then true).
template <int U, int UNR, class F> __device__ __forceinline__ bool unroll_until(F &&f)
{
    if constexpr (U == UNR) {
        return false;
    } else {
        if (f(std::integral_constant<int, U>{})) return true;
        return unroll_until<U + 1, UNR>(f);
    }
}

// Tile order: the hardware hands consecutive workgroups to the 8 XCDs in
// turn, each XCD with its own L2.  Workgroup `bid` is given logical tile
// (bid % 8) * (T / 8) + bid / 8, so every XCD works through one contiguous
// range of tiles; within the logical order, groups of 8 row tiles sweep the
// column tiles so neighbouring tiles share A rows and B columns in that L2.
__device__ __forceinline__ void tile_of(int64_t bid, int64_t TM, int64_t TN, int64_t GM,
                                        int64_t *tm, int64_t *tn)
{
    const int64_t T = TM * TN;
    const int64_t T8 = T / 8;
    int64_t lt = bid;
    if (bid < 8 * T8) lt = (bid % 8) * T8 + bid / 8;
    const int64_t group = lt / (GM * TN);
    const int64_t first = group * GM;
    const int64_t gsz = (TM - first) < GM ? (TM - first) : GM;
    const int64_t in = lt % (GM * TN);
    *tm = first + in % gsz;
    *tn = in / gsz;
}

// Row tiles per group of the tile order.  When the tiles of one XCD's share
// (T / 8) are whole rows of column tiles, one group is that share, so each
// row block of A is read by one XCD only (the projection on fp32 X at L*B =
// 8192, 3d = 3072: 4 row tiles of 16); otherwise groups of 8 row tiles.
inline int64_t group_rows(int64_t M, int64_t N, int64_t bm, int64_t bn)
{
    const int64_t TM = (M + bm - 1) / bm, TN = (N + bn - 1) / bn, T8 = TM * TN / 8;
    if (T8 >= TN && T8 % TN == 0 && T8 / TN <= 8) return T8 / TN;
    return 8;
}

// Shape, strides and options of one launch (passed by value).
struct MM {
    int64_t M, N, K;
    int64_t lda, ldb, ldc;   // row strides (elements) of A, B and C as stored
    int64_t sa, sb, sc;      // element offsets between the batches (blockIdx.y)
    int64_t ksplit;          // k-range per split (>= K: no split)
    int gm;                  // row tiles per group of the tile order
    bool accumulate;
    // causal products (gemm_lds only; -1: off), row m seeing columns
    // n <= c + m: cskip = c skips tiles with no such column, whose C is never
    // read; klim = c ends each row tile's reduction after k = c + its last
    // row, the rest of its A row being zeros
    int64_t cskip = -1, klim = -1;
};

// C[M, N] (+)= A . B, where A is given as [M, K] (AKM = false) or [K, M]
// (AKM = true, i.e. C = A^T B) and B as [N, K] (KN = false, C = A B^T) or
// [K, N], each with its own row stride; blockIdx.y selects a batch (base
// offsets sa, sb, sc).  With several splits block s of a tile covers k in
// [s * ksplit, (s + 1) * ksplit) and writes its partial product to
// C + s * M * ldc, to be summed in order by split_reduce.  C is fp32, or
// bf16 (rounded to nearest even; no accumulation) when TC is bf16.
template <class Cfg, typename TA, bool AKM, typename TB, bool KN, bool FAST, typename TC>
__global__ __launch_bounds__(Cfg::NT, Cfg::MINB) void gemm_bf16_mfma(
    MM p, const TA *__restrict__ A, const TB *__restrict__ Bm, TC *__restrict__ C)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, LDK = Cfg::LDK;
    constexpr int WM = Cfg::WM, WN = Cfg::WN, TI = Cfg::TI, TJ = Cfg::TJ;
    constexpr int STAGE = (BM + BN) * LDK;               // bf16 elements per LDS stage
    __shared__ __attribute__((aligned(16))) bf16_bits smem[2 * STAGE];

    const int64_t M = p.M, N = p.N, lda = p.lda, ldb = p.ldb, ldc = p.ldc;
    int64_t K = p.K;
    const bool accumulate = p.accumulate;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;
    A += (int64_t)blockIdx.y * p.sa;
    Bm += (int64_t)blockIdx.y * p.sb;
    C += (int64_t)blockIdx.y * p.sc;
    const int64_t TM = (M + BM - 1) / BM, TN = (N + BN - 1) / BN;
    const int64_t split = (int64_t)blockIdx.x / (TM * TN);
    if (split > 0 || p.ksplit < K) {   // this block's k-range
        const int64_t kb = split * p.ksplit;
        A += AKM ? kb * lda : kb;
        Bm += KN ? kb * ldb : kb;
        K = (K - kb) < p.ksplit ? (K - kb) : p.ksplit;
        C += split * M * ldc;
    }
    int64_t tm, tn;
    tile_of((int64_t)blockIdx.x % (TM * TN), TM, TN, p.gm, &tm, &tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;

    bf16_bits *As0 = smem, *Bs0 = smem + BM * LDK;
    bf16_bits *As1 = smem + STAGE, *Bs1 = smem + STAGE + BM * LDK;

    typedef typename std::conditional<AKM, KLoader<Cfg, BM, TA, FAST>,
                                      RowLoader<Cfg, BM, TA, FAST>>::type AL;
    typedef typename std::conditional<KN, KLoader<Cfg, BN, TB, FAST>,
                                      RowLoader<Cfg, BN, TB, FAST>>::type BL;
    typename AL::Offsets aoff;
    typename BL::Offsets boff;
    AL::init(aoff, lda, M, m0, tid);
    BL::init(boff, ldb, N, n0, tid);
    AL la0;
    BL lb0;
    la0.off = &aoff;
    lb0.off = &boff;

    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int r32 = lane & 31;
    const int kg = (lane >> 5) * 8;
    // MFMAs of k16 steps [ks0, ks1) of the tile in LDS
    auto compute_steps = [&](const bf16_bits *As, const bf16_bits *Bs, int ks0, int ks1) {
#pragma unroll 2   // full unrolling hoists every fragment read and spills
        for (int ks = ks0; ks < ks1; ++ks) {
            bf16x8 af[TI], bfr[TJ];
#pragma unroll
            for (int i = 0; i < TI; ++i)
                af[i] = *(const bf16x8 *)(As + (wm * WM + i * 32 + r32) * LDK + ks * 16 + kg);
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                bfr[j] = *(const bf16x8 *)(Bs + (wn * WN + j * 32 + r32) * LDK + ks * 16 + kg);
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
    };
    auto compute = [&](const bf16_bits *As, const bf16_bits *Bs) {
        compute_steps(As, Bs, 0, BK / 16);
    };
    // The whole k-tile with the fragments of step ks + 1 read while the
    // MFMAs of step ks run (two fragment buffers), and `tail` (the LDS writes
    // of the next k-tile) issued among the MFMAs of the last step.  The
    // scheduling hints keep the compiler from bunching the reads: one
    // fragment read after every few MFMAs.
    auto compute_db = [&](const bf16_bits *As, const bf16_bits *Bs, auto &&tail) {
        constexpr int KS = BK / 16;
        constexpr int NF = TI + TJ;                     // fragment reads per step
        constexpr int MF = TI * TJ;                     // MFMAs per step
        bf16x8 af[2][TI], bfr[2][TJ];
        auto rd = [&](int buf, int ks) {
#pragma unroll
            for (int i = 0; i < TI; ++i)
                af[buf][i] = *(const bf16x8 *)(As + (wm * WM + i * 32 + r32) * LDK + ks * 16 + kg);
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                bfr[buf][j] = *(const bf16x8 *)(Bs + (wn * WN + j * 32 + r32) * LDK + ks * 16 + kg);
        };
        rd(0, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < KS) rd(cur ^ 1, ks + 1);
            if (ks + 1 == KS) tail();
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
#if SRU_GEMM_HINTS
            if (ks + 1 < KS) {
#pragma unroll
                for (int t = 0; t < NF; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, MF / NF > 0 ? MF / NF : 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
#endif
            // no code moves across steps: at most two fragment sets are live
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Software pipeline: k-tile kt is in LDS stage kt % 2 while the loads of
    // the next STAGES k-tiles are in flight (one register stage, or a ring of
    // three or more).  The body has no conditional
    // loads or stores (prefetch indices are clamped to the last k-tile; the
    // surplus loads re-read it), which keeps the compiler's wait counts
    // exact: a stage waits only for its own loads.
    const int64_t KT = (K + BK - 1) / BK;
    auto kc = [&](int64_t kt) { return (kt < KT ? kt : KT - 1) * BK; };
    if constexpr (Cfg::STAGES >= 3) {
        // A ring of NS register stages: tile kt + NS is requested while tile
        // kt is multiplied, and tile kt + 1 is written to the other LDS stage
        // during the last MFMAs of tile kt, NS - 1 tiles after its loads were
        // issued.  Long-K problems with one block per CU need this depth to
        // cover a round trip to HBM.
        constexpr int NS = Cfg::STAGES;
        constexpr int UNR = NS % 2 == 0 ? NS : 2 * NS;   // stage and LDS parity repeat
        AL la[NS];
        BL lb[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            la[i].off = &aoff;
            lb[i].off = &boff;
        }
        bf16_bits *Asl[2] = {As0, As1}, *Bsl[2] = {Bs0, Bs1};
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            la[i].load(A, lda, M, K, m0, kc(i), tid);
            lb[i].load(Bm, ldb, N, K, n0, kc(i), tid);
        }
        la[0].store(As0, tid);
        lb[0].store(Bs0, tid);
        __syncthreads();
        auto body = [&](int64_t kt, auto u_) -> bool {
            constexpr int u = decltype(u_)::value;
            constexpr int rs = u % NS, rn = (u + 1) % NS, ls = u % 2, ln = (u + 1) % 2;
            la[rs].load(A, lda, M, K, m0, kc(kt + NS), tid);
            lb[rs].load(Bm, ldb, N, K, n0, kc(kt + NS), tid);
            if constexpr (Cfg::DB) {
                compute_db(Asl[ls], Bsl[ls], [&] {
                    la[rn].store(Asl[ln], tid);
                    lb[rn].store(Bsl[ln], tid);
                });
            } else {
                compute(Asl[ls], Bsl[ls]);
                la[rn].store(Asl[ln], tid);
                lb[rn].store(Bsl[ln], tid);
            }
            __syncthreads();
            return kt + 1 >= KT;
        };
        for (int64_t kt = 0;; kt += UNR)
            if (unroll_until<0, UNR>([&](auto u_) { return body(kt + decltype(u_)::value, u_); }))
                break;
    } else {
    la0.load(A, lda, M, K, m0, 0, tid);
    lb0.load(Bm, ldb, N, K, n0, 0, tid);
    la0.store(As0, tid);
    lb0.store(Bs0, tid);
    static_assert(Cfg::STAGES == 1, "one register stage here; three or more above");
    {
        __syncthreads();
        // 256 x 256 wave tiles hold no second fragment set: plain steps there
        constexpr bool kDB = Cfg::DB && !(TI * TJ >= 16);
        if constexpr (kDB) {
        for (int64_t kt = 0;; kt += 2) {
            la0.load(A, lda, M, K, m0, kc(kt + 1), tid);
            lb0.load(Bm, ldb, N, K, n0, kc(kt + 1), tid);
            compute_db(As0, Bs0, [&] {
                la0.store(As1, tid);
                lb0.store(Bs1, tid);
            });
            __syncthreads();
            if (kt + 1 >= KT) break;
            la0.load(A, lda, M, K, m0, kc(kt + 2), tid);
            lb0.load(Bm, ldb, N, K, n0, kc(kt + 2), tid);
            compute_db(As1, Bs1, [&] {
                la0.store(As0, tid);
                lb0.store(Bs0, tid);
            });
            __syncthreads();
            if (kt + 2 >= KT) break;
        }
        } else {
        for (int64_t kt = 0;; kt += 2) {
            la0.load(A, lda, M, K, m0, kc(kt + 1), tid);
            lb0.load(Bm, ldb, N, K, n0, kc(kt + 1), tid);
            compute(As0, Bs0);
            la0.store(As1, tid);
            lb0.store(Bs1, tid);
            __syncthreads();
            if (kt + 1 >= KT) break;
            la0.load(A, lda, M, K, m0, kc(kt + 2), tid);
            lb0.load(Bm, ldb, N, K, n0, kc(kt + 2), tid);
            compute(As1, Bs1);
            la0.store(As0, tid);
            lb0.store(Bs0, tid);
            __syncthreads();
            if (kt + 2 >= KT) break;
        }
        }
    }

    }

    // Epilogue, one 32-row band of the wave tile at a time: stage it in LDS
    // (the 32x32 accumulator layout holds column lane & 31 and rows
    // 8*(r/4) + 4*(lane/32) + r%4) and write it back as 16-byte row segments.
    // Each wave uses its own staging area; LDS operations of one wave complete
    // in order, so no barrier is needed between bands.
    constexpr int EPI_LD = Cfg::EPI_LD;
    float *stage = (float *)smem + wave * (32 * EPI_LD);
    constexpr int C4 = WN / 4;                           // float4 per staged row
    const int64_t nw = n0 + wn * WN;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
                stage[row * EPI_LD + j * 32 + r32] = acc[i][j][r];
            }
        const int64_t mw = m0 + wm * WM + i * 32;
#pragma unroll 4
        for (int it = 0; it < 32 * C4 / 64; ++it) {
            const int idx = it * 64 + lane;
            const int row = idx / C4, c4 = idx % C4;
            const int64_t m = mw + row, n = nw + c4 * 4;
            if (m >= M) continue;
            const float4 v = *(const float4 *)(stage + row * EPI_LD + c4 * 4);
            TC *q = C + m * ldc + n;
            if constexpr (sizeof(TC) == 2) {
                if (FAST) {
                    if (n < N) *(u32x2 *)q = u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
                } else {
                    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) q[e] = f32_to_bf16(vv[e]);
                }
            } else if (FAST) {   // N, ldc and the batch offset multiples of 4
                if (n < N) {
                    float4 o = v;
                    if (accumulate) {
                        const float4 c = *(const float4 *)q;
                        o.x += c.x; o.y += c.y; o.z += c.z; o.w += c.w;
                    }
                    *(float4 *)q = o;
                }
            } else {
                const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < N) q[e] = accumulate ? q[e] + vv[e] : vv[e];
            }
        }
    }
}

// ---- bf16 x bf16^T with operands copied straight into LDS ------------------
// C[M, N] (+)= A[M, K] B[N, K]^T for bf16 A and B (16-byte aligned rows; K a
// multiple of 64), fp32 C.  Each k-tile of A and B (rows of 64 bf16 = 128
// bytes) travels from memory to LDS by global_load_lds_dwordx4: one instruction moves 64 lanes x 16 bytes
// into 1 KB of LDS, so the operands take no registers on the way and no LDS
// write instructions.  NS LDS stages form a ring: k-tile kt + NS - 1 is
// requested while k-tile kt is multiplied, and a wave waits (vmcnt) only for
// its own requests of k-tile kt before the barrier that publishes the stage.
// Inside a row the sixteen-byte piece holding k-chunk c sits at position
// c ^ ((row / 2) % 8): LDS serves a 16-byte-per-lane read 16 lanes (256
// bytes, all 64 banks) at a time, and two 128-byte rows share one bank line,
// so the fragment reads of sixteen consecutive rows then touch every bank
// once.  (fp32 A is not taken: converted as its fragments
// are read, by every wave that reads them, it is slower than the register-
// staged kernel, which converts each element once.)
// ---- K-major operands in LDS: transposing reads ---------------------------
// An operand stored K-major (rows along k, columns along M or N) keeps that
// layout in LDS: a k-tile is 64 rows of the tile's 128 or 256 columns, copied
// memory -> LDS in 1 KB requests of whole rows.  The MFMA operand (8
// consecutive k of one column per lane) is read back with ds_read_b64_tr_b16:
// within a group of 16 lanes, lane i receives the i-th 16-bit element of each
// of the four 8-byte pieces that lanes 4j + i / 4 address (j = 0..3), so when
// lanes 4j .. 4j + 3 address row k0 + j, columns c .. c + 15, lane i gets
// column c + i at k0 .. k0 + 3, and two such reads give the 8 k of the
// 32x32x16 operand.
//
// The 16-byte pieces of a row (P = 0..31, columns 8P .. 8P + 7; 0..15 for
// 128 columns) are stored at position tr_pos(P, row): writing P = 4a + 2b +
// c, position c + 2 (a mod 4) + 8 b + 16 (a / 4), XOR 2 (row mod 4).  A read
// of 16 columns touches pieces 4a + 2b + {0, 1} of four consecutive rows: the
// XOR spreads the four rows over four bank groups and b puts the two
// 16-column halves of a 32-column block eight positions apart, so each
// half-wave's 256 bytes fall on distinct banks (rows are 512 or 256 bytes,
// whole bank lines).
__device__ __forceinline__ int tr_pos(int P, int row)
{
    const int c = P & 1, b = (P >> 1) & 1, a = P >> 2;
    return (c + 2 * (a & 3) + 8 * b + 16 * (a >> 2)) ^ (2 * (row & 3));
}
__device__ __forceinline__ int tr_piece(int pos, int row)   // the inverse of tr_pos
{
    const int q = pos ^ (2 * (row & 3));
    return 4 * (((q >> 1) & 3) + 4 * (q >> 4)) + 2 * ((q >> 3) & 1) + (q & 1);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// The 32x32x16 operand of columns c .. c + 31 (c a multiple of 32) at k-step
// ks from a K-major tile at `base` (rows of ROWB bytes): lane l gets column
// c + l % 32, k = 16 ks + 8 (l / 32) + 0..7.
template <int ROWB>
__device__ __forceinline__ bf16x8 tr_frag(const char *base, int c, int ks, int lane)
{
    const int g = lane >> 4, pl = lane & 15;
    const int col = c + 16 * (g & 1) + 4 * (pl & 3);
    const int P = col >> 3, h8 = (col >> 2) & 1;
    const int r0 = 16 * ks + 8 * (g >> 1) + (pl >> 2), r1 = r0 + 4;
    typedef __attribute__((address_space(3))) i16x4 *lds_p;
    const char *b = base + h8 * 8;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_p)(b + r0 * ROWB + tr_pos(P, r0) * 16));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_p)(b + r1 * ROWB + tr_pos(P, r1) * 16));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// position key of a 128-byte LDS row (see above)
__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & 7; }

template <int BM_, int BN_, int NS_, int WGM_, int WGN_, int MINB_>
struct LdsCfg {
    static constexpr int BM = BM_, BN = BN_, NS = NS_, WGM = WGM_, WGN = WGN_, MINB = MINB_;
    static constexpr int NT = 64 * WGM * WGN, NW = NT / 64;
    static constexpr int WM = BM / WGM, WN = BN / WGN, TI = WM / 32, TJ = WN / 32;
    static constexpr int EPI_LD = WN + 4;
};

// Stage layout for an A of element type TA: BM rows of 64 A elements (128 or
// 256 bytes), then B: BN rows of 64 bf16 (128 bytes), or with BKN (B stored
// K-major, [K, N]) 64 k-rows of BN bf16 in the transposed-read layout of
// tr_pos; 1 KB requests.  The first half of the waves copies A (IPWA
// requests each), the second half B (IPWB each).
template <class Cfg, typename TA, bool BKN = false> struct LdsStage {
    static constexpr int AROW = 64 * (int)sizeof(TA);   // bytes of one A row
    static constexpr int APR = AROW / 16;                // 16-byte pieces per A row
    static constexpr int A_BYTES = Cfg::BM * AROW;
    static constexpr int BROW = BKN ? 2 * Cfg::BN : 128; // bytes of one B row in LDS
    static constexpr int BRQ = 1024 / BROW;              // B rows per request
    static constexpr int BYTES = A_BYTES + Cfg::BN * 128;
    static constexpr int QA = A_BYTES / 1024;            // requests for A
    static constexpr int QB = Cfg::BN * 128 / 1024;      // requests for B
    static constexpr int HW = Cfg::NW / 2;               // waves per operand
    static constexpr int IPWA = QA / HW, IPWB = QB / HW; // requests per wave per stage
    static constexpr int IPW = IPWA > IPWB ? IPWA : IPWB;
    static_assert(IPWA * HW == QA && IPWB * HW == QB, "whole 1 KB requests per wave");
    static_assert(Cfg::NW * 16 * Cfg::EPI_LD * 4 <= Cfg::NS * BYTES, "epilogue staging fits");
    static_assert(!BKN || Cfg::BN == 128 || Cfg::BN == 256, "K-major B: 128 or 256 columns");
};

// 256 x 256 tiles, 16 waves of 64 x 64, two stages: long reductions on grids
// that fill the chip (four waves per SIMD hide more of the barrier and LDS
// latency than two).  256 x 128 tiles, 8 waves of 64 x 64, three stages: long
// reductions where the large tiles would leave CUs idle but these fill them
// (N = 512).  128 x 128 tiles, 16 waves of 32 x 32, four stages (one block
// per CU): long reductions on smaller grids, where an operand streamed from
// HBM needs requests several k-tiles ahead.  128 x 128 tiles, 4 waves, two stages (two
// blocks per CU): short reductions.
typedef LdsCfg<256, 256, 2, 4, 4, 1> LdsBig;
typedef LdsCfg<256, 128, 3, 4, 2, 1> LdsMid;
typedef LdsCfg<128, 128, 4, 4, 4, 1> LdsDeep;
typedef LdsCfg<128, 128, 2, 2, 2, 2> LdsSmall;

template <class Cfg, typename TA, typename TC, bool BKN = false>
__global__ __launch_bounds__(Cfg::NT, Cfg::MINB) void gemm_lds(MM p, const TA *__restrict__ A,
                                                               const bf16_bits *__restrict__ B,
                                                               TC *__restrict__ C)
{
    typedef LdsStage<Cfg, TA, BKN> St;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, NS = Cfg::NS, IPW = St::IPW;
    constexpr int WM = Cfg::WM, WN = Cfg::WN, TI = Cfg::TI, TJ = Cfg::TJ;
    constexpr int SB = St::BYTES, AROW = St::AROW, APR = St::APR;
    __shared__ __attribute__((aligned(16))) char smem[NS * SB];

    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb, ldc = p.ldc;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
    const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;
    A += (int64_t)blockIdx.y * p.sa;
    B += (int64_t)blockIdx.y * p.sb;
    C += (int64_t)blockIdx.y * p.sc;
    const int64_t TM = (M + BM - 1) / BM, TN = (N + BN - 1) / BN;
    int64_t tm, tn;
    tile_of((int64_t)blockIdx.x, TM, TN, p.gm, &tm, &tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;
    if (p.cskip >= 0 && n0 >= p.cskip + m0 + BM) return;   // the whole block: uniform
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;    // low half of a flat LDS address

    // Request q fills 1 KB of the stage: 8 rows of A (q < QA) or of B, each
    // row's 128 bytes as eight 16-byte pieces; lane l takes piece l % 8 of row
    // l / 8, and in a row the piece at position s holds k-chunk s ^ lds_swz(row).
    // With BKN a B request is BRQ k-rows of BN columns instead: lane l takes
    // position l % (BN / 8) of k-row l / (BN / 8), which holds the piece
    // tr_piece(position, row).
    // A wave's requests are all rows of A or all rows of B, so the wave keeps
    // one uniform base (its first row, at k = 0; a scalar register pair) and a
    // 32-bit byte offset per lane and request.  Rows past M or N (columns past
    // N for BKN) repeat the last row (piece): loaded, never stored.
    static_assert(sizeof(TA) == 2 && AROW == 128, "bf16 A");
    constexpr int IPWA = St::IPWA, IPWB = St::IPWB;
    const bool isA = wave < St::HW;                      // uniform
    const int q0 = isA ? wave * IPWA : St::QA + (wave - St::HW) * IPWB;   // first request
    const char *wbase;
    uint32_t voff[IPW];
    if (BKN && !isA) {
        constexpr int BPR = Cfg::BN / 8;                 // pieces per k-row
        const int64_t r0 = (int64_t)(q0 - St::QA) * St::BRQ;   // the wave's first k-row
        wbase = (const char *)(B + r0 * ldb);
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int rr = i * St::BRQ + lane / BPR;     // k-row from the wave's first
            int64_t col = n0 + 8 * tr_piece(lane % BPR, (int)r0 + rr);
            if (col > N - 8) col = N - 8;
            voff[i] = (uint32_t)(((int64_t)rr * ldb + col) * 2);
        }
    } else {
        const int64_t r0 = isA ? q0 * 8 : (q0 - St::QA) * 8;   // the wave's first row in the tile
        const int64_t last = isA ? M - 1 - m0 : N - 1 - n0;     // last valid row in the tile
        const int64_t ld = isA ? lda : ldb;
        const int64_t rb = r0 < last ? r0 : last;
        wbase = (const char *)((isA ? A + m0 * ld : B + n0 * ld) + rb * ld);
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int row = (int)r0 + i * 8 + lane / APR;
            const int c = (lane % APR) ^ lds_swz(row);
            const int64_t rr = row < last ? row : last;
            voff[i] = (uint32_t)((rr - rb) * ld * 2 + 16 * c);
        }
    }
    int64_t KT = K / 64;
    if (p.klim >= 0) {   // k-tiles up to the last one holding k = klim + the tile's last row
        const int64_t kt_end = (p.klim + m0 + BM - 1) / 64 + 1;
        KT = kt_end < KT ? kt_end : KT;
    }
    const int64_t kstep = (BKN && !isA) ? 64 * ldb * 2 : 128;   // bytes per k-tile
    // requests of k-tile kt into stage st; past the last k-tile the last one
    // is requested again, so every iteration waits on the same count
    auto issue = [&](int64_t kt, int st) {
        const char *kb = wbase + (kt < KT ? kt : KT - 1) * kstep;
        if (isA) {
#pragma unroll
            for (int i = 0; i < IPWA; ++i)
                dma16s(kb, voff[i], lds0 + st * SB + (q0 + i) * 1024);
        } else {
#pragma unroll
            for (int i = 0; i < IPWB; ++i)
                dma16s(kb, voff[i], lds0 + st * SB + (q0 + i) * 1024);
        }
    };

    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int r32 = lane & 31, hi = lane >> 5;
    // fragment of 8 k-values (16 ks + 8 hi ..) of A row `row` / B row `row`
    auto afrag = [&](int st, int row, int ks) -> bf16x8 {
        const int c = 2 * ks + hi;
        return *(const bf16x8 *)(smem + st * SB + row * AROW + ((c ^ lds_swz(row)) << 4));
    };
    // B: rows of [N, K] (row = the column of C), or with BKN the 32 columns
    // from row - row % 32 of the K-major tile
    auto bfrag = [&](int st, int row, int ks) -> bf16x8 {
        if constexpr (BKN)
            return tr_frag<St::BROW>(smem + st * SB + St::A_BYTES, row - r32, ks, lane);
        const int c = 2 * ks + hi;
        return *(const bf16x8 *)(smem + st * SB + St::A_BYTES + row * 128 + ((c ^ lds_swz(row)) << 4));
    };

#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st, st);
    for (int64_t kt = 0; kt < KT; ++kt) {
        const int st = (int)(kt % NS);
        if (isA)                                         // this wave's share of k-tile kt
            wait_vmcnt<(NS - 2) * IPWA>();
        else
            wait_vmcnt<(NS - 2) * IPWB>();
        wait_lgkm0();                                    // and its reads of the last stage
        __builtin_amdgcn_s_barrier();
        bf16x8 a[2][TI], b[2][TJ];
        auto rd = [&](int buf, int ks) {
#pragma unroll
            for (int i = 0; i < TI; ++i) a[buf][i] = afrag(st, wm * WM + i * 32 + r32, ks);
#pragma unroll
            for (int j = 0; j < TJ; ++j) b[buf][j] = bfrag(st, wn * WN + j * 32 + r32, ks);
        };
        // the first fragments are read while the copies are issued
        rd(0, 0);
        __builtin_amdgcn_sched_barrier(0);
        issue(kt + NS - 1, (int)((kt + NS - 1) % NS));   // into the stage read last time
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int cur = ks & 1;
            if (ks < 3) rd(cur ^ 1, ks + 1);
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], b[cur][j],
                                                                        acc[i][j], 0, 0, 0);
            if (ks < 3) {   // one fragment read between groups of MFMAs
                constexpr int NF = TI + TJ, MF = TI * TJ;
#pragma unroll
                for (int t = 0; t < NF; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, MF / NF > 0 ? MF / NF : 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_vmcnt<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();

    // epilogue through LDS, one 16-row half of a 32-row band per wave at a
    // time (the 32x32 accumulator holds column lane & 31, rows
    // 8 (r / 4) + 4 (lane / 32) + r % 4: values r = 8 h .. 8 h + 7 are the
    // rows of half h)
    constexpr int EPI_LD = Cfg::EPI_LD, C4 = WN / 4;
    float *stage = (float *)smem + wave * (16 * EPI_LD);
    const int64_t nw = n0 + wn * WN;
    const bool vec = N % 4 == 0 && ldc % 4 == 0 && p.sc % 4 == 0 &&
                     ((uintptr_t)C & (4 * sizeof(TC) - 1)) == 0;
    const bool accumulate = p.accumulate;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int r = 8 * h; r < 8 * h + 8; ++r)
                    stage[(8 * (r / 4 - 2 * h) + 4 * hi + (r % 4)) * EPI_LD + j * 32 + r32] =
                        acc[i][j][r];
            const int64_t mw = m0 + wm * WM + i * 32 + 16 * h;
#pragma unroll 4
            for (int it = 0; it < 16 * C4 / 64; ++it) {
                const int idx = it * 64 + lane;
                const int row = idx / C4, c4 = idx % C4;
                const int64_t m = mw + row, n = nw + c4 * 4;
                const float4 v = *(const float4 *)(stage + row * EPI_LD + c4 * 4);
                if (m >= M) continue;
                TC *q = C + m * ldc + n;
                if constexpr (std::is_same<TC, bf16_bits>::value) {   // rounded, never accumulated
                    if (vec) {
                        if (n < N) *(u32x2 *)q = u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
                    } else {
                        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < N) q[e] = f32_to_bf16(vv[e]);
                    }
                } else if (vec) {
                    if (n < N) {
                        float4 o = v;
                        if (accumulate) {
                            const float4 c = *(const float4 *)q;
                            o.x += c.x; o.y += c.y; o.z += c.z; o.w += c.w;
                        }
                        *(float4 *)q = o;
                    }
                } else {
                    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) q[e] = accumulate ? q[e] + vv[e] : vv[e];
                }
            }
        }
    }
}

// ---- both operands K-major: C (+)= A^T B with A [K, M], B [K, N] ----------
// The weight gradient's layout (the reduction index L*B is the slow one): a
// k-tile of each operand is 64 rows of 256 columns, copied and read back as
// described at tr_pos.
// 256 x 256 tiles, 16 waves of 64 x 64, two stages.  With several splits
// block s of a tile covers k in [s ksplit, (s + 1) ksplit) and writes its
// partial product to C + s M ldc (summed in order by split_reduce).
template <class Cfg>
__global__ __launch_bounds__(Cfg::NT, Cfg::MINB) void gemm_lds_t(MM p, const bf16_bits *__restrict__ A,
                                                                 const bf16_bits *__restrict__ B,
                                                                 float *__restrict__ C)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, NW = Cfg::NW, NS = Cfg::NS;
    constexpr int WM = Cfg::WM, WN = Cfg::WN, TI = Cfg::TI, TJ = Cfg::TJ;
    static_assert(BM == 256 && BN == 256 && NS == 2, "256-column rows, two stages");
    constexpr int ROWB = 512, SA = 64 * ROWB, SB = 2 * SA, HW = NW / 2, IPW = (SA / 1024) / HW;
    static_assert(IPW * HW * 1024 == SA, "whole requests per wave");
    __shared__ __attribute__((aligned(16))) char smem[NS * SB];

    const int64_t M = p.M, N = p.N, lda = p.lda, ldb = p.ldb, ldc = p.ldc;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;
    const int64_t TM = (M + BM - 1) / BM, TN = (N + BN - 1) / BN;
    const int64_t split = (int64_t)blockIdx.x / (TM * TN);
    const int64_t kb = split * p.ksplit;
    const int64_t K = (p.K - kb) < p.ksplit ? (p.K - kb) : p.ksplit;
    C += split * M * ldc;
    int64_t tm, tn;
    tile_of((int64_t)blockIdx.x % (TM * TN), TM, TN, p.gm, &tm, &tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    // copies: waves 0 .. HW - 1 take A's requests, the others B's; request q
    // fills rows 2q, 2q + 1 of the operand's k-tile, lane l position l % 32
    // of row 2q + l / 32.  Columns past M or N repeat the last whole piece
    // (loaded, never stored).
    const bool isA = wave < HW;
    const int q0 = (isA ? wave : wave - HW) * IPW;
    const int64_t ld = isA ? lda : ldb, c0 = isA ? m0 : n0, cols = isA ? M : N;
    const char *wbase = (const char *)((isA ? A : B) + (kb + 2 * q0) * ld);
    uint32_t voff[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int row = 2 * (q0 + i) + lane / 32;
        int64_t col = c0 + 8 * tr_piece(lane % 32, row);
        if (col > cols - 8) col = cols - 8;
        voff[i] = (uint32_t)(((int64_t)(2 * i + lane / 32) * ld + col) * 2);
    }
    const uint32_t qbase = lds0 + (isA ? 0 : SA) + q0 * 1024;
    const int64_t KT = K / 64, kstep = 64 * ld * 2;
    auto issue = [&](int64_t kt, int st) {
        const char *b = wbase + (kt < KT ? kt : KT - 1) * kstep;
#pragma unroll
        for (int i = 0; i < IPW; ++i) dma16s(b, voff[i], qbase + st * SB + i * 1024);
    };

    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto frag = [&](int st, int region, int c, int ks) -> bf16x8 {
        return tr_frag<ROWB>(smem + st * SB + region, c, ks, lane);
    };

    issue(0, 0);
    for (int64_t kt = 0; kt < KT; ++kt) {
        const int st = (int)(kt & 1);
        wait_vmcnt<0>();
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        bf16x8 a[2][TI], b[2][TJ];
        auto rd = [&](int buf, int ks) {
#pragma unroll
            for (int i = 0; i < TI; ++i) a[buf][i] = frag(st, 0, wm * WM + 32 * i, ks);
#pragma unroll
            for (int j = 0; j < TJ; ++j) b[buf][j] = frag(st, SA, wn * WN + 32 * j, ks);
        };
        rd(0, 0);
        __builtin_amdgcn_sched_barrier(0);
        issue(kt + 1, st ^ 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int cur = ks & 1;
            if (ks < 3) rd(cur ^ 1, ks + 1);
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], b[cur][j],
                                                                        acc[i][j], 0, 0, 0);
            if (ks < 3) {   // the fragment reads spread among the MFMAs
                constexpr int NF = 2 * (TI + TJ), MF = TI * TJ;
#pragma unroll
                for (int t = 0; t < NF; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, MF / NF > 0 ? MF / NF : 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_vmcnt<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();

    // epilogue as gemm_lds's (16-row halves of each 32-row band through LDS)
    constexpr int EPI_LD = Cfg::EPI_LD, C4 = WN / 4;
    static_assert(NW * 16 * EPI_LD * 4 <= NS * SB, "epilogue staging fits");
    float *stage = (float *)smem + wave * (16 * EPI_LD);
    const int64_t nw = n0 + wn * WN;
    const bool vec = N % 4 == 0 && ldc % 4 == 0 && ((uintptr_t)C & 15u) == 0;
    const bool accumulate = p.accumulate;
    const int r32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int r = 8 * h; r < 8 * h + 8; ++r)
                    stage[(8 * (r / 4 - 2 * h) + 4 * hi + (r % 4)) * EPI_LD + j * 32 + r32] =
                        acc[i][j][r];
            const int64_t mw = m0 + wm * WM + i * 32 + 16 * h;
#pragma unroll 4
            for (int it = 0; it < 16 * C4 / 64; ++it) {
                const int idx = it * 64 + lane;
                const int row = idx / C4, c4 = idx % C4;
                const int64_t m = mw + row, n = nw + c4 * 4;
                const float4 v = *(const float4 *)(stage + row * EPI_LD + c4 * 4);
                if (m >= M) continue;
                float *q = C + m * ldc + n;
                if (vec) {
                    if (n < N) {
                        float4 o = v;
                        if (accumulate) {
                            const float4 c = *(const float4 *)q;
                            o.x += c.x; o.y += c.y; o.z += c.z; o.w += c.w;
                        }
                        *(float4 *)q = o;
                    }
                } else {
                    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) q[e] = accumulate ? q[e] + vv[e] : vv[e];
                }
            }
        }
    }
}

// The weight-gradient products (A as [K, M], B as [K, N]) gemm_lds_t takes:
// bf16 operands, whole 64-deep k-tiles per split, 16-byte aligned rows and
// columns in whole 16-byte pieces (M, N multiples of 8), no batches, row
// strides below 2^24 elements.
bool lds_t_ok(const GemmArgs &g)
{
    if (!g.a_bf16 || !g.b_bf16 || g.K % 64 != 0 || g.batch > 1) return false;
    const int64_t lda = g.lda ? g.lda : g.M, ldb = g.ldb ? g.ldb : g.N;
    auto al16 = [](const void *q) { return ((uintptr_t)q & 15u) == 0; };
    return g.M % 8 == 0 && g.N % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0 && al16(g.A) &&
           al16(g.Bm) && lda < (int64_t(1) << 24) && ldb < (int64_t(1) << 24);
}

// The bf16 x bf16^T products that gemm_lds takes: whole 64-deep k-tiles,
// 16-byte aligned operand rows and batch offsets, and row strides below 2^24
// elements (a wave's 64 rows then span less than 2^31 bytes: 32-bit lane
// offsets).
bool lds_path_ok(const GemmArgs &g)
{
    if (!g.a_bf16 || !g.b_bf16 || g.b_kn || g.K % 64 != 0 || g.K < 64) return false;
    const int64_t lda = g.lda ? g.lda : g.K, ldb = g.ldb ? g.ldb : g.K;
    auto al16 = [](const void *q) { return ((uintptr_t)q & 15u) == 0; };
    return lda % 8 == 0 && ldb % 8 == 0 && g.sa % 8 == 0 && g.sb % 8 == 0 && al16(g.A) &&
           al16(g.Bm) && lda < (int64_t(1) << 24) && ldb < (int64_t(1) << 24);
}

template <class Cfg, typename TA, typename TC, bool BKN = false>
hipError_t lds_launch_cfg(const GemmArgs &g, hipStream_t s)
{
    MM p;
    p.M = g.M;
    p.N = g.N;
    p.K = g.K;
    p.lda = g.lda ? g.lda : g.K;
    p.ldb = g.ldb ? g.ldb : (BKN ? g.N : g.K);
    p.ldc = g.ldc ? g.ldc : g.N;
    p.sa = g.sa;
    p.sb = g.sb;
    p.sc = g.sc;
    p.ksplit = g.K;
    p.gm = (int)group_rows(g.M, g.N, Cfg::BM, Cfg::BN);
    p.accumulate = g.accumulate;
    p.cskip = g.causal_skip;
    p.klim = g.causal_klim;
    const int64_t tiles = ((g.M + Cfg::BM - 1) / Cfg::BM) * ((g.N + Cfg::BN - 1) / Cfg::BN);
    hipLaunchKernelGGL((gemm_lds<Cfg, TA, TC, BKN>),
                       dim3((unsigned)tiles, (unsigned)(g.batch > 0 ? g.batch : 1)),
                       dim3(Cfg::NT), 0, s, p, (const TA *)g.A, (const bf16_bits *)g.Bm, (TC *)g.C);
    return hipGetLastError();
}

#ifndef SRU_LDS_BIG_MIN_K
#define SRU_LDS_BIG_MIN_K 512
#endif

template <typename TA, typename TC, bool BKN = false>
hipError_t lds_launch_t(const GemmArgs &g, hipStream_t s)
{
    // the large tiles once they give every CU one and the reduction is long
    // enough to amortise their prologue and epilogue (from K = 512: the SRU++
    // output projection at K = d' = 512, L*B = 16384, 3d = 6144 runs about
    // 30 us faster on them than on the small tiles); deep small tiles for
    // other long reductions; two small blocks per CU for short ones
    const int64_t nb = g.batch > 0 ? g.batch : 1;
    const int64_t big = ((g.M + 255) / 256) * ((g.N + 255) / 256) * nb;
    const int64_t mid = ((g.M + 255) / 256) * ((g.N + 127) / 128) * nb;
    if (g.K >= SRU_LDS_BIG_MIN_K && big >= 256) return lds_launch_cfg<LdsBig, TA, TC, BKN>(g, s);
    if (g.K >= 1024 && mid >= 256 && mid % 256 == 0)
        return lds_launch_cfg<LdsMid, TA, TC, BKN>(g, s);
    if (g.K >= 1024) return lds_launch_cfg<LdsDeep, TA, TC, BKN>(g, s);
    return lds_launch_cfg<LdsSmall, TA, TC, BKN>(g, s);
}

hipError_t lds_launch(const GemmArgs &g, hipStream_t s) { return lds_launch_t<bf16_bits, float>(g, s); }

// bf16 A (K-contiguous) times a bf16 B given as [K, N]: whole 64-deep
// k-tiles, 16-byte aligned rows and batch offsets, N a multiple of 8 (whole
// 16-byte pieces of a k-row), row strides below 2^24 elements.
#ifndef SRU_LDS_KN
#define SRU_LDS_KN 1
#endif
bool lds_kn_path_ok(const GemmArgs &g)
{
    if (!SRU_LDS_KN || !g.a_bf16 || !g.b_bf16 || !g.b_kn || g.K % 64 != 0 || g.K < 64 ||
        g.N % 8 != 0)
        return false;
    const int64_t lda = g.lda ? g.lda : g.K, ldb = g.ldb ? g.ldb : g.N;
    auto al16 = [](const void *q) { return ((uintptr_t)q & 15u) == 0; };
    return lda % 8 == 0 && ldb % 8 == 0 && g.sa % 8 == 0 && g.sb % 8 == 0 && al16(g.A) &&
           al16(g.Bm) && lda < (int64_t(1) << 24) && ldb < (int64_t(1) << 24);
}

// dst[i] = bf16(src[i]) (nearest even), four elements per lane and step.
__global__ __launch_bounds__(256) void round_bf16_kernel(int64_t n, const float *__restrict__ src,
                                                         bf16_bits *__restrict__ dst)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += stride) {
        if (i + 4 <= n) {
            const float4 v = *(const float4 *)(src + i);
            *(u32x2 *)(dst + i) = u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
        } else {
            for (int64_t e = i; e < n; ++e) dst[e] = f32_to_bf16(src[e]);
        }
    }
}

// dst[c][r] = src[r][c] for a rows x cols matrix of 2-byte elements, one
// 64 x 64 tile per block.  VEC (rows % 8 == 0 and cols % 8 == 0): every
// global access moves 16 bytes (8 elements of a row in, 8 of a column out)
// and the tile is turned in LDS; otherwise element by element.  The LDS row
// of 66 elements (33 dwords) spreads the column gathers over the banks.
template <bool VEC>
__global__ __launch_bounds__(256) void transpose16(int64_t rows, int64_t cols,
                                                   const uint16_t *__restrict__ src,
                                                   uint16_t *__restrict__ dst)
{
    __shared__ uint16_t t[64][66];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    if constexpr (VEC) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int id = tid + 256 * h, row = id >> 3, cc = (id & 7) * 8;
            const int64_t r = r0 + row, c = c0 + cc;
            if (r < rows && c < cols) {   // whole 8-element chunks: cols % 8 == 0
                const uint4 v = *(const uint4 *)(src + r * cols + c);
                uint32_t *tp = (uint32_t *)&t[row][cc];
                tp[0] = v.x;
                tp[1] = v.y;
                tp[2] = v.z;
                tp[3] = v.w;
            }
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int id = tid + 256 * h, oc = id >> 3, rr = (id & 7) * 8;
            const int64_t c = c0 + oc, r = r0 + rr;
            if (c < cols && r < rows) {   // rows % 8 == 0
                uint32_t w[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    w[k] = uint32_t(t[rr + 2 * k][oc]) | (uint32_t(t[rr + 2 * k + 1][oc]) << 16);
                *(uint4 *)(dst + c * rows + r) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    } else {
        const int tx = tid & 63, ty = tid >> 6;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int64_t r = r0 + ty * 16 + k, c = c0 + tx;
            if (r < rows && c < cols) t[ty * 16 + k][tx] = src[r * cols + c];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int64_t c = c0 + ty * 16 + k, r = r0 + tx;
            if (r < rows && c < cols) dst[c * rows + r] = t[tx][ty * 16 + k];
        }
    }
}

__global__ __launch_bounds__(256) void transpose32(int64_t rows, int64_t cols,
                                                   const float *__restrict__ src,
                                                   float *__restrict__ dst)
{
    __shared__ float t[64][65];
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int64_t r = r0 + ty * 16 + k, c = c0 + tx;
        if (r < rows && c < cols) t[ty * 16 + k][tx] = src[r * cols + c];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int64_t c = c0 + ty * 16 + k, r = r0 + tx;
        if (r < rows && c < cols) dst[c * rows + r] = t[tx][ty * 16 + k];
    }
}

// ---- fp32 path ------------------------------------------------------------
constexpr int FT = 64, FK = 16;

// A as [M, K] or, with AKM, [K, M]; B as [N, K] or, with KN, [K, N]; row
// strides and batch offsets as in MM.
template <typename TA, bool AKM, typename TB, bool KN>
__global__ __launch_bounds__(256) void gemm_f32(MM p, const TA *__restrict__ A,
                                                const TB *__restrict__ Bm,
                                                float *__restrict__ C)
{
    __shared__ float As[FK][FT + 4];
    __shared__ float Bs[FK][FT + 4];
    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    A += (int64_t)blockIdx.z * p.sa;
    Bm += (int64_t)blockIdx.z * p.sb;
    C += (int64_t)blockIdx.z * p.sc;
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * FT, n0 = (int64_t)blockIdx.y * FT;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += FK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + i * 256;      // 0 .. 1023 = FT x FK
            if (!AKM) {  // A[m][k] -> As[k][m]
                const int r = idx / FK, kk = idx % FK;
                const int64_t m = m0 + r, k = k0 + kk;
                As[kk][r] = (m < M && k < K) ? load_as_f32(A + m * lda + k) : 0.0f;
            } else {     // A[k][m] -> As[k][m]
                const int kk = idx / FT, r = idx % FT;
                const int64_t m = m0 + r, k = k0 + kk;
                As[kk][r] = (m < M && k < K) ? load_as_f32(A + k * lda + m) : 0.0f;
            }
            if (!KN) {  // B[n][k] -> Bs[k][n]
                const int r = idx / FK, kk = idx % FK;
                const int64_t n = n0 + r, k = k0 + kk;
                Bs[kk][r] = (n < N && k < K) ? load_as_f32(Bm + n * ldb + k) : 0.0f;
            } else {    // B[k][n] -> Bs[k][n]
                const int kk = idx / FT, r = idx % FT;
                const int64_t n = n0 + r, k = k0 + kk;
                Bs[kk][r] = (n < N && k < K) ? load_as_f32(Bm + k * ldb + n) : 0.0f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < FK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            if (n >= N) continue;
            float *q = C + m * p.ldc + n;
            *q = p.accumulate ? *q + acc[i][j] : acc[i][j];
        }
    }
}

// splits > 1: partial products to ws ([splits, M, N], dense), k-range per
// split ksplit (a multiple of the k-tile; one batch only); otherwise
// straight into C.
template <class Cfg, typename TA, bool AKM, typename TB, bool KN, typename TC = float>
hipError_t mfma_launch_cfg(const GemmArgs &g, hipStream_t s, int64_t splits = 1,
                           int64_t ksplit = 0, float *ws = nullptr)
{
    MM p;
    p.M = g.M;
    p.N = g.N;
    p.K = g.K;
    p.lda = g.lda ? g.lda : (AKM ? g.M : g.K);
    p.ldb = g.ldb ? g.ldb : (KN ? g.N : g.K);
    p.ldc = g.ldc ? g.ldc : g.N;
    p.sa = g.sa;
    p.sb = g.sb;
    p.sc = g.sc;
    p.gm = (int)group_rows(g.M, g.N, Cfg::BM, Cfg::BN);
    p.ksplit = splits > 1 ? ksplit : g.K;
    p.accumulate = splits > 1 ? false : g.accumulate;
    const int64_t batch = g.batch > 0 ? g.batch : 1;
    TC *C = (TC *)g.C;
    if (splits > 1) {
        C = (TC *)ws;
        p.ldc = g.N;
        p.sc = 0;
    }
    // fast variant: whole k-tiles; 4-aligned C rows and batch offsets;
    // row-major operands with 16-byte aligned rows and offsets and a k-tile
    // window below 2^32 bytes; K-major operands with even strides, row
    // counts and offsets (row pairs load aligned)
    constexpr int64_t kWin = int64_t(1) << 32;
    auto row_ok = [&](int64_t ld, int64_t off, int rows, int64_t es) {
        const int64_t v = 16 / es;
        return ld % v == 0 && off % v == 0 && ld * rows * es < kWin;
    };
    auto kmaj_ok = [&](int64_t ld, int64_t rows, int64_t off, int64_t es) {
        return ld % 2 == 0 && rows % 2 == 0 && off % 2 == 0 && ld * Cfg::BK * es < kWin;
    };
    auto al16 = [](const void *q) { return ((uintptr_t)q & 15u) == 0; };
    const bool fast =
        al16(g.A) && al16(g.Bm) && al16(C) &&
        g.K % Cfg::BK == 0 && g.N % 4 == 0 && p.ldc % 4 == 0 && p.sc % 4 == 0 &&
        (AKM ? kmaj_ok(p.lda, g.M, p.sa, sizeof(TA)) : row_ok(p.lda, p.sa, Cfg::BM, sizeof(TA))) &&
        (KN ? kmaj_ok(p.ldb, g.N, p.sb, sizeof(TB)) : row_ok(p.ldb, p.sb, Cfg::BN, sizeof(TB)));
    if (fast) {
        const int64_t tiles = ((g.M + Cfg::BM - 1) / Cfg::BM) * ((g.N + Cfg::BN - 1) / Cfg::BN);
        hipLaunchKernelGGL((gemm_bf16_mfma<Cfg, TA, AKM, TB, KN, true, TC>),
                           dim3((unsigned)(tiles * splits), (unsigned)batch), dim3(Cfg::NT), 0, s,
                           p, (const TA *)g.A, (const TB *)g.Bm, C);
    } else {
        // bounds-checked loads: one register stage, 128 x 128 tiles
        const int64_t t1 = ((g.M + CfgSmall::BM - 1) / CfgSmall::BM) *
                           ((g.N + CfgSmall::BN - 1) / CfgSmall::BN);
        hipLaunchKernelGGL((gemm_bf16_mfma<CfgSmall, TA, AKM, TB, KN, false, TC>),
                           dim3((unsigned)(t1 * splits), (unsigned)batch), dim3(CfgSmall::NT), 0,
                           s, p, (const TA *)g.A, (const TB *)g.Bm, C);
    }
    return hipGetLastError();
}

int64_t tiles_of(const GemmArgs &g, int bm, int bn)
{
    return ((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn) * (g.batch > 0 ? g.batch : 1);
}

template <typename TA, bool KN, typename TC = float>
hipError_t mfma_launch(const GemmArgs &g, hipStream_t s)
{
    // large tiles once they give every CU (256) at least one
    const int64_t big = tiles_of(g, 256, 256), wide = tiles_of(g, 256, 192);
    if constexpr (!KN) {   // B as [N, K]
        if (SRU_GEMM_WIDE && big >= 256 && big % 256 != 0 && wide % 256 == 0)
            return mfma_launch_cfg<CfgWide8, TA, false, bf16_bits, KN, TC>(g, s);
    }
    if (big >= 256)
        return mfma_launch_cfg<CfgBig8, TA, false, bf16_bits, KN, TC>(g, s);
    if constexpr (sizeof(TA) == 2 && !KN)
        return mfma_launch_cfg<CfgSmallDeep, TA, false, bf16_bits, KN, TC>(g, s);
    return mfma_launch_cfg<CfgSmall, TA, false, bf16_bits, KN, TC>(g, s);
}

// C = P[0] + P[1] + ... + P[splits - 1] (+ C first when accumulating), the
// partial products added in split order: the result does not depend on
// scheduling.
__global__ __launch_bounds__(256) void split_reduce(const float *__restrict__ P, int64_t n,
                                                    int64_t splits, float *__restrict__ C,
                                                    bool accumulate)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float sum = P[i];
    for (int64_t s = 1; s < splits; ++s) sum += P[s * n + i];
    C[i] = accumulate ? C[i] + sum : sum;
}

// Tiles and split of the reduction over L*B for the weight gradient.  A
// block takes one of the resident slots (128 x 128 tiles: 512, two per CU;
// 256 x 256 tiles: 256, one per CU), and a launch of n blocks runs in
// ceil(n / slots) rounds, each as long as one block's k-tiles.  A k-tile
// round moves the same operand bytes per CU in both configurations (~1.6 us
// measured), so the large tiles cover four times the output per round.  The
// partial sums cost a write and a read of M x N floats per split; at ~5 TB/s
// that is M*N/1e6 k-tile rounds per split.  Pick the configuration and split
// count with the least total (ties: the small tiles, fewer splits), at least
// 8 k-tiles per split.
constexpr int64_t kWgradMinKt = 8, kWgradMaxSplits = 64;

struct WgradPlan {
    bool big;          // 256 x 256 tiles
    int64_t splits;    // 1: no partial sums
};

WgradPlan wgrad_plan(int64_t M, int64_t N, int64_t K)
{
    const int64_t kt = K / 64;                           // both configurations: 64-deep k-tiles
    if (K % 64 != 0 || kt < 2 * kWgradMinKt) return {false, 1};
    const double reduce = (double)M * (double)N * 1e-6;
    WgradPlan best{false, 1};
    double best_cost = -1.0;
    for (int big = 0; big < 2; ++big) {
        const int64_t t = big ? 256 : 128, slots = big ? 256 : 512;
        const int64_t tiles = ((M + t - 1) / t) * ((N + t - 1) / t);
        for (int64_t sp = 1; sp <= kt / kWgradMinKt && sp <= kWgradMaxSplits; ++sp) {
            const double rounds = (double)((tiles * sp + slots - 1) / slots);
            const double cost = rounds * (double)((kt + sp - 1) / sp) + (sp > 1 ? reduce * sp : 0.0);
            if (best_cost < 0.0 || cost < best_cost) {
                best_cost = cost;
                best = {big != 0, sp};
            }
        }
    }
    return best;
}

// The weight gradient on the K-major LDS-copy kernel (256 x 256 tiles);
// splits as mfma_launch_cfg's.
hipError_t lds_t_launch(const GemmArgs &g, hipStream_t s, int64_t splits, int64_t ksplit,
                        float *ws)
{
    MM p;
    p.M = g.M;
    p.N = g.N;
    p.K = g.K;
    p.lda = g.lda ? g.lda : g.M;
    p.ldb = g.ldb ? g.ldb : g.N;
    p.ldc = g.ldc ? g.ldc : g.N;
    p.sa = p.sb = p.sc = 0;
    p.gm = 8;
    p.ksplit = splits > 1 ? ksplit : g.K;
    p.accumulate = splits > 1 ? false : g.accumulate;
    float *C = g.C;
    if (splits > 1) {
        C = ws;
        p.ldc = g.N;
    }
    const int64_t tiles = ((g.M + 255) / 256) * ((g.N + 255) / 256) * (splits > 1 ? splits : 1);
    hipLaunchKernelGGL((gemm_lds_t<LdsBig>), dim3((unsigned)tiles), dim3(LdsBig::NT), 0, s, p,
                       (const bf16_bits *)g.A, (const bf16_bits *)g.Bm, C);
    return hipGetLastError();
}

template <class Cfg, typename TA, typename TB>
hipError_t wgrad_launch_cfg(const GemmArgs &g, int64_t sp, float *ws, hipStream_t s)
{
    // bf16 operands on the 256 x 256 plan: the LDS-copy kernel
    constexpr bool lds_t = std::is_same<TA, bf16_bits>::value &&
                           std::is_same<TB, bf16_bits>::value && Cfg::BM == 256 && Cfg::BN == 256;
    const bool use_t = lds_t && lds_t_ok(g);
    if (sp <= 1) return use_t ? lds_t_launch(g, s, 1, 0, nullptr)
                              : mfma_launch_cfg<Cfg, TA, true, TB, true>(g, s);
    const int64_t kt = g.K / Cfg::BK;
    const int64_t ksplit = ((kt + sp - 1) / sp) * Cfg::BK;
    const int64_t used = (g.K + ksplit - 1) / ksplit;      // splits with work
    hipError_t e = use_t ? lds_t_launch(g, s, used, ksplit, ws)
                         : mfma_launch_cfg<Cfg, TA, true, TB, true>(g, s, used, ksplit, ws);
    if (e != hipSuccess) return e;
    const int64_t n = g.M * g.N;
    hipLaunchKernelGGL(split_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ws, n,
                       used, g.C, g.accumulate);
    return hipGetLastError();
}

template <typename TA, typename TB>
hipError_t wgrad_launch(const GemmArgs &g, float *ws, hipStream_t s)
{
    const WgradPlan pl = wgrad_plan(g.M, g.N, g.K);
    return pl.big ? wgrad_launch_cfg<CfgBig8, TA, TB>(g, pl.splits, ws, s)
                  : wgrad_launch_cfg<CfgSmall, TA, TB>(g, pl.splits, ws, s);
}

template <typename TA, bool AKM, typename TB, bool KN>
hipError_t f32_launch(const GemmArgs &g, hipStream_t s)
{
    MM p;
    p.M = g.M;
    p.N = g.N;
    p.K = g.K;
    p.lda = g.lda ? g.lda : (AKM ? g.M : g.K);
    p.ldb = g.ldb ? g.ldb : (KN ? g.N : g.K);
    p.ldc = g.ldc ? g.ldc : g.N;
    p.sa = g.sa;
    p.sb = g.sb;
    p.sc = g.sc;
    p.ksplit = g.K;
    p.gm = 1;
    p.accumulate = g.accumulate;
    dim3 grid((unsigned)((g.M + FT - 1) / FT), (unsigned)((g.N + FT - 1) / FT),
              (unsigned)(g.batch > 0 ? g.batch : 1));
    hipLaunchKernelGGL((gemm_f32<TA, AKM, TB, KN>), grid, dim3(256), 0, s, p, (const TA *)g.A,
                       (const TB *)g.Bm, g.C);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_round_bf16(int64_t n, const float *src, void *dst, hipStream_t s)
{
    const int64_t blocks = (n + 1023) / 1024;
    hipLaunchKernelGGL(round_bf16_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)),
                       dim3(256), 0, s, n, src, (bf16_bits *)dst);
    return hipGetLastError();
}

hipError_t launch_transpose(int64_t rows, int64_t cols, const void *src, void *dst, bool two_byte,
                            hipStream_t s)
{
    dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
    if (two_byte && rows % 8 == 0 && cols % 8 == 0)
        hipLaunchKernelGGL((transpose16<true>), grid, dim3(256), 0, s, rows, cols,
                           (const uint16_t *)src, (uint16_t *)dst);
    else if (two_byte)
        hipLaunchKernelGGL((transpose16<false>), grid, dim3(256), 0, s, rows, cols,
                           (const uint16_t *)src, (uint16_t *)dst);
    else
        hipLaunchKernelGGL(transpose32, grid, dim3(256), 0, s, rows, cols, (const float *)src,
                           (float *)dst);
    return hipGetLastError();
}

size_t wgrad_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    const int64_t sp = wgrad_plan(M, N, K).splits;
    return sp <= 1 ? 0 : (size_t)(sp * M * N) * sizeof(float);
}

size_t wgrad_b_copy_bytes(int64_t M, int64_t N, int64_t K)
{
    const WgradPlan pl = wgrad_plan(M, N, K);
    if (!pl.big || M % 8 != 0 || N % 8 != 0 || K % 64 != 0) return 0;
    return ((size_t)K * (size_t)N * 2 + 255) & ~(size_t)255;
}

hipError_t launch_gemm_wgrad(const GemmArgs &g, bool f32_math, float *ws, hipStream_t s,
                             bool b_copy)
{
    // bf16 A, fp32 B: B rounded into the workspace (after the partial sums)
    // gives the bf16 operands the K-major LDS-copy kernel takes, with the
    // values the product would round B to as it loads it
    if (b_copy && !f32_math && g.a_bf16 && !g.b_bf16 && ws && g.batch <= 1 &&
        (g.ldb == 0 || g.ldb == g.N) && wgrad_b_copy_bytes(g.M, g.N, g.K) > 0) {
        const size_t part = (wgrad_workspace_bytes(g.M, g.N, g.K) + 255) & ~(size_t)255;
        bf16_bits *Bb = (bf16_bits *)((char *)ws + part);
        hipError_t e = launch_round_bf16(g.K * g.N, (const float *)g.Bm, Bb, s);
        if (e != hipSuccess) return e;
        GemmArgs g2 = g;
        g2.Bm = Bb, g2.b_bf16 = true, g2.ldb = g.N;
        return wgrad_launch<bf16_bits, bf16_bits>(g2, ws, s);
    }
    if (f32_math) {
        if (g.a_bf16)
            return g.b_bf16 ? f32_launch<bf16_bits, true, bf16_bits, true>(g, s)
                            : f32_launch<bf16_bits, true, float, true>(g, s);
        return g.b_bf16 ? f32_launch<float, true, bf16_bits, true>(g, s)
                        : f32_launch<float, true, float, true>(g, s);
    }
    if (g.a_bf16)
        return g.b_bf16 ? wgrad_launch<bf16_bits, bf16_bits>(g, ws, s)
                        : wgrad_launch<bf16_bits, float>(g, ws, s);
    return g.b_bf16 ? wgrad_launch<float, bf16_bits>(g, ws, s) : wgrad_launch<float, float>(g, ws, s);
}

namespace {
template <typename TA, typename TB, typename TC = float>
hipError_t tn_launch(const GemmArgs &g, hipStream_t s)
{
    if (tiles_of(g, 256, 256) >= 256)
        return mfma_launch_cfg<CfgBig8, TA, true, TB, true, TC>(g, s);
    return mfma_launch_cfg<CfgSmall, TA, true, TB, true, TC>(g, s);
}
}  // namespace

hipError_t launch_gemm_tn(const GemmArgs &g, hipStream_t s)
{
    if (g.a_bf16)
        return g.b_bf16 ? tn_launch<bf16_bits, bf16_bits>(g, s) : tn_launch<bf16_bits, float>(g, s);
    return g.b_bf16 ? tn_launch<float, bf16_bits>(g, s) : tn_launch<float, float>(g, s);
}

hipError_t launch_gemm_tn_bf16_out(const GemmArgs &g, hipStream_t s)
{
    if (!g.a_bf16 || !g.b_bf16 || g.accumulate) return hipErrorInvalidValue;
    return tn_launch<bf16_bits, bf16_bits, bf16_bits>(g, s);
}

hipError_t launch_gemm_bf16_out(const GemmArgs &g, hipStream_t s)
{
    if (!g.b_bf16 || g.b_kn || g.accumulate) return hipErrorInvalidValue;
    if (g.a_bf16) {
        if (lds_path_ok(g)) return lds_launch_t<bf16_bits, bf16_bits>(g, s);
        return mfma_launch<bf16_bits, false, bf16_bits>(g, s);
    }
    return mfma_launch<float, false, bf16_bits>(g, s);
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t s)
{
    if (g.b_bf16) {
        if (lds_path_ok(g)) return lds_launch(g, s);
        if (lds_kn_path_ok(g)) return lds_launch_t<bf16_bits, float, true>(g, s);
        if (g.a_bf16)
            return g.b_kn ? mfma_launch<bf16_bits, true>(g, s) : mfma_launch<bf16_bits, false>(g, s);
        return g.b_kn ? mfma_launch<float, true>(g, s) : mfma_launch<float, false>(g, s);
    }
    if (g.a_bf16)
        return g.b_kn ? f32_launch<bf16_bits, false, float, true>(g, s)
                      : f32_launch<bf16_bits, false, float, false>(g, s);
    return g.b_kn ? f32_launch<float, false, float, true>(g, s)
                  : f32_launch<float, false, float, false>(g, s);
}

}  // namespace sru
