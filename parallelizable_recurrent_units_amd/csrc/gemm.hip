// gemm.hip -- the projection of Eq. 1 (SRU++ paper, background section):
// the three gate matrices of all timesteps (and both directions) in one
// GEMM, U = X~ W^T, and its input gradient dX = dU W.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 (gfx950) with fp32 accumulation.  The
// A operand may arrive as fp32; it is rounded to bf16 (nearest even) while
// it is staged into LDS, so no separate conversion pass touches HBM.
// W is bf16 in HBM and is used either as [N, K] (forward: C = A W^T, both
// operands K-contiguous) or as [K, N] (backward-data: C = A W, W is
// transposed while it is staged into LDS).
//
// fp32 path (W in fp32): LDS-tiled FMA kernel, fp32 products and sums.
#include "device_common.h"
#include "internal.h"

namespace sru {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDK = BK + 8;   // padded LDS row (bf16 elements): 80 bytes
constexpr int NT = 256;       // 4 waves, 2 x 2, each 64 x 64

struct alignas(16) Bf16x8 { bf16_bits v[8]; };

// ---- A tile loader: BM x BK, into registers then LDS ----------------------
template <typename TA, bool VEC>
struct ALoader {
    // fp32: 4 float4 per thread; bf16: 2 x (8 bf16) per thread
    static constexpr int N = sizeof(TA) == 4 ? 4 : 2;
    uint4 reg[N];
    __device__ void load(const TA *A, int64_t M, int64_t K, int64_t m0, int64_t k0, int tid)
    {
        constexpr int V = 16 / sizeof(TA);          // elements per 16 bytes
        constexpr int PER_ROW = BK / V;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT;
            const int row = idx / PER_ROW, cv = idx % PER_ROW;
            const int64_t m = m0 + row, k = k0 + cv * V;
            if (VEC) {
                if (m < M && k < K)
                    reg[i] = *(const uint4 *)(A + m * K + k);
                else
                    reg[i] = make_uint4(0, 0, 0, 0);
            } else {
                TA tmp[V];
#pragma unroll
                for (int e = 0; e < V; ++e)
                    tmp[e] = (m < M && k + e < K) ? A[m * K + k + e] : TA(0);
                reg[i] = *(const uint4 *)tmp;
            }
        }
    }
    __device__ void store(bf16_bits *As, int tid) const
    {
        constexpr int V = 16 / sizeof(TA);
        constexpr int PER_ROW = BK / V;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT;
            const int row = idx / PER_ROW, cv = idx % PER_ROW;
            bf16_bits *dst = As + row * LDK + cv * V;
            if (sizeof(TA) == 4) {
                const float4 f = *(const float4 *)&reg[i];
                uint2 packed;
                packed.x = uint32_t(f32_to_bf16(f.x)) | (uint32_t(f32_to_bf16(f.y)) << 16);
                packed.y = uint32_t(f32_to_bf16(f.z)) | (uint32_t(f32_to_bf16(f.w)) << 16);
                *(uint2 *)dst = packed;
            } else {
                *(uint4 *)dst = reg[i];
            }
        }
    }
};

// ---- B tile loader: produces Bs[n][k] (BN x BK) ---------------------------
template <bool KN, bool VEC>
struct BLoader {
    uint4 reg[2];
    __device__ void load(const bf16_bits *Bm, int64_t N, int64_t K, int64_t n0, int64_t k0,
                         int tid)
    {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + i * NT;
            if (!KN) {  // B[n][k], 4 x 8 bf16 per row of BK
                const int row = idx / 4, cv = idx % 4;
                const int64_t n = n0 + row, k = k0 + cv * 8;
                if (VEC) {
                    reg[i] = (n < N && k < K) ? *(const uint4 *)(Bm + n * K + k)
                                              : make_uint4(0, 0, 0, 0);
                } else {
                    bf16_bits tmp[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        tmp[e] = (n < N && k + e < K) ? Bm[n * K + k + e] : bf16_bits(0);
                    reg[i] = *(const uint4 *)tmp;
                }
            } else {    // B[k][n], BK rows of BN: 16 x 8 bf16 per row
                const int kr = idx / 16, cv = idx % 16;
                const int64_t k = k0 + kr, n = n0 + cv * 8;
                if (VEC) {
                    reg[i] = (k < K && n < N) ? *(const uint4 *)(Bm + k * N + n)
                                              : make_uint4(0, 0, 0, 0);
                } else {
                    bf16_bits tmp[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        tmp[e] = (k < K && n + e < N) ? Bm[k * N + n + e] : bf16_bits(0);
                    reg[i] = *(const uint4 *)tmp;
                }
            }
        }
    }
    __device__ void store(bf16_bits *Bs, int tid) const
    {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + i * NT;
            if (!KN) {
                const int row = idx / 4, cv = idx % 4;
                *(uint4 *)(Bs + row * LDK + cv * 8) = reg[i];
            } else {
                const int kr = idx / 16, cv = idx % 16;
                const bf16_bits *v = (const bf16_bits *)&reg[i];
#pragma unroll
                for (int e = 0; e < 8; ++e) Bs[(cv * 8 + e) * LDK + kr] = v[e];
            }
        }
    }
};

// C[M, N] (+)= A[M, K] . B  with B given as [N, K] (KN = false) or [K, N].
template <typename TA, bool KN, bool AVEC, bool BVEC>
__global__ __launch_bounds__(NT) void gemm_bf16_mfma(int64_t M, int64_t N, int64_t K,
                                                     const TA *__restrict__ A,
                                                     const bf16_bits *__restrict__ Bm,
                                                     float *__restrict__ C, bool accumulate)
{
    __shared__ __attribute__((aligned(16))) bf16_bits As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) bf16_bits Bs[2][BN * LDK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    const int64_t n0 = (int64_t)blockIdx.y * BN;

    ALoader<TA, AVEC> la;
    BLoader<KN, BVEC> lb;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t KT = (K + BK - 1) / BK;
    la.load(A, M, K, m0, 0, tid);
    lb.load(Bm, N, K, n0, 0, tid);
    la.store(As[0], tid);
    lb.store(Bs[0], tid);
    __syncthreads();

    const int r32 = lane & 31;
    const int kg = (lane >> 5) * 8;
    for (int64_t kt = 0; kt < KT; ++kt) {
        const int buf = (int)(kt & 1);
        if (kt + 1 < KT) {
            la.load(A, M, K, m0, (kt + 1) * BK, tid);
            lb.load(Bm, N, K, n0, (kt + 1) * BK, tid);
        }
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *(const bf16x8 *)(As[buf] + (wm * 64 + i * 32 + r32) * LDK + ks * 16 + kg);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = *(const bf16x8 *)(Bs[buf] + (wn * 64 + j * 32 + r32) * LDK + ks * 16 + kg);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (kt + 1 < KT) {
            la.store(As[buf ^ 1], tid);
            lb.store(Bs[buf ^ 1], tid);
        }
        __syncthreads();
    }

    // 32x32 accumulator layout: lane holds column (lane & 31) and rows
    // 8*(r/4) + 4*(lane/32) + (r%4), r = 0..15.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + r32;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
                if (row < M) {
                    float *p = C + row * N + col;
                    *p = accumulate ? *p + acc[i][j][r] : acc[i][j][r];
                }
            }
        }
}

// ---- fp32 path ------------------------------------------------------------
constexpr int FT = 64, FK = 16;

template <typename TA, bool KN>
__global__ __launch_bounds__(256) void gemm_f32(int64_t M, int64_t N, int64_t K,
                                                const TA *__restrict__ A,
                                                const float *__restrict__ Bm,
                                                float *__restrict__ C, bool accumulate)
{
    __shared__ float As[FK][FT + 4];
    __shared__ float Bs[FK][FT + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * FT, n0 = (int64_t)blockIdx.y * FT;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += FK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + i * 256;      // 0 .. 1023 = FT x FK
            {   // A[m][k] -> As[k][m]
                const int r = idx / FK, kk = idx % FK;
                const int64_t m = m0 + r, k = k0 + kk;
                As[kk][r] = (m < M && k < K) ? load_as_f32(A + m * K + k) : 0.0f;
            }
            if (!KN) {  // B[n][k] -> Bs[k][n]
                const int r = idx / FK, kk = idx % FK;
                const int64_t n = n0 + r, k = k0 + kk;
                Bs[kk][r] = (n < N && k < K) ? Bm[n * K + k] : 0.0f;
            } else {    // B[k][n] -> Bs[k][n]
                const int kk = idx / FT, r = idx % FT;
                const int64_t n = n0 + r, k = k0 + kk;
                Bs[kk][r] = (n < N && k < K) ? Bm[k * N + n] : 0.0f;
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
            float *p = C + m * N + n;
            *p = accumulate ? *p + acc[i][j] : acc[i][j];
        }
    }
}

template <typename TA, bool KN, bool AVEC, bool BVEC>
hipError_t mfma_launch(const GemmArgs &g, hipStream_t s)
{
    dim3 grid((unsigned)((g.M + BM - 1) / BM), (unsigned)((g.N + BN - 1) / BN));
    hipLaunchKernelGGL((gemm_bf16_mfma<TA, KN, AVEC, BVEC>), grid, dim3(NT), 0, s, g.M, g.N, g.K,
                       (const TA *)g.A, (const bf16_bits *)g.Bm, g.C, g.accumulate);
    return hipGetLastError();
}

template <typename TA, bool KN>
hipError_t mfma_dispatch_vec(const GemmArgs &g, hipStream_t s)
{
    const int64_t va = 16 / sizeof(TA);
    const bool avec = (g.K % va) == 0;
    const bool bvec = KN ? (g.N % 8 == 0) : (g.K % 8 == 0);
    if (avec && bvec) return mfma_launch<TA, KN, true, true>(g, s);
    if (avec) return mfma_launch<TA, KN, true, false>(g, s);
    if (bvec) return mfma_launch<TA, KN, false, true>(g, s);
    return mfma_launch<TA, KN, false, false>(g, s);
}

template <typename TA, bool KN>
hipError_t f32_launch(const GemmArgs &g, hipStream_t s)
{
    dim3 grid((unsigned)((g.M + FT - 1) / FT), (unsigned)((g.N + FT - 1) / FT));
    hipLaunchKernelGGL((gemm_f32<TA, KN>), grid, dim3(256), 0, s, g.M, g.N, g.K,
                       (const TA *)g.A, (const float *)g.Bm, g.C, g.accumulate);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs &g, hipStream_t s)
{
    if (g.b_bf16) {
        if (g.a_bf16)
            return g.b_kn ? mfma_dispatch_vec<bf16_bits, true>(g, s)
                          : mfma_dispatch_vec<bf16_bits, false>(g, s);
        return g.b_kn ? mfma_dispatch_vec<float, true>(g, s)
                      : mfma_dispatch_vec<float, false>(g, s);
    }
    if (g.a_bf16)
        return g.b_kn ? f32_launch<bf16_bits, true>(g, s) : f32_launch<bf16_bits, false>(g, s);
    return g.b_kn ? f32_launch<float, true>(g, s) : f32_launch<float, false>(g, s);
}

}  // namespace sru
