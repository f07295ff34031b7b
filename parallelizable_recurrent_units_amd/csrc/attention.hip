// attention.hip -- the U-producer of an SRU++ layer (SRU++ paper, section on
// SRU++): single-head scaled dot-product attention over one segment, with the
// previous segment's keys and values as extra context, a residual weight
// alpha and optional layer normalisation before the output projection:
//   Q = X~ Wq^T, [K | V] = Q~ [Wk; Wv]^T, A = softmax(Q~ K~^T / sqrt(d')) V~,
//   R = Q + alpha A (optionally layernorm(R)), U = R~ Wo^T.
// The five products run on the projection kernels (the per-sequence products
// as batched launches over strided rows of the [L, B, .] layouts); the row
// softmax with its mask and the residual / normalisation are the two kernels
// below.  K and V are kept in bf16, the precision the products consume.
//
// The backward (chain rule; the pages give none) recomputes the scores, the
// weights and A from the forward's Q and KV, then runs the gradient through
// U's product, the normalisation and residual (attn_residual_bwd), the
// softmax (attn_softmax_bwd) and the products of Q, K and V, eleven products
// on the projection kernels in all.  The previous segment's keys and values
// are constants: no gradient flows into them.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace sru {
namespace {

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

constexpr float kLog2e = 1.4426950408889634f;

// One wave per row (b, t) of S [B, L, Lk]: p_j = softmax over the visible
// keys of S[j] / sqrt(d'), written as bf16; masked keys get 0.  Query t sees
// keys j < Lk, or j <= Lm + t when causal.  NR > 0: the row (Lk <= 64 NR) is
// kept in registers; NR == 0: any length, three passes over the row.
template <int NR>
__global__ __launch_bounds__(256) void attn_softmax(const float *__restrict__ S,
                                                    bf16_bits *__restrict__ P, int64_t rows,
                                                    int64_t L, int64_t Lk, int64_t Lm, int causal,
                                                    float scale)
{
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int64_t t = row % L;
    const int64_t nk = causal ? (Lm + t + 1 < Lk ? Lm + t + 1 : Lk) : Lk;
    const float *s = S + row * Lk;
    bf16_bits *p = P + row * Lk;
    const float c = scale * kLog2e;   // exp(x) = exp2(x log2 e)
    if constexpr (NR > 0) {
        float v[NR];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int64_t j = lane + 64 * i;
            v[i] = j < nk ? s[j] * c : -INFINITY;
            mx = fmaxf(mx, v[i]);
        }
        mx = wave_max(mx);
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int64_t j = lane + 64 * i;
            v[i] = j < nk ? __builtin_amdgcn_exp2f(v[i] - mx) : 0.0f;
            sum += v[i];
        }
        const float inv = 1.0f / wave_sum(sum);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int64_t j = lane + 64 * i;
            if (j < Lk) p[j] = f32_to_bf16(v[i] * inv);
        }
    } else {
        float mx = -INFINITY;
        for (int64_t j = lane; j < nk; j += 64) mx = fmaxf(mx, s[j] * c);
        mx = wave_max(mx);
        float sum = 0.0f;
        for (int64_t j = lane; j < nk; j += 64) sum += __builtin_amdgcn_exp2f(s[j] * c - mx);
        const float inv = 1.0f / wave_sum(sum);
        for (int64_t j = lane; j < Lk; j += 64)
            p[j] = f32_to_bf16(j < nk ? __builtin_amdgcn_exp2f(s[j] * c - mx) * inv : 0.0f);
    }
}

// One wave per row of width dp: R = Q + alpha O, then, when ln, the layer
// normalisation gamma (R - mean) / sqrt(var + eps) + beta (biased variance,
// taken about the mean in a second pass).  NR > 0: dp <= 64 NR, the row stays
// in registers; NR == 0: any width, the row is re-read from R.
template <int NR>
__global__ __launch_bounds__(256) void attn_residual(const float *__restrict__ Q,
                                                     const float *__restrict__ O,
                                                     const float *__restrict__ gamma,
                                                     const float *__restrict__ beta,
                                                     float *__restrict__ R, int64_t rows,
                                                     int64_t dp, float alpha, int ln, float eps)
{
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const float *q = Q + row * dp;
    const float *o = O + row * dp;
    float *r = R + row * dp;
    if constexpr (NR > 0) {
        float v[NR];
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int64_t e = lane + 64 * i;
            v[i] = e < dp ? fmaf(alpha, o[e], q[e]) : 0.0f;
            sum += v[i];
        }
        if (!ln) {
#pragma unroll
            for (int i = 0; i < NR; ++i)
                if (lane + 64 * i < dp) r[lane + 64 * i] = v[i];
            return;
        }
        const float mean = wave_sum(sum) / (float)dp;
        float sq = 0.0f;
#pragma unroll
        for (int i = 0; i < NR; ++i)
            if (lane + 64 * i < dp) sq += (v[i] - mean) * (v[i] - mean);
        const float inv = 1.0f / sqrtf(wave_sum(sq) / (float)dp + eps);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int64_t e = lane + 64 * i;
            if (e < dp) r[e] = fmaf(gamma[e] * (v[i] - mean), inv, beta[e]);
        }
    } else {
        float sum = 0.0f;
        for (int64_t e = lane; e < dp; e += 64) {
            const float v = fmaf(alpha, o[e], q[e]);
            r[e] = v;
            sum += v;
        }
        if (!ln) return;
        const float mean = wave_sum(sum) / (float)dp;
        float sq = 0.0f;
        for (int64_t e = lane; e < dp; e += 64) sq += (r[e] - mean) * (r[e] - mean);
        const float inv = 1.0f / sqrtf(wave_sum(sq) / (float)dp + eps);
        for (int64_t e = lane; e < dp; e += 64) r[e] = fmaf(gamma[e] * (r[e] - mean), inv, beta[e]);
    }
}

hipError_t launch_softmax(int64_t L, int64_t B, int64_t dp, int64_t Lm, int causal,
                          const float *S, bf16_bits *P, hipStream_t s)
{
    const int64_t rows = B * L, Lk = Lm + L;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    const float scale = 1.0f / sqrtf((float)dp);
#define SRU_SOFTMAX(NR)                                                                        \
    hipLaunchKernelGGL((attn_softmax<NR>), grid, block, 0, s, S, P, rows, L, Lk, Lm, causal,   \
                       scale)
    if (Lk <= 256)
        SRU_SOFTMAX(4);
    else if (Lk <= 512)
        SRU_SOFTMAX(8);
    else if (Lk <= 1024)
        SRU_SOFTMAX(16);
    else if (Lk <= 2048)
        SRU_SOFTMAX(32);
    else
        SRU_SOFTMAX(0);
#undef SRU_SOFTMAX
    return hipGetLastError();
}

hipError_t launch_residual(const AttnArgs &a, const float *O, hipStream_t s)
{
    const int64_t rows = a.L * a.B;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
#define SRU_RESIDUAL(NR)                                                                        \
    hipLaunchKernelGGL((attn_residual<NR>), grid, block, 0, s, a.Q, O, a.gamma, a.beta, a.R,  \
                       rows, a.dp, a.alpha, a.layernorm, a.eps)
    if (a.dp <= 256)
        SRU_RESIDUAL(4);
    else if (a.dp <= 1024)
        SRU_RESIDUAL(16);
    else
        SRU_RESIDUAL(0);
#undef SRU_RESIDUAL
    return hipGetLastError();
}

// ---- fused forward: scores, online softmax, weights x values, residual, norm ----
//
// For d' in {64, 128, 256, 512} the forward's attention core runs in one
// kernel that keeps the scores and weights on chip.  A workgroup of four waves
// owns 64 queries of one sequence b and walks the visible keys in tiles of 32.
// Wave w holds queries 32 (w % 2) .. + 31 and channel half h = w / 2 of the
// d' channels; per tile it
//   forms its half of S^T = K Q~^T over its channels (v_mfma_f32_32x32x16_bf16,
//     keys as rows, queries as columns, so a lane's accumulators belong to one
//     query), and adds the other half from its partner wave through LDS,
//   runs the online softmax per query (the running maximum is raised, and the
//     sums and accumulators rescaled, only when a tile's maximum exceeds it by
//     more than 2^8: the unnormalised weights stay <= 2^8),
//   accumulates its channel half of O^T += V^T P^T (the weights rounded to
//     bf16 as the operand; the normaliser sums the same rounded weights),
// and it ends with A = O / sum, R = Q + alpha A and the layer normalisation
// (the row sums exchanged between the two halves), all in registers.  R is
// the only output.  Both waves of a pair form the same scores and weights
// from the same operands, bit for bit.
//
// K tiles come straight from the [Lk, B, 2d'] rows; V is first transposed
// once per call into V^T tiles [B, Lk / 32, d', 32] (each tile one contiguous
// block, keys padded with zeros to a multiple of 32), so that both go from
// memory into LDS by global_load_lds_dwordx4 in whole 1 KB pieces, without
// registers.  Two LDS stages: the next tile is copied while the current one
// is used, and the tile after next is touched into L2.
//
// Within a 16-key step of the weights x values product, lane half hi of the
// B operand takes keys 8 hi .. 8 hi + 7.  The S^T accumulator of lane half hi
// holds rows 8 i + 4 hi + j (i, j = 0..3), so the A operand row r of the score
// product reads K row 16 (i / 2) + 8 hi + 4 (i % 2) + j (r = 8 i + 4 hi + j):
// accumulator values 8 s .. 8 s + 7 of a lane are then exactly keys
// 16 s + 8 hi .. + 7, the B operand of step s.
constexpr int kFusedKT = 32;      // keys per tile
constexpr int kFusedBQ = 64;      // queries per workgroup
constexpr float kFusedLazy = 8.0f;

typedef __bf16 fbf16x8 __attribute__((ext_vector_type(8)));
typedef float ff32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t fu32x4 __attribute__((ext_vector_type(4)));

int64_t fused_keys_padded(int64_t Lk) { return (Lk + kFusedKT - 1) / kFusedKT * kFusedKT; }

// The fused kernel takes d' in {64, 128, 256, 512}, with the per-lane copy
// offsets of a tile (32 key rows of [Lk, B, 2d'] bf16) and the key counts
// inside 31 bits.
bool fused_forward_ok(int64_t L, int64_t B, int64_t dp, int64_t Lm)
{
    if (dp != 64 && dp != 128 && dp != 256 && dp != 512) return false;
    const int64_t Lkp = fused_keys_padded(Lm + L), lim = (int64_t)1 << 31;
    return kFusedKT * B * 4 * dp < lim && Lkp < lim;
}

template <int DP> struct FusedLay {
    static constexpr int DPH = DP / 2;                  // channels per wave
    static constexpr int KROW = 2 * DP;                 // bytes of one key row of K
    // d' = 512: a K row is one 1 KB request; the rows sit 16 bytes apart
    // beyond their length, so that the 16 rows a quarter-wave reads fall on 16
    // different bank groups and every fragment of a lane is its first one plus
    // a constant (no per-fragment address arithmetic).  Other d': rows packed,
    // the pieces swizzled by fk_swz.
    static constexpr bool PADK = DP == 512;
    static constexpr int KPITCH = PADK ? KROW + 16 : KROW;
    static constexpr int K_BYTES = kFusedKT * KPITCH;   // the tile's K rows
    static constexpr int V_BYTES = DP * 2 * kFusedKT;   // the tile's V^T block
    static constexpr int SB = K_BYTES + V_BYTES;        // one stage
    static constexpr int QK = kFusedKT * KROW / 1024;   // 1 KB requests for K
    static constexpr int REQ = QK + V_BYTES / 1024;
    static constexpr int IPW = REQ / 4;                 // requests per wave
    static constexpr int XB = 4 * 4096;                 // partial scores, 4 KB per wave
    static_assert(IPW * 4 == REQ && QK == 2 * IPW, "K requests on waves 0, 1");
};

// Position keys of the 16-byte pieces (XOR on the piece index).  K rows: the
// 16 rows a quarter-wave reads at once (16 u .. 16 u + 15 in some order) land
// on 16 different 16-byte bank groups.  V^T rows (64 bytes, four to a bank
// line): the 16 consecutive rows of a quarter-wave likewise.
template <int DP> __device__ __forceinline__ int fk_swz(int row)
{
    if constexpr (DP == 64) return (row >> 1) & 7;   // 128-byte rows, two to a bank line
    return row & 15;
}
__device__ __forceinline__ int fv_swz(int row) { return (row >> 2) & 3; }

// V^T tiles [B, Lkp / 32, dp, 32] from the V half of KV [Lk, B, 2 dp], zeros
// for keys past Lk.  64 keys x 64 channels per block through LDS.
__global__ __launch_bounds__(256) void attn_v_transpose(const bf16_bits *__restrict__ KV,
                                                        bf16_bits *__restrict__ Vt, int64_t Lk,
                                                        int64_t Lkp, int64_t B, int64_t dp)
{
    __shared__ bf16_bits tile[64][64 + 2];
    const int64_t k0 = (int64_t)blockIdx.x * 64, e0 = (int64_t)blockIdx.y * 64, b = blockIdx.z;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = tid + 256 * i, kk = idx >> 3, ec = (idx & 7) * 8;
        const int64_t k = k0 + kk;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (k < Lk) v = *(const uint4 *)(KV + (k * B + b) * 2 * dp + dp + e0 + ec);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            tile[kk][ec + 2 * j] = (bf16_bits)(w[j] & 0xffffu);
            tile[kk][ec + 2 * j + 1] = (bf16_bits)(w[j] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = tid + 256 * i, ee = idx >> 3, kc = (idx & 7) * 8;
        const int64_t k = k0 + kc;
        if (k >= Lkp) continue;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = (uint32_t)tile[kc + 2 * j][ee] | ((uint32_t)tile[kc + 2 * j + 1][ee] << 16);
        bf16_bits *dst = Vt + ((b * (Lkp / kFusedKT) + k / kFusedKT) * dp + e0 + ee) * kFusedKT +
                         k % kFusedKT;
        *(uint4 *)dst = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

struct FusedArgs {
    int64_t L, B, Lm, Lk, Lkp;
    int causal, layernorm;
    float alpha, eps;
    const float *Q;
    const bf16_bits *KV, *Vt;
    const float *gamma, *beta;
    float *R;
    bf16_bits *Rb;         // R rounded to bf16 (the U product's operand), or null
};

template <int DP>
__global__ __launch_bounds__(256, 1) void attn_fwd_fused(FusedArgs a)
{
    typedef FusedLay<DP> Lay;
    constexpr int SB = Lay::SB, IPW = Lay::IPW, DPH = Lay::DPH;
    constexpr int NKS = DPH / 16, NOB = DPH / 32;       // score k-steps, O blocks per wave
    // two stages, the partial scores, then 1 KB that the L2 prefetches land in
    __shared__ __attribute__((aligned(16))) char smem[2 * SB + Lay::XB + 1024];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar registers
    const int qg = wave & 1, h = wave >> 1, r32 = lane & 31, hi = lane >> 5;
    const int64_t L = a.L, B = a.B, Lk = a.Lk, Lkp = a.Lkp;

    // workgroup -> (sequence, query block); consecutive workgroups go to
    // different XCDs, so a sequence's blocks are gathered on one XCD (whose
    // L2 then serves its keys and values to all of them)
    const int64_t nqb = (L + kFusedBQ - 1) / kFusedBQ, nwg = nqb * B;
    int64_t id = blockIdx.x;
    if (nwg % 8 == 0) id = (id % 8) * (nwg / 8) + id / 8;
    const int64_t b = id / nqb, qb = id % nqb;
    const int64_t t0w = qb * kFusedBQ + 32 * qg, t = t0w + r32;
    const bool tv = t < L;
    auto keys_of = [&](int64_t tq) -> int64_t {   // keys query tq sees
        return a.causal ? (a.Lm + tq + 1 < Lk ? a.Lm + tq + 1 : Lk) : Lk;
    };
    const int64_t tl = (qb + 1) * kFusedBQ < L ? (qb + 1) * kFusedBQ - 1 : L - 1;
    const int ntiles = (int)((keys_of(tl) + kFusedKT - 1) / kFusedKT);
    const int nk_wave = t0w < L ? (int)keys_of(t0w + 31 < L ? t0w + 31 : L - 1) : 0;
    const int nk_q = (int)keys_of(t);

    // Q~ fragments (B operand of S^T): query r32, channels DPH h + 16 ks + 8 hi .. + 7
    fbf16x8 qf[NKS];
    const float *qrow = a.Q + (t * B + b) * DP + DPH * h;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        fu32x4 u = {0u, 0u, 0u, 0u};
        if (tv) {
            const float4 x0 = *(const float4 *)(qrow + 16 * ks + 8 * hi);
            const float4 x1 = *(const float4 *)(qrow + 16 * ks + 8 * hi + 4);
            u[0] = pack_bf16x2(x0.x, x0.y);
            u[1] = pack_bf16x2(x0.z, x0.w);
            u[2] = pack_bf16x2(x1.x, x1.y);
            u[3] = pack_bf16x2(x1.z, x1.w);
        }
        qf[ks] = __builtin_bit_cast(fbf16x8, u);
    }

    // The tile's copies: waves 0, 1 copy K rows, waves 2, 3 the V^T block.
    // Every request is a per-lane 32-bit byte offset from a wave-uniform base
    // (the tile's first K row of sequence b, or the tile's V^T block).
    const bool kwave = wave < 2;
    // V^T request q: rows 16 (q - QK) + lane / 4; the piece swizzle of such a
    // row is (lane / 16) % 4, so one offset serves every request
    const uint32_t voff_v = (uint32_t)((lane >> 2) * 64 + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
    // K request q (packed rows): rows q RPQ + lane / CPR
    constexpr int CPR = DP / 8, RPQ = 1024 / Lay::KROW;    // pieces per row, rows per request
    uint32_t koff[Lay::PADK ? 1 : IPW];
    int krow_of[Lay::PADK ? 1 : IPW];
#pragma unroll
    for (int i = 0; i < (Lay::PADK ? 1 : IPW); ++i) {
        const int row = (wave * IPW + i) * RPQ + lane / CPR;
        const int c = (lane % CPR) ^ fk_swz<DP>(row);
        krow_of[i] = row;
        koff[i] = (uint32_t)(row * B * 4 * DP + 16 * c);
    }
    const char *kbase = (const char *)(a.KV + b * 2 * DP);
    const char *vbase = (const char *)(a.Vt + b * (Lkp / kFusedKT) * DP * kFusedKT);
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    char *xbuf = smem + 2 * SB;                          // partial scores [wave][16][64 lanes]
    // L2 prefetch of a later tile: the workgroups of a sequence walk its keys
    // in step, so without it every tile's first touch of a line is a miss that
    // all of them wait for.  Each lane copies 16 bytes of one 128-byte line
    // (every line of the tile's K rows and V^T block) into a 1 KB LDS area
    // nobody reads; PF requests per wave, always issued (past the last item the
    // last line again), so that the waits can count them.
    constexpr int PF_ITEMS = DP, PF = (PF_ITEMS + 255) / 256;
    auto prefetch = [&](int kt) {
        kt = kt < ntiles ? kt : ntiles - 1;
        const uint32_t dummy = __builtin_amdgcn_readfirstlane(lds0 + 2 * SB + Lay::XB);
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            int j = tid + 256 * i;
            j = j < PF_ITEMS ? j : PF_ITEMS - 1;
            const void *src;
            if (j < DP / 2) {
                constexpr int LPR = DP / 64;   // 128-byte lines per key row
                int64_t key = (int64_t)kt * kFusedKT + j / LPR;
                key = key < Lk ? key : Lk - 1;
                src = a.KV + (key * B + b) * 2 * DP + (j % LPR) * 64;
            } else {
                src = vbase + (int64_t)kt * Lay::V_BYTES + (j - DP / 2) * 128;
            }
            dma16(src, dummy);
        }
    };
    auto issue = [&](int kt, int st) {
        const uint32_t ldss = lds0 + st * SB;
        if (kwave) {
            const char *base = kbase + (int64_t)kt * kFusedKT * B * 4 * DP;
            // rows past the last key (the last tile) repeat it; they are masked
            const int last = (int)(Lk - 1 - (int64_t)kt * kFusedKT);
            if constexpr (Lay::PADK) {   // request q = K row q
                const uint32_t rstride = (uint32_t)(B * 4 * DP);   // bytes between key rows
#pragma unroll
                for (int i = 0; i < IPW; ++i) {
                    int q = wave * IPW + i;
                    q = q < last ? q : last;
                    dma16s(base, 16 * lane + (uint32_t)q * rstride,
                           __builtin_amdgcn_readfirstlane(ldss + (wave * IPW + i) * Lay::KPITCH));
                }
            } else {
#pragma unroll
                for (int i = 0; i < IPW; ++i) {
                    const int over = krow_of[i] > last ? krow_of[i] - last : 0;
                    dma16s(base, koff[i] - (uint32_t)(over * B * 4 * DP),
                           __builtin_amdgcn_readfirstlane(ldss + (wave * IPW + i) * 1024));
                }
            }
        } else {
            const char *base = vbase + (int64_t)kt * Lay::V_BYTES;
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int q = wave * IPW + i - Lay::QK;
                dma16s(base, voff_v + (uint32_t)q * 1024u,
                       __builtin_amdgcn_readfirstlane(ldss + Lay::K_BYTES + q * 1024));
            }
        }
    };

    ff32x16 o[NOB];
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[ob][e] = 0.0f;
    float mrun = -INFINITY, lsum = 0.0f;
    const float csc = kLog2e / sqrtf((float)DP);

    // the K row this lane reads for the score product (see above), and the
    // byte offsets of its fragment pieces
    const int ri = r32 >> 3, rhi = (r32 >> 2) & 1, rj = r32 & 3;
    const int krow = 16 * (ri >> 1) + 8 * rhi + 4 * (ri & 1) + rj;
    const int c0 = 2 * (DPH / 16) * h + hi;              // first piece of this wave's channels
    const int fk = fk_swz<DP>(krow);
    // byte offset of K piece c0 + 2 ks of row krow: kof + 32 ks when padded
    const int kof = Lay::PADK ? krow * Lay::KPITCH + 16 * c0 : krow * Lay::KPITCH;
    auto kpiece = [&](int ks) -> int {
        return Lay::PADK ? kof + 32 * ks : kof + (((c0 + 2 * ks) ^ fk) << 4);
    };
    // V^T row DPH h + 32 ob + r32, keys 16 s + 8 hi ..: vo[s] + 2048 ob
    // ((DPH h + 32 ob) is a multiple of 4, so the row's swizzle is r32's)
    const int fv = fv_swz(r32);
    const int vo0 = Lay::K_BYTES + (DPH * h + r32) * 64 + ((hi ^ fv) << 4);
    const int vo1 = Lay::K_BYTES + (DPH * h + r32) * 64 + (((2 + hi) ^ fv) << 4);
    // the wave's fewest visible keys (its first query): tiles below it need no mask
    const int nk_min = t0w < L ? (int)keys_of(t0w) : 0;

    // One tile: wait for its copies, request the next, the score half, the
    // exchange with the partner wave, scaled and masked scores in v[].
    // Returns false when no query of the wave sees the tile.
    float v[16];
    bool full = false;   // the tile is visible to every query of the wave: no mask
    auto scores = [&](int kt) -> bool {
        const int st = kt & 1;
        // this wave's copies of tile kt are done once at most the PF
        // prefetch requests issued after them are in flight
        if (kt == 0)
            wait_vmcnt<0>();
        else
            wait_vmcnt<PF>();
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        if (kt + 1 < ntiles) {
            issue(kt + 1, st ^ 1);
            prefetch(kt + 3);
        }
        const bool active = kt * kFusedKT < nk_wave;     // the same in both waves of the pair
        ff32x16 sacc;
        if (active) {
            const char *kst = smem + st * SB;
            // two accumulation chains (even and odd k-steps), added at the end
            ff32x16 s1;
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[e] = s1[e] = 0.0f;
            fbf16x8 kf[4];
#pragma unroll
            for (int j = 0; j < 4 && j < NKS; ++j) kf[j] = *(const fbf16x8 *)(kst + kpiece(j));
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const fbf16x8 cur = kf[ks & 3];
                if (ks + 4 < NKS) kf[ks & 3] = *(const fbf16x8 *)(kst + kpiece(ks + 4));
                if (ks & 1)
                    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[ks], s1, 0, 0, 0);
                else
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[ks], sacc, 0, 0, 0);
            }
            // keep four K reads in flight ahead of the MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int ks = 0; ks + 4 < NKS; ++ks) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            sacc += s1;
            // this half to the partner: [wave][4 pieces][64 lanes][4 floats]
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *(float4 *)(xbuf + ((wave * 4 + q4) * 64 + lane) * 16) =
                    make_float4(sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]);
        }
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        if (!active) return false;
        const int pw = wave ^ 2;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 x = *(const float4 *)(xbuf + ((pw * 4 + q4) * 64 + lane) * 16);
            sacc[4 * q4] += x.x;
            sacc[4 * q4 + 1] += x.y;
            sacc[4 * q4 + 2] += x.z;
            sacc[4 * q4 + 3] += x.w;
        }
        // accumulator value 4 i + j: key kt*32 + 16 (i / 2) + 8 hi + 4 (i % 2) + j
        full = (kt + 1) * kFusedKT <= nk_min;
        if (full) {
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = sacc[e] * csc;
        } else {
            const int kb = kt * kFusedKT + 8 * hi;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = kb + 16 * (e >> 3) + (e & 7);
                v[e] = key < nk_q ? sacc[e] * csc : -INFINITY;
            }
        }
        return true;
    };
    auto tile_max = [&]() -> float {
        float mt = v[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mt = fmaxf(mt, v[e]);
        return fmaxf(mt, __shfl_xor(mt, 32, 64));
    };
    // weights (rounded to bf16) and O^T += V^T P^T for this wave's channels
    auto accumulate = [&](int st) {
        const char *vst = smem + st * SB;
        fu32x4 pu[2];
        float ps = 0.0f;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x0 = v[8 * s2 + 2 * i], x1 = v[8 * s2 + 2 * i + 1];
                float p0 = __builtin_amdgcn_exp2f(x0 - mrun), p1 = __builtin_amdgcn_exp2f(x1 - mrun);
                if (!full) {   // masked scores are -inf; mrun may be too
                    p0 = x0 > -INFINITY ? p0 : 0.0f;
                    p1 = x1 > -INFINITY ? p1 : 0.0f;
                }
                pu[s2][i] = pack_bf16x2(p0, p1);
                ps += __uint_as_float(pu[s2][i] << 16) + __uint_as_float(pu[s2][i] & 0xffff0000u);
            }
        lsum += ps;
        const fbf16x8 pf0 = __builtin_bit_cast(fbf16x8, pu[0]);
        const fbf16x8 pf1 = __builtin_bit_cast(fbf16x8, pu[1]);
        // V^T piece of row DPH h + 32 ob + r32 holding keys 16 s + 8 hi ..
        fbf16x8 vf[4];
        // step n = s NOB + ob: consecutive MFMAs update different blocks
        auto vread = [&](int n) {
            const int ob = n % NOB, s2 = n / NOB;
            return *(const fbf16x8 *)(vst + (s2 ? vo1 : vo0) + ob * 32 * 64);
        };
#pragma unroll
        for (int j = 0; j < 4 && j < 2 * NOB; ++j) vf[j] = vread(j);
#pragma unroll
        for (int n = 0; n < 2 * NOB; ++n) {
            const fbf16x8 cur = vf[n & 3];
            if (n + 4 < 2 * NOB) vf[n & 3] = vread(n + 4);
            o[n % NOB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, n < NOB ? pf0 : pf1, o[n % NOB],
                                                                0, 0, 0);
        }
        // keep four V reads in flight ahead of the MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int n = 0; n + 4 < 2 * NOB; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };

    prefetch(1);
    prefetch(2);
    issue(0, 0);
    // tile 0 holds key 0, which every query sees: its maximum starts mrun
    if (scores(0)) {
        mrun = tile_max();
        accumulate(0);
    }
    int kt = 1;
    while (kt < ntiles) {
        // the common case: the running maximum stays within 2^8 of each
        // tile's maximum, and O is never rescaled
        bool raise = false;
        for (; kt < ntiles; ++kt) {
            if (!scores(kt)) continue;
            const float mt = tile_max();
            if (__any(mt > mrun + kFusedLazy)) {
                raise = true;
                break;
            }
            accumulate(kt & 1);
        }
        if (!raise) break;
        // a tile raised some query's maximum: rescale, then finish the tile
        const float mt = tile_max();
        const float mnew = mt > mrun + kFusedLazy ? mt : mrun;
        const float f = __builtin_amdgcn_exp2f(mrun - mnew);
        lsum *= f;
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob) o[ob] *= f;
        mrun = mnew;
        accumulate(kt & 1);
        ++kt;
    }
    wait_vmcnt<0>();   // no copy may land in LDS after the workgroup ends

    // A = O / sum, R = Q + alpha A, layer norm.  Lane holds query r32 and
    // channels DPH h + 32 ob + 8 i + 4 hi + j (value 4 i + j of block ob).
    float l = lsum + __shfl_xor(lsum, 32, 64);
    const float inv = 1.0f / l;
    float sum = 0.0f;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 qv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (tv) qv = *(const float4 *)(qrow + 32 * ob + 8 * i + 4 * hi);
            o[ob][4 * i] = fmaf(a.alpha, o[ob][4 * i] * inv, qv.x);
            o[ob][4 * i + 1] = fmaf(a.alpha, o[ob][4 * i + 1] * inv, qv.y);
            o[ob][4 * i + 2] = fmaf(a.alpha, o[ob][4 * i + 2] * inv, qv.z);
            o[ob][4 * i + 3] = fmaf(a.alpha, o[ob][4 * i + 3] * inv, qv.w);
            sum += (o[ob][4 * i] + o[ob][4 * i + 1]) + (o[ob][4 * i + 2] + o[ob][4 * i + 3]);
        }
    if (a.layernorm) {
        // the row's sums: this lane pair's half, then the partner wave's half
        float *xs = (float *)xbuf;                       // [wave][32 queries]
        auto row_total = [&](float part) -> float {
            part += __shfl_xor(part, 32, 64);
            __builtin_amdgcn_s_barrier();                // the last reads of xs are done
            if (hi == 0) xs[wave * 32 + r32] = part;
            wait_lgkm0();
            __builtin_amdgcn_s_barrier();
            const float other = xs[(wave ^ 2) * 32 + r32];
            return h == 0 ? part + other : other + part;
        };
        const float mean = row_total(sum) / (float)DP;
        float sq = 0.0f;
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
            for (int e = 0; e < 16; ++e) sq += (o[ob][e] - mean) * (o[ob][e] - mean);
        const float rs = 1.0f / sqrtf(row_total(sq) / (float)DP + a.eps);
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e0 = DPH * h + 32 * ob + 8 * i + 4 * hi;
                const float4 gm = *(const float4 *)(a.gamma + e0);
                const float4 bt = *(const float4 *)(a.beta + e0);
                o[ob][4 * i] = fmaf(gm.x * (o[ob][4 * i] - mean), rs, bt.x);
                o[ob][4 * i + 1] = fmaf(gm.y * (o[ob][4 * i + 1] - mean), rs, bt.y);
                o[ob][4 * i + 2] = fmaf(gm.z * (o[ob][4 * i + 2] - mean), rs, bt.z);
                o[ob][4 * i + 3] = fmaf(gm.w * (o[ob][4 * i + 3] - mean), rs, bt.w);
            }
    }
    if (tv) {
        float *rrow = a.R + (t * B + b) * DP + DPH * h;
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(float4 *)(rrow + 32 * ob + 8 * i + 4 * hi) =
                    make_float4(o[ob][4 * i], o[ob][4 * i + 1], o[ob][4 * i + 2], o[ob][4 * i + 3]);
        if (a.Rb) {
            bf16_bits *brow = a.Rb + (t * B + b) * DP + DPH * h;
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *(uint2 *)(brow + 32 * ob + 8 * i + 4 * hi) =
                        make_uint2(pack_bf16x2(o[ob][4 * i], o[ob][4 * i + 1]),
                                   pack_bf16x2(o[ob][4 * i + 2], o[ob][4 * i + 3]));
        }
    }
}

hipError_t launch_fused(const AttnArgs &a, bf16_bits *Vt, bf16_bits *Rb, hipStream_t s)
{
    const int64_t Lk = a.Lm + a.L, Lkp = fused_keys_padded(Lk);
    hipLaunchKernelGGL(attn_v_transpose, dim3((unsigned)((Lkp + 63) / 64), (unsigned)(a.dp / 64),
                                              (unsigned)a.B),
                       dim3(256), 0, s, (const bf16_bits *)a.KV, Vt, Lk, Lkp, a.B, a.dp);
    FusedArgs f;
    f.L = a.L, f.B = a.B, f.Lm = a.Lm, f.Lk = Lk, f.Lkp = Lkp;
    f.causal = a.causal, f.layernorm = a.layernorm;
    f.alpha = a.alpha, f.eps = a.eps;
    f.Q = a.Q, f.KV = (const bf16_bits *)a.KV, f.Vt = Vt;
    f.gamma = a.gamma, f.beta = a.beta, f.R = a.R, f.Rb = Rb;
    const dim3 grid((unsigned)(((a.L + kFusedBQ - 1) / kFusedBQ) * a.B)), block(256);
    switch (a.dp) {
    case 64: hipLaunchKernelGGL(attn_fwd_fused<64>, grid, block, 0, s, f); break;
    case 128: hipLaunchKernelGGL(attn_fwd_fused<128>, grid, block, 0, s, f); break;
    case 256: hipLaunchKernelGGL(attn_fwd_fused<256>, grid, block, 0, s, f); break;
    default: hipLaunchKernelGGL(attn_fwd_fused<512>, grid, block, 0, s, f); break;
    }
    return hipGetLastError();
}

// ---- backward -----------------------------------------------------------

constexpr int kResRowsPerWave = 4;    // rows of attn_residual_bwd per wave (16 per block)

// The residual and normalisation backward, one wave per row, kResRowsPerWave
// rows per wave.  From dR (the gradient of R) it recomputes S = Q + alpha O
// and, when ln, xh = (S - mean) / sqrt(var + eps), and writes
//   dS = (dR gamma - mean(dR gamma) - xh mean(dR gamma xh)) / sqrt(var + eps)
//        (dS = dR without the norm) to dQ (the residual path into Q),
//   dO = alpha dS and D[row] = dO . O (the softmax backward's row term).
// Each block adds its rows' dR xh, dR and dS . O into one partial row
// part[block] = [dgamma (dp) | dbeta (dp) | dalpha], summed later in block
// order.  dp <= 64 NR (the row stays in registers).
template <int NR>
__global__ __launch_bounds__(256) void attn_residual_bwd(
    const float *__restrict__ Q, const float *__restrict__ O, const float *__restrict__ dR,
    const float *__restrict__ gamma, float *__restrict__ dQ, float *__restrict__ dO,
    float *__restrict__ D, float *__restrict__ part, int64_t rows, int64_t dp, float alpha,
    int ln, float eps)
{
    __shared__ float red[4][2 * 64 * NR + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float pg[NR], pb[NR], g[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        pg[i] = 0.0f;
        pb[i] = 0.0f;
        const int64_t e = lane + 64 * i;
        g[i] = (ln && e < dp) ? gamma[e] : 1.0f;
    }
    float pa = 0.0f;
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * kResRowsPerWave;
    for (int r = 0; r < kResRowsPerWave; ++r) {
        const int64_t row = row0 + r;
        if (row >= rows) break;
        const float *q = Q + row * dp, *o = O + row * dp, *dr = dR + row * dp;
        float sv[NR], ov[NR], dv[NR];
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int64_t e = lane + 64 * i;
            const bool in = e < dp;
            ov[i] = in ? o[e] : 0.0f;
            dv[i] = in ? dr[e] : 0.0f;
            sv[i] = in ? fmaf(alpha, ov[i], q[e]) : 0.0f;
            sum += sv[i];
        }
        float ds[NR];
        if (ln) {
            const float mean = wave_sum(sum) / (float)dp;
            float sq = 0.0f;
#pragma unroll
            for (int i = 0; i < NR; ++i)
                if (lane + 64 * i < dp) sq += (sv[i] - mean) * (sv[i] - mean);
            const float inv = 1.0f / sqrtf(wave_sum(sq) / (float)dp + eps);
            float m1 = 0.0f, m2 = 0.0f;
            float xh[NR];
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                xh[i] = lane + 64 * i < dp ? (sv[i] - mean) * inv : 0.0f;
                const float dxh = dv[i] * g[i];
                m1 += dxh;
                m2 += dxh * xh[i];
                pg[i] = fmaf(dv[i], xh[i], pg[i]);
                pb[i] += dv[i];
            }
            m1 = wave_sum(m1) / (float)dp;
            m2 = wave_sum(m2) / (float)dp;
#pragma unroll
            for (int i = 0; i < NR; ++i) ds[i] = (dv[i] * g[i] - m1 - xh[i] * m2) * inv;
        } else {
#pragma unroll
            for (int i = 0; i < NR; ++i) ds[i] = dv[i];
        }
        float dot = 0.0f, da = 0.0f;
        float *dq = dQ + row * dp, *dop = dO + row * dp;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int64_t e = lane + 64 * i;
            if (e < dp) {
                const float d_o = alpha * ds[i];
                dq[e] = ds[i];
                dop[e] = d_o;
                dot = fmaf(d_o, ov[i], dot);
                da = fmaf(ds[i], ov[i], da);
            }
        }
        dot = wave_sum(dot);
        if (lane == 0) D[row] = dot;
        pa += da;
    }
    // this block's partial row, the four waves added in order
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        red[wave][lane + 64 * i] = pg[i];
        red[wave][64 * NR + lane + 64 * i] = pb[i];
    }
    pa = wave_sum(pa);
    if (lane == 0) red[wave][2 * 64 * NR] = pa;
    __syncthreads();
    float *out = part + (int64_t)blockIdx.x * (2 * dp + 1);
    for (int64_t e = threadIdx.x; e < 2 * dp + 1; e += 256) {
        const int64_t c = e < dp ? e : (e < 2 * dp ? 64 * NR + (e - dp) : 2 * 64 * NR);
        out[e] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
    }
}

// dgamma, dbeta (when ln) and dalpha: the blocks' partial rows added in a
// fixed order (bit-reproducible run to run).  A block of 16 waves owns 64
// consecutive entries: wave w adds the partial rows of residue w (mod 16) in
// increasing order, eight loads in flight, then the 16 sums are added in
// wave order.
constexpr int kPartWaves = 16;

__global__ __launch_bounds__(64 * kPartWaves) void attn_part_reduce(const float *__restrict__ part,
                                                                    int64_t nblk, int64_t dp,
                                                                    float *__restrict__ dgamma,
                                                                    float *__restrict__ dbeta,
                                                                    float *__restrict__ dalpha)
{
    constexpr int U = 8;
    __shared__ float red[kPartWaves][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t n = 2 * dp + 1, e = (int64_t)blockIdx.x * 64 + lane;
    float acc = 0.0f;
    if (e < n) {
        int64_t b = wv;
        for (; b + (U - 1) * kPartWaves < nblk; b += U * kPartWaves) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = part[(b + u * kPartWaves) * n + e];
#pragma unroll
            for (int u = 0; u < U; ++u) acc += v[u];
        }
        for (; b < nblk; b += kPartWaves) acc += part[b * n + e];
    }
    red[wv][lane] = acc;
    __syncthreads();
    if (wv != 0 || e >= n) return;
    float t = red[0][lane];
#pragma unroll
    for (int w = 1; w < kPartWaves; ++w) t += red[w][lane];
    if (e < dp) {
        if (dgamma) dgamma[e] = t;
    } else if (e < 2 * dp) {
        if (dbeta) dbeta[e - dp] = t;
    } else {
        *dalpha = t;
    }
}

// The softmax backward, one wave per row (b, t) of the [B, L, Lk] scores:
// the weights p are recomputed from S exactly as attn_softmax forms them
// (fp32, before rounding), and
//   dS'[j] = p_j (dP[j] - D[t B + b]) / sqrt(d')   for the visible keys,
// 0 for the masked ones, written as bf16 (the operand of the dQ and dK
// products).  NR > 0: the row (Lk <= 64 NR) stays in registers; NR == 0:
// any length, extra passes over the row.
template <int NR>
__global__ __launch_bounds__(256) void attn_softmax_bwd(const float *__restrict__ S,
                                                        const float *__restrict__ dP,
                                                        const float *__restrict__ D,
                                                        bf16_bits *__restrict__ dSp, int64_t rows,
                                                        int64_t L, int64_t B, int64_t Lk,
                                                        int64_t Lm, int causal, float scale)
{
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int64_t b = row / L, t = row % L;
    const int64_t nk = causal ? (Lm + t + 1 < Lk ? Lm + t + 1 : Lk) : Lk;
    const float *s = S + row * Lk, *gp = dP + row * Lk;
    bf16_bits *o = dSp + row * Lk;
    const float c = scale * kLog2e;
    const float d = D[t * B + b];
    if constexpr (NR > 0) {
        float v[NR];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int64_t j = lane + 64 * i;
            v[i] = j < nk ? s[j] * c : -INFINITY;
            mx = fmaxf(mx, v[i]);
        }
        mx = wave_max(mx);
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int64_t j = lane + 64 * i;
            v[i] = j < nk ? __builtin_amdgcn_exp2f(v[i] - mx) : 0.0f;
            sum += v[i];
        }
        const float inv = 1.0f / wave_sum(sum);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int64_t j = lane + 64 * i;
            if (j < Lk) o[j] = f32_to_bf16(j < nk ? v[i] * inv * (gp[j] - d) * scale : 0.0f);
        }
    } else {
        float mx = -INFINITY;
        for (int64_t j = lane; j < nk; j += 64) mx = fmaxf(mx, s[j] * c);
        mx = wave_max(mx);
        float sum = 0.0f;
        for (int64_t j = lane; j < nk; j += 64) sum += __builtin_amdgcn_exp2f(s[j] * c - mx);
        const float inv = 1.0f / wave_sum(sum);
        for (int64_t j = lane; j < Lk; j += 64)
            o[j] = f32_to_bf16(j < nk ? __builtin_amdgcn_exp2f(s[j] * c - mx) * inv *
                                            (gp[j] - d) * scale
                                      : 0.0f);
    }
}

// The same for rows whose length is a multiple of 4 (Lk <= 256 NV): each lane
// holds four consecutive keys per group of 256, S and dP are read with 16-byte
// loads up front, the weights are exponentiated once, and dS' leaves as
// 8-byte stores.
template <int NV>
__global__ __launch_bounds__(256) void attn_softmax_bwd_v4(const float *__restrict__ S,
                                                           const float *__restrict__ dP,
                                                           const float *__restrict__ D,
                                                           bf16_bits *__restrict__ dSp, int64_t rows,
                                                           int64_t L, int64_t B, int64_t Lk,
                                                           int64_t Lm, int causal, float scale)
{
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int64_t b = row / L, t = row % L;
    const int64_t nk = causal ? (Lm + t + 1 < Lk ? Lm + t + 1 : Lk) : Lk;
    const float4 *s4 = (const float4 *)(S + row * Lk), *g4 = (const float4 *)(dP + row * Lk);
    const float c = scale * kLog2e;
    const float d = D[t * B + b];
    float sv[NV][4], gv[NV][4];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int64_t j = 4 * (lane + 64 * i);
        float4 x = make_float4(0.0f, 0.0f, 0.0f, 0.0f), y = x;
        if (j < Lk) {
            x = s4[lane + 64 * i];
            y = g4[lane + 64 * i];
        }
        sv[i][0] = x.x, sv[i][1] = x.y, sv[i][2] = x.z, sv[i][3] = x.w;
        gv[i][0] = y.x, gv[i][1] = y.y, gv[i][2] = y.z, gv[i][3] = y.w;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t j = 4 * (lane + 64 * i) + e;
            sv[i][e] = j < nk ? sv[i][e] * c : -INFINITY;
            mx = fmaxf(mx, sv[i][e]);
        }
    mx = wave_max(mx);
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t j = 4 * (lane + 64 * i) + e;
            sv[i][e] = j < nk ? __builtin_amdgcn_exp2f(sv[i][e] - mx) : 0.0f;
            sum += sv[i][e];
        }
    const float inv = 1.0f / wave_sum(sum);
    bf16_bits *o = dSp + row * Lk;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int64_t j = 4 * (lane + 64 * i);
        if (j >= Lk) continue;
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            r[e] = j + e < nk ? sv[i][e] * inv * (gv[i][e] - d) * scale : 0.0f;
        *(uint2 *)(o + j) = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
    }
}

struct WsLayout {
    size_t s_off, p_off, o_off, total;   // bytes
};

WsLayout ws_layout(int64_t L, int64_t B, int64_t dp, int64_t Lm)
{
    auto up = [](size_t n) { return (n + 255) & ~(size_t)255; };
    const size_t sp = (size_t)B * (size_t)L * (size_t)(Lm + L);
    WsLayout w;
    w.s_off = 0;
    w.p_off = up(sp * 4);
    w.o_off = w.p_off + up(sp * 2);
    w.total = w.o_off + up((size_t)L * (size_t)B * (size_t)dp * 4);
    return w;
}

// The attention core: S_b [L, Lk] = Q~_b K_b^T for every sequence b (Q's rows
// t*B + b), P = the masked softmax of S / sqrt(d') in bf16, and O_b = P_b V_b
// into O's rows t*B + b.
hipError_t attend(int64_t L, int64_t B, int64_t dp, int64_t Lm, int causal, const float *Q,
                  const bf16_bits *KV, float *S, bf16_bits *P, float *O, hipStream_t s,
                  const bf16_bits *Qb = nullptr)
{
    const int64_t Lk = Lm + L;
    hipError_t e;
    {   // with Qb (Q rounded to bf16, the values the product would round Q to)
        // both operands are bf16 rows along d' and go straight into LDS
        GemmArgs g;
        g.M = L, g.N = Lk, g.K = dp;
        g.A = Qb ? (const void *)Qb : (const void *)Q, g.a_bf16 = Qb != nullptr;
        g.lda = B * dp, g.sa = dp;
        g.Bm = KV, g.b_bf16 = true, g.b_kn = false, g.ldb = B * 2 * dp, g.sb = 2 * dp;
        g.C = S, g.ldc = Lk, g.sc = L * Lk, g.accumulate = false;
        g.batch = B;
        g.causal_skip = causal ? Lm : -1;   // the softmax reads no masked score
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    if ((e = launch_softmax(L, B, dp, Lm, causal, S, P, s)) != hipSuccess) return e;
    GemmArgs g;
    g.M = L, g.N = dp, g.K = Lk;
    g.A = P, g.a_bf16 = true, g.lda = Lk, g.sa = L * Lk;
    g.Bm = KV + dp, g.b_bf16 = true, g.b_kn = true, g.ldb = B * 2 * dp, g.sb = 2 * dp;
    g.C = O, g.ldc = B * dp, g.sc = dp, g.accumulate = false;
    g.batch = B;
    g.causal_klim = causal ? Lm : -1;       // masked weights are zeros
    return launch_gemm(g, s);
}

// Workspace of the backward (bytes, each region 256-byte aligned).
struct BwdLayout {
    size_t s_off, p_off, dp_off, dsp_off, o_off, dr_off, dq_off, do_off, dkv_off, d_off,
        part_off, wg_off, wot_off, qb_off, rb_off, dob_off, total;
    int64_t nblk;
};

BwdLayout bwd_layout(int64_t L, int64_t B, int64_t d, int64_t dp, int64_t Lm, int64_t n3)
{
    auto up = [](size_t n) { return (n + 255) & ~(size_t)255; };
    const size_t sp = (size_t)B * (size_t)L * (size_t)(Lm + L), LB = (size_t)(L * B);
    BwdLayout w;
    w.nblk = ((int64_t)LB + 4 * kResRowsPerWave - 1) / (4 * kResRowsPerWave);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += up(bytes);
        return at;
    };
    w.s_off = take(sp * 4);
    w.p_off = take(sp * 2);
    w.dp_off = take(sp * 4);
    w.dsp_off = take(sp * 2);
    w.o_off = take(LB * dp * 4);
    w.dr_off = take(LB * dp * 4);
    w.dq_off = take(LB * dp * 4);
    w.do_off = take(LB * dp * 4);
    w.dkv_off = take(LB * 2 * dp * 2);   // [dK | dV], bf16
    w.d_off = take(LB * 4);
    w.part_off = take((size_t)w.nblk * (size_t)(2 * dp + 1) * 4);
    w.wot_off = take((size_t)n3 * (size_t)dp * 2);                 // Wo^T, for a bf16 dU
    // Q, R and dO rounded to bf16: the values the products would round them
    // to as they load them, made once so that both operands of those products
    // are bf16 (copied straight into LDS)
    w.qb_off = take(LB * dp * 2);
    w.rb_off = take(LB * dp * 2);
    w.dob_off = take(LB * dp * 2);
    size_t wg = wgrad_workspace_bytes(n3, dp, (int64_t)LB);
    const size_t w2 = wgrad_workspace_bytes(2 * dp, dp, (int64_t)LB);
    const size_t w3 = wgrad_workspace_bytes(dp, d, (int64_t)LB);
    wg = wg > w2 ? wg : w2;
    wg = wg > w3 ? wg : w3;
    w.wg_off = take(wg);
    w.total = off;
    return w;
}

}  // namespace

size_t attention_backward_workspace_bytes(int64_t L, int64_t B, int64_t d, int64_t dp,
                                          int64_t Lm, int64_t n3)
{
    return bwd_layout(L, B, d, dp, Lm, n3).total;
}

hipError_t launch_attention_backward(const AttnBwdArgs &a, hipStream_t s)
{
    const int64_t L = a.L, B = a.B, d = a.d, dp = a.dp, Lm = a.Lm, Lk = Lm + L, LB = L * B;
    const int64_t n3 = a.n3;
    const BwdLayout w = bwd_layout(L, B, d, dp, Lm, n3);
    char *ws = (char *)a.workspace;
    float *S = (float *)(ws + w.s_off);
    bf16_bits *P = (bf16_bits *)(ws + w.p_off);
    float *dP = (float *)(ws + w.dp_off);
    bf16_bits *dSp = (bf16_bits *)(ws + w.dsp_off);
    float *O = (float *)(ws + w.o_off);
    float *dR = (float *)(ws + w.dr_off);
    float *dQ = (float *)(ws + w.dq_off);
    float *dO = (float *)(ws + w.do_off);
    // [dK | dV] written rounded to bf16: the values the two products that read
    // it would round it to as they load it
    bf16_bits *dKVb = (bf16_bits *)(ws + w.dkv_off);
    float *D = (float *)(ws + w.d_off);
    float *part = (float *)(ws + w.part_off);
    float *wg = (float *)(ws + w.wg_off);
    bf16_bits *Qb = (bf16_bits *)(ws + w.qb_off);
    bf16_bits *Rb = (bf16_bits *)(ws + w.rb_off);
    bf16_bits *dOb = (bf16_bits *)(ws + w.dob_off);
    const bf16_bits *KV = a.KV;
    hipError_t e;
    if ((e = launch_round_bf16(LB * dp, a.Q, Qb, s)) != hipSuccess) return e;
    if ((e = launch_round_bf16(LB * dp, a.R, Rb, s)) != hipSuccess) return e;
    // the forward's weights and A, recomputed from Q and KV
    if ((e = attend(L, B, dp, Lm, a.causal, a.Q, KV, S, P, O, s, Qb)) != hipSuccess) return e;
    {   // dR [LB, d'] = dU Wo: with a bf16 dU, Wo^T [d', n3] is formed first so
        // that both operands are bf16 rows along the reduction (the kernel that
        // copies them straight into LDS); with an fp32 dU, Wo is read as [K, N]
        GemmArgs g;
        g.M = LB, g.N = dp, g.K = n3;
        g.A = a.dU, g.a_bf16 = a.du_bf16;
        g.b_bf16 = true;
        if (a.du_bf16) {
            bf16_bits *WoT = (bf16_bits *)(ws + w.wot_off);
            if ((e = launch_transpose(n3, dp, a.Wo, WoT, true, s)) != hipSuccess) return e;
            g.Bm = WoT, g.b_kn = false;
        } else {
            g.Bm = a.Wo, g.b_kn = true;
        }
        g.C = dR, g.accumulate = false;
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    {   // dWo [n3, d'] = dU^T R~
        GemmArgs g;
        g.M = n3, g.N = dp, g.K = LB;
        g.A = a.dU, g.a_bf16 = a.du_bf16;
        g.Bm = Rb, g.b_bf16 = true;
        g.C = a.dWo, g.accumulate = false;
        if ((e = launch_gemm_wgrad(g, false, wg, s)) != hipSuccess) return e;
    }
    {   // the residual and normalisation: dQ = dS, dO = alpha dS, D, partials
        const dim3 grid((unsigned)w.nblk), block(256);
#define SRU_RES_BWD(NR)                                                                          \
    hipLaunchKernelGGL((attn_residual_bwd<NR>), grid, block, 0, s, a.Q, O, dR, a.gamma, dQ, dO, \
                       D, part, LB, dp, a.alpha, a.layernorm, a.eps)
        if (dp <= 128)
            SRU_RES_BWD(2);
        else if (dp <= 256)
            SRU_RES_BWD(4);
        else if (dp <= 512)
            SRU_RES_BWD(8);
        else
            SRU_RES_BWD(16);
#undef SRU_RES_BWD
        hipLaunchKernelGGL(attn_part_reduce, dim3((unsigned)((2 * dp + 1 + 63) / 64)),
                           dim3(64 * kPartWaves), 0, s, part, w.nblk, dp,
                           a.layernorm ? a.dgamma : nullptr, a.layernorm ? a.dbeta : nullptr,
                           a.dalpha);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_round_bf16(LB * dp, dO, dOb, s)) != hipSuccess) return e;
    }
    {   // dP_b [L, Lk] = dO~_b V~_b^T
        GemmArgs g;
        g.M = L, g.N = Lk, g.K = dp;
        g.A = dOb, g.a_bf16 = true, g.lda = B * dp, g.sa = dp;
        g.Bm = KV + dp, g.b_bf16 = true, g.b_kn = false, g.ldb = B * 2 * dp, g.sb = 2 * dp;
        g.C = dP, g.ldc = Lk, g.sc = L * Lk, g.accumulate = false;
        g.batch = B;
        g.causal_skip = a.causal ? Lm : -1;   // the softmax backward reads none masked
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    {   // dS' = p (dP - D) / sqrt(d') in bf16
        const int64_t rows = B * L;
        const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
        const float scale = 1.0f / sqrtf((float)dp);
#define SRU_SM_BWD(NR)                                                                           \
    hipLaunchKernelGGL((attn_softmax_bwd<NR>), grid, block, 0, s, S, dP, D, dSp, rows, L, B, Lk, \
                       Lm, a.causal, scale)
#define SRU_SM_BWD4(NV)                                                                          \
    hipLaunchKernelGGL((attn_softmax_bwd_v4<NV>), grid, block, 0, s, S, dP, D, dSp, rows, L, B,  \
                       Lk, Lm, a.causal, scale)
        if (Lk % 4 == 0 && Lk <= 2048) {
            if (Lk <= 512)
                SRU_SM_BWD4(2);
            else if (Lk <= 1024)
                SRU_SM_BWD4(4);
            else
                SRU_SM_BWD4(8);
        } else if (Lk <= 256)
            SRU_SM_BWD(4);
        else if (Lk <= 512)
            SRU_SM_BWD(8);
        else if (Lk <= 1024)
            SRU_SM_BWD(16);
        else if (Lk <= 2048)
            SRU_SM_BWD(32);
        else
            SRU_SM_BWD(0);
#undef SRU_SM_BWD4
#undef SRU_SM_BWD
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {   // dQ_b += dS'_b K~_b (K read as [Lk, d'] = [K, N])
        GemmArgs g;
        g.M = L, g.N = dp, g.K = Lk;
        g.A = dSp, g.a_bf16 = true, g.lda = Lk, g.sa = L * Lk;
        g.Bm = KV, g.b_bf16 = true, g.b_kn = true, g.ldb = B * 2 * dp, g.sb = 2 * dp;
        g.C = dQ, g.ldc = B * dp, g.sc = dp, g.accumulate = true;
        g.batch = B;
        g.causal_klim = a.causal ? Lm : -1;   // dS' is zero at masked keys
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    {   // this segment's keys: dK_b [L, d'] = dS'_b[:, Lm:]^T Q~_b, into dKV[:, :d']
        GemmArgs g;
        g.M = L, g.N = dp, g.K = L;
        g.A = dSp + Lm, g.a_bf16 = true, g.lda = Lk, g.sa = L * Lk;
        g.Bm = Qb, g.b_bf16 = true, g.ldb = B * dp, g.sb = dp;
        g.C = (float *)dKVb, g.ldc = B * 2 * dp, g.sc = 2 * dp, g.accumulate = false;
        g.batch = B;
        if ((e = launch_gemm_tn_bf16_out(g, s)) != hipSuccess) return e;
    }
    {   // and values: dV_b [L, d'] = P_b[:, Lm:]^T dO~_b, into dKV[:, d':]
        GemmArgs g;
        g.M = L, g.N = dp, g.K = L;
        g.A = P + Lm, g.a_bf16 = true, g.lda = Lk, g.sa = L * Lk;
        g.Bm = dOb, g.b_bf16 = true, g.ldb = B * dp, g.sb = dp;
        g.C = (float *)(dKVb + dp), g.ldc = B * 2 * dp, g.sc = 2 * dp, g.accumulate = false;
        g.batch = B;
        if ((e = launch_gemm_tn_bf16_out(g, s)) != hipSuccess) return e;
    }
    {   // dWkv [2d', d'] = [dK | dV]^T Q~
        GemmArgs g;
        g.M = 2 * dp, g.N = dp, g.K = LB;
        g.A = dKVb, g.a_bf16 = true;
        g.Bm = Qb, g.b_bf16 = true;
        g.C = a.dWkv, g.accumulate = false;
        if ((e = launch_gemm_wgrad(g, false, wg, s)) != hipSuccess) return e;
    }
    {   // dQ += [dK | dV] Wkv (Wkv [2d', d'] read as [K, N])
        GemmArgs g;
        g.M = LB, g.N = dp, g.K = 2 * dp;
        g.A = dKVb, g.a_bf16 = true;
        g.Bm = a.Wkv, g.b_bf16 = true, g.b_kn = true;
        g.C = dQ, g.accumulate = true;
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    // dQ is final: rounded to bf16 once, into Q~'s space (the products that
    // read Q~ have run), for its two products below
    bf16_bits *dQb = Qb;
    if ((e = launch_round_bf16(LB * dp, dQ, dQb, s)) != hipSuccess) return e;
    {   // dWq [d', d] = dQ~^T X~
        GemmArgs g;
        g.M = dp, g.N = d, g.K = LB;
        g.A = dQb, g.a_bf16 = true;
        g.Bm = a.X, g.b_bf16 = a.x_bf16;
        g.C = a.dWq, g.accumulate = false;
        if ((e = launch_gemm_wgrad(g, false, wg, s)) != hipSuccess) return e;
    }
    // dX (+)= dQ~ Wq (Wq [d', d] read as [K, N]): both operands go straight
    // into LDS
    GemmArgs g;
    g.M = LB, g.N = d, g.K = dp;
    g.A = dQb, g.a_bf16 = true;
    g.Bm = a.Wq, g.b_bf16 = true, g.b_kn = true;
    g.C = a.dX, g.accumulate = a.dx_accumulate;
    return launch_gemm(g, s);
}

// Fused shapes: the V^T copy, then R rounded to bf16 (the U product's
// operand, copied straight into LDS by the bf16 x bf16^T kernel).
size_t fused_vt_bytes(int64_t L, int64_t B, int64_t dp, int64_t Lm)
{
    const size_t n = (size_t)B * (size_t)dp * (size_t)fused_keys_padded(Lm + L) * 2;
    return (n + 255) & ~(size_t)255;
}

size_t attention_workspace_bytes(int64_t L, int64_t B, int64_t dp, int64_t Lm)
{
    if (fused_forward_ok(L, B, dp, Lm))
        return fused_vt_bytes(L, B, dp, Lm) + (size_t)L * (size_t)B * (size_t)dp * 2;
    return ws_layout(L, B, dp, Lm).total;
}

hipError_t launch_attention_forward(const AttnArgs &a, hipStream_t s)
{
    const int64_t L = a.L, B = a.B, d = a.d, dp = a.dp, Lm = a.Lm, LB = L * B;
    const WsLayout w = ws_layout(L, B, dp, Lm);
    char *ws = (char *)a.workspace;
    float *S = (float *)(ws + w.s_off);
    bf16_bits *P = (bf16_bits *)(ws + w.p_off);
    float *O = (float *)(ws + w.o_off);
    bf16_bits *KV = (bf16_bits *)a.KV;
    hipError_t e;
    {   // Q [L*B, d'] = X~ Wq^T
        GemmArgs g;
        g.M = LB, g.N = dp, g.K = d;
        g.A = a.X, g.a_bf16 = a.x_bf16;
        g.Bm = a.Wq, g.b_bf16 = true, g.b_kn = false;
        g.C = a.Q, g.accumulate = false;
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    {   // this segment's rows of [K | V] (bf16) = Q~ [Wk; Wv]^T
        GemmArgs g;
        g.M = LB, g.N = 2 * dp, g.K = dp;
        g.A = a.Q, g.a_bf16 = false;
        g.Bm = a.Wkv, g.b_bf16 = true, g.b_kn = false;
        g.C = (float *)(KV + Lm * B * 2 * dp), g.accumulate = false;
        if ((e = launch_gemm_bf16_out(g, s)) != hipSuccess) return e;
    }
    const bool fused = fused_forward_ok(L, B, dp, Lm);
    bf16_bits *Rb = fused ? (bf16_bits *)(ws + fused_vt_bytes(L, B, dp, Lm)) : nullptr;
    if (fused) {
        if ((e = launch_fused(a, (bf16_bits *)ws, Rb, s)) != hipSuccess) return e;
    } else {
        if ((e = attend(L, B, dp, Lm, a.causal, a.Q, KV, S, P, O, s)) != hipSuccess) return e;
        if ((e = launch_residual(a, O, s)) != hipSuccess) return e;
    }
    {   // U [L*B, ndir*3d] = R~ Wo^T, fp32 or rounded to bf16; R~ is the fused
        // kernel's bf16 copy of R, or R rounded as the product loads it
        GemmArgs g;
        g.M = LB, g.N = a.n3, g.K = dp;
        g.A = fused ? (const void *)Rb : (const void *)a.R, g.a_bf16 = fused;
        g.Bm = a.Wo, g.b_bf16 = true, g.b_kn = false;
        g.C = (float *)a.U, g.accumulate = false;
        if ((e = a.u_bf16 ? launch_gemm_bf16_out(g, s) : launch_gemm(g, s)) != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace sru
