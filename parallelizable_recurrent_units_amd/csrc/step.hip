// step.hip -- one decoding step of a unidirectional SRU layer: the "run as an
// RNN at inference" side of the recurrence ("Parallelizing Legendre Memory
// Unit Training", abstract; SRU++ paper, background section, Eqs. 1-5).  For
// the B input rows of one time step, Eq. 1 gives the three gate inputs of
// every channel, and Eqs. 2-5 advance the carried state c:
//   u = x~ W^T, f = sigma(u_f + v c + b), r = sigma(u_r + v' c + b'),
//   c' = f c + (1 - f) u_cand, h = r c' + (1 - r) alpha x.
// x~ = bf16(x) (nearest even) when W is bf16, as in the projection; the
// highway term uses x itself.
//
// One wave per channel j.  It keeps rows j, d + j and 2d + j of W (the three
// gates of channel j) in registers, then for each batch row forms the three
// dot products with x~ (per-lane partial sums over 8-element pieces, then a
// wave reduction); the cell runs one batch row per lane.  W is read from
// memory once per step; x (B x d) is read by every wave from the caches.
// From 8 batch rows on, with bf16 W, step_mfma16 and step_mfma below form
// the products on the matrix cores instead.
#include "device_common.h"
#include "internal.h"

namespace sru {
namespace {

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// 8 consecutive elements as fp32 (bf16 widened exactly).
template <typename T> __device__ __forceinline__ void load8(const T *p, float (&o)[8]);
template <> __device__ __forceinline__ void load8<float>(const float *p, float (&o)[8])
{
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    o[0] = a.x, o[1] = a.y, o[2] = a.z, o[3] = a.w;
    o[4] = b.x, o[5] = b.y, o[6] = b.z, o[7] = b.w;
}
template <> __device__ __forceinline__ void load8<bf16_bits>(const bf16_bits *p, float (&o)[8])
{
    const u32x4s v = *(const u32x4s *)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(v[i] << 16);
        o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ float round_bf16(float x) { return bf16_to_f32(f32_to_bf16(x)); }

// Applies Eqs. 2-5 for (b, j) given the state c, the three gate inputs and
// the highway input xv.
__device__ __forceinline__ void cell(const StepArgs &a, int64_t b, int64_t j, float vf, float vr,
                                     float bf, float br, float c, float uf, float ur, float ux,
                                     float xv)
{
    const float yf = fmaf(vf, c, uf + bf) * kNegLog2e;
    const float yr = fmaf(vr, c, ur + br) * kNegLog2e;
    const float cn = gate_blend(yf, c, ux);              // f c + (1 - f) u_cand
    a.h[b * a.d + j] = gate_blend(yr, cn, a.alpha * xv); // r c' + (1 - r) alpha x
    a.c_next[b * a.d + j] = cn;
}

// VEC (d % 8 == 0): 8-element pieces; NC > 0: a W row of d <= 512 NC
// elements stays in registers (NC pieces per lane); NC == 0: W is re-read
// for every batch row.  Without VEC every element is loaded on its own.
// Batch row 0's x pieces are requested together with W.
// Batch rows go in groups of 64: after the wave reduction of row b0 + i,
// lane i keeps its three gate inputs, and the cell then runs for the whole
// group at once, one batch row per lane (one round of state loads).
template <typename TW, typename TX, bool VEC, int NC>
__global__ __launch_bounds__(256) void step_cell(StepArgs a)
{
    const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (j >= a.d) return;
    const int64_t d = a.d;
    const TW *W = (const TW *)a.W;
    const TX *X = (const TX *)a.x;
    const bool rnd = sizeof(TW) == 2;                    // x~ = bf16(x) with bf16 W
    const float vf = a.v[j], vr = a.v[d + j], bf = a.b[j], br = a.b[d + j];
    float w[3][NC > 0 ? NC : 1][8];
    float x0[NC > 0 ? NC : 1][8];                        // batch row 0, requested with W
    if constexpr (VEC && NC > 0) {
#pragma unroll
        for (int g = 0; g < 3; ++g)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int64_t k = 512 * c + 8 * lane;
                if (k < d)
                    load8(W + (g * d + j) * d + k, w[g][c]);
                else
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[g][c][e] = 0.0f;
            }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int64_t k = 512 * c + 8 * lane;
            if (k < d)
                load8(X + k, x0[c]);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e) x0[c][e] = 0.0f;
        }
    }
    // the three dot products of batch row b, summed over the wave
    auto dots = [&](int64_t b, float (&u)[3]) {
        float s[3] = {0.0f, 0.0f, 0.0f};
        if constexpr (VEC && NC > 0) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int64_t k = 512 * c + 8 * lane;
                if (k >= d) continue;
                float xv[8];
                if (b == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) xv[e] = x0[c][e];
                } else {
                    load8(X + b * d + k, xv);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float xt = rnd ? round_bf16(xv[e]) : xv[e];
#pragma unroll
                    for (int g = 0; g < 3; ++g) s[g] = fmaf(w[g][c][e], xt, s[g]);
                }
            }
        } else if constexpr (VEC) {
            for (int64_t k = 8 * lane; k < d; k += 512) {
                float xv[8], wv[8];
                load8(X + b * d + k, xv);
#pragma unroll
                for (int g = 0; g < 3; ++g) {
                    load8(W + (g * d + j) * d + k, wv);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        s[g] = fmaf(wv[e], rnd ? round_bf16(xv[e]) : xv[e], s[g]);
                }
            }
        } else {
            for (int64_t k = lane; k < d; k += 64) {
                const float xv = load_as_f32(X + b * d + k);
                const float xt = rnd ? round_bf16(xv) : xv;
#pragma unroll
                for (int g = 0; g < 3; ++g)
                    s[g] = fmaf(load_as_f32(W + (g * d + j) * d + k), xt, s[g]);
            }
        }
#pragma unroll
        for (int g = 0; g < 3; ++g) u[g] = wave_sum(s[g]);
    };
    for (int64_t b0 = 0; b0 < a.B; b0 += 64) {
        const int nb = a.B - b0 < 64 ? (int)(a.B - b0) : 64;
        // this lane's state and highway input, requested before the products
        float cp = 0.0f, xh = 0.0f;
        if (lane < nb) {
            const int64_t b = b0 + lane;
            if (a.c_prev) cp = a.c_prev[b * d + j];
            xh = load_as_f32(X + b * d + j);
        }
        float mine[3] = {0.0f, 0.0f, 0.0f};
        for (int i = 0; i < nb; ++i) {
            float u[3];
            dots(b0 + i, u);
            if (lane == i) {
                mine[0] = u[0];
                mine[1] = u[1];
                mine[2] = u[2];
            }
        }
        if (lane < nb) cell(a, b0 + lane, j, vf, vr, bf, br, cp, mine[0], mine[1], mine[2], xh);
    }
}

// Batches of rows with bf16 W (d % 32 == 0, d <= 2048): the products as
// bf16 MFMAs.  A block owns 32 channels and 32 batch rows.  It rounds its x
// rows to bf16 into LDS once (row pitch d + 8 keeps the fragment reads of
// eight rows on different banks); wave w multiplies them by the 32 W rows of
// gate w % 3 over part w / 3 of the KP parts of the reduction
// (v_mfma_f32_32x32x16_bf16, W fragments loaded straight from memory, 16 at
// a time, the first 16 requested together with the x rows); the parts meet
// in LDS, over the x~ rows, and the block applies the cell to its 32 x 32
// (batch row, channel) pairs, whose state and highway inputs it also loaded
// before the products.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kStepRows = 32;

// four consecutive x values rounded to bf16, as two packed pairs
template <typename TX> __device__ __forceinline__ uint2 load4_bf16(const TX *p);
template <> __device__ __forceinline__ uint2 load4_bf16<float>(const float *p)
{
    const float4 v = *(const float4 *)p;
    return uint2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
}
template <> __device__ __forceinline__ uint2 load4_bf16<bf16_bits>(const bf16_bits *p)
{
    return *(const uint2 *)p;                            // already bf16: x~ = x
}

template <typename TX, int KP>
__global__ __launch_bounds__(192 * KP) void step_mfma(StepArgs a)
{
    constexpr int NT = 192 * KP;                         // 3 gates x KP parts, one wave each
    constexpr int NP = (kStepRows * 32 + NT - 1) / NT;   // cell pairs per thread
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int d = (int)a.d, P = d + 8;                   // LDS row pitch (bf16)
    bf16_bits *xs = (bf16_bits *)smem;                   // [32][P]
    float *red = (float *)smem;                          // [KP][3][32][33], after the products
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ngroups = d / 32;
    const int j0 = (int)(blockIdx.x % ngroups) * 32;
    const int64_t b0 = (int64_t)(blockIdx.x / ngroups) * kStepRows;
    const TX *X = (const TX *)a.x;
    const bf16_bits *W = (const bf16_bits *)a.W;

    // the first U W fragments of this wave (gate wave % 3, part wave / 3 of
    // the reduction), the cell's per-pair inputs and the x rows are all
    // requested before anything waits on them
    const int g = wave % 3, kp = wave / 3;
    const int part = d / KP, steps = part / 16;
    const int r32 = lane & 31, hi = lane >> 5;
    const bf16_bits *wrow = W + (int64_t)(g * d + j0 + r32) * d + kp * part + 8 * hi;
    constexpr int U = 16;
    bf16x8_t wf[U];
    auto load_w = [&](int ks) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ks + u < steps) wf[u] = *(const bf16x8_t *)(wrow + 16 * (ks + u));
    };
    load_w(0);

    float cp[NP], xv[NP], vf[NP], vr[NP], bf[NP], br[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int idx = tid + p * NT, r = idx / 32, j = j0 + idx % 32;
        const int64_t b = b0 + r;
        cp[p] = xv[p] = vf[p] = vr[p] = bf[p] = br[p] = 0.0f;
        if (idx < kStepRows * 32 && b < a.B) {
            cp[p] = a.c_prev ? a.c_prev[b * d + j] : 0.0f;
            xv[p] = load_as_f32(X + b * d + j);
            vf[p] = a.v[j], vr[p] = a.v[d + j], bf[p] = a.b[j], br[p] = a.b[d + j];
        }
    }

    // x~ rows b0 .. b0 + 31 (rows past B repeat the last one; never written),
    // SB 4-element pieces per thread in flight
    const int q = d / 4, total = kStepRows * q;
    constexpr int SB = 8;
    for (int base = 0; base < total; base += SB * NT) {
        uint2 v[SB];
#pragma unroll
        for (int s = 0; s < SB; ++s) {
            const int i = base + s * NT + tid;
            v[s] = uint2{0u, 0u};
            if (i < total) {
                const int r = i / q, k = 4 * (i - r * q);
                const int64_t b = b0 + r < a.B ? b0 + r : a.B - 1;
                v[s] = load4_bf16(X + b * d + k);
            }
        }
#pragma unroll
        for (int s = 0; s < SB; ++s) {
            const int i = base + s * NT + tid;
            if (i < total) {
                const int r = i / q, k = 4 * (i - r * q);
                *(uint2 *)(xs + r * P + k) = v[s];
            }
        }
    }
    __syncthreads();

    const bf16_bits *xrow = xs + r32 * P + kp * part + 8 * hi;
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    for (int ks = 0;;) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ks + u < steps) {
                const bf16x8_t xf = *(const bf16x8_t *)(xrow + 16 * (ks + u));
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, wf[u], acc, 0, 0, 0);
            }
        ks += U;
        if (ks >= steps) break;
        load_w(ks);
    }
    __syncthreads();                                     // x~ no longer read: red may overwrite it
    // acc holds row (batch) 8 (r / 4) + 4 hi + r % 4, column (channel) r32
    float *rw = red + ((kp * 3 + g) * 32) * 33;
#pragma unroll
    for (int r = 0; r < 16; ++r) rw[(8 * (r / 4) + 4 * hi + (r % 4)) * 33 + r32] = acc[r];
    __syncthreads();

#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int idx = tid + p * NT, r = idx / 32, n = idx % 32;
        const int64_t b = b0 + r;
        if (idx >= kStepRows * 32 || b >= a.B) continue;
        float u[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int gg = 0; gg < 3; ++gg)
#pragma unroll
            for (int k = 0; k < KP; ++k) u[gg] += red[((k * 3 + gg) * 32 + r) * 33 + n];
        cell(a, b, j0 + n, vf[p], vr[p], bf[p], br[p], cp[p], u[0], u[1], u[2], xv[p]);
    }
}

template <int KP> size_t step_mfma_lds(int64_t d)
{
    const size_t xs = (size_t)kStepRows * (d + 8) * 2, red = (size_t)KP * 3 * 32 * 33 * 4;
    return xs > red ? xs : red;
}

template <typename TX, int KP> hipError_t step_mfma_launch(const StepArgs &a, hipStream_t s)
{
    static const hipError_t attr = hipFuncSetAttribute(
        (const void *)step_mfma<TX, KP>, hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)step_mfma_lds<KP>(2048));
    if (attr != hipSuccess) return attr;
    const int64_t blocks = (a.d / 32) * ((a.B + kStepRows - 1) / kStepRows);
    hipLaunchKernelGGL((step_mfma<TX, KP>), dim3((unsigned)blocks), dim3(192 * KP),
                       step_mfma_lds<KP>(a.d), s, a);
    return hipGetLastError();
}

// The same with 16 channels x 16 batch rows per block
// (v_mfma_f32_16x16x32_bf16): half the W rows and x rows per block, so four
// times the blocks, for batches too small to occupy the chip with 32 x 32
// blocks.  Operand lane l holds row l % 16 (a batch row of x~, a channel's W
// row) and k-chunk l / 16 of the 32-deep step; the accumulator holds column
// (channel) l % 16, rows (batch) 4 (l / 16) .. + 3.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kStep16 = 16;

template <typename TX, int KP>
__global__ __launch_bounds__(192 * KP) void step_mfma16(StepArgs a)
{
    constexpr int NT = 192 * KP;
    constexpr int NP = (kStep16 * kStep16 + NT - 1) / NT;   // cell pairs per thread
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int d = (int)a.d, P = d + 8;                   // LDS row pitch (bf16)
    bf16_bits *xs = (bf16_bits *)smem;                   // [16][P]
    float *red = (float *)smem;                          // [KP][3][16][17], after the products
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ngroups = d / kStep16;
    const int j0 = (int)(blockIdx.x % ngroups) * kStep16;
    const int64_t b0 = (int64_t)(blockIdx.x / ngroups) * kStep16;
    const TX *X = (const TX *)a.x;
    const bf16_bits *W = (const bf16_bits *)a.W;

    const int g = wave % 3, kp = wave / 3;
    const int part = d / KP, steps = part / 32;
    const int r16 = lane & 15, q4 = lane >> 4;
    const bf16_bits *wrow = W + (int64_t)(g * d + j0 + r16) * d + kp * part + 8 * q4;
    constexpr int U = 16;
    bf16x8_t wf[U];
    auto load_w = [&](int ks) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ks + u < steps) wf[u] = *(const bf16x8_t *)(wrow + 32 * (ks + u));
    };
    load_w(0);

    float cp[NP], xv[NP], vf[NP], vr[NP], bf[NP], br[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int idx = tid + p * NT, r = idx / kStep16, j = j0 + idx % kStep16;
        const int64_t b = b0 + r;
        cp[p] = xv[p] = vf[p] = vr[p] = bf[p] = br[p] = 0.0f;
        if (idx < kStep16 * kStep16 && b < a.B) {
            cp[p] = a.c_prev ? a.c_prev[b * d + j] : 0.0f;
            xv[p] = load_as_f32(X + b * d + j);
            vf[p] = a.v[j], vr[p] = a.v[d + j], bf[p] = a.b[j], br[p] = a.b[d + j];
        }
    }

    // x~ rows b0 .. b0 + 15 (rows past B repeat the last one; never written)
    const int q = d / 4, total = kStep16 * q;
    constexpr int SB = 8;
    for (int base = 0; base < total; base += SB * NT) {
        uint2 v[SB];
#pragma unroll
        for (int s = 0; s < SB; ++s) {
            const int i = base + s * NT + tid;
            v[s] = uint2{0u, 0u};
            if (i < total) {
                const int r = i / q, k = 4 * (i - r * q);
                const int64_t b = b0 + r < a.B ? b0 + r : a.B - 1;
                v[s] = load4_bf16(X + b * d + k);
            }
        }
#pragma unroll
        for (int s = 0; s < SB; ++s) {
            const int i = base + s * NT + tid;
            if (i < total) {
                const int r = i / q, k = 4 * (i - r * q);
                *(uint2 *)(xs + r * P + k) = v[s];
            }
        }
    }
    __syncthreads();

    const bf16_bits *xrow = xs + r16 * P + kp * part + 8 * q4;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int ks = 0;;) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ks + u < steps) {
                const bf16x8_t xf = *(const bf16x8_t *)(xrow + 32 * (ks + u));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf, wf[u], acc, 0, 0, 0);
            }
        ks += U;
        if (ks >= steps) break;
        load_w(ks);
    }
    __syncthreads();                                     // x~ no longer read: red may overwrite it
    float *rw = red + ((kp * 3 + g) * kStep16) * 17;
#pragma unroll
    for (int i = 0; i < 4; ++i) rw[(4 * q4 + i) * 17 + r16] = acc[i];
    __syncthreads();

#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int idx = tid + p * NT, r = idx / kStep16, n = idx % kStep16;
        const int64_t b = b0 + r;
        if (idx >= kStep16 * kStep16 || b >= a.B) continue;
        float u[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int gg = 0; gg < 3; ++gg)
#pragma unroll
            for (int k = 0; k < KP; ++k) u[gg] += red[((k * 3 + gg) * kStep16 + r) * 17 + n];
        cell(a, b, j0 + n, vf[p], vr[p], bf[p], br[p], cp[p], u[0], u[1], u[2], xv[p]);
    }
}

template <int KP> size_t step_mfma16_lds(int64_t d)
{
    const size_t xs = (size_t)kStep16 * (d + 8) * 2, red = (size_t)KP * 3 * kStep16 * 17 * 4;
    return xs > red ? xs : red;
}

template <typename TX, int KP> hipError_t step_mfma16_launch(const StepArgs &a, hipStream_t s)
{
    static const hipError_t attr = hipFuncSetAttribute(
        (const void *)step_mfma16<TX, KP>, hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)step_mfma16_lds<KP>(2048));
    if (attr != hipSuccess) return attr;
    const int64_t blocks = (a.d / kStep16) * ((a.B + kStep16 - 1) / kStep16);
    hipLaunchKernelGGL((step_mfma16<TX, KP>), dim3((unsigned)blocks), dim3(192 * KP),
                       step_mfma16_lds<KP>(a.d), s, a);
    return hipGetLastError();
}

// A block's time goes with the bytes it streams (its W rows and its x rows),
// and blocks beyond the 256 CUs run in further rounds: the smaller blocks
// when they finish sooner by that measure.
bool step_small_blocks(const StepArgs &a)
{
    const int64_t sx = a.x_bf16 ? 2 : 4;
    auto est = [&](int64_t ch) {
        const int64_t blocks = (a.d / ch) * ((a.B + ch - 1) / ch);
        return (blocks + 255) / 256 * (3 * ch * a.d * 2 + ch * a.d * sx);
    };
    return est(kStep16) < est(kStepRows);
}

template <typename TW, typename TX>
hipError_t step_launch(const StepArgs &a, hipStream_t s)
{
    if constexpr (sizeof(TW) == 2) {
        if (a.B >= 8 && a.d % 32 == 0 && a.d <= 2048) {
            if (step_small_blocks(a))
                return a.d % 128 == 0  ? step_mfma16_launch<TX, 4>(a, s)
                       : a.d % 64 == 0 ? step_mfma16_launch<TX, 2>(a, s)
                                       : step_mfma16_launch<TX, 1>(a, s);
            return a.d % 64 == 0 ? step_mfma_launch<TX, 4>(a, s) : step_mfma_launch<TX, 2>(a, s);
        }
    }
    const dim3 grid((unsigned)((a.d + 3) / 4)), block(256);
    const bool vec = a.d % 8 == 0;
    if (vec && a.d <= 512)
        hipLaunchKernelGGL((step_cell<TW, TX, true, 1>), grid, block, 0, s, a);
    else if (vec && a.d <= 1024)
        hipLaunchKernelGGL((step_cell<TW, TX, true, 2>), grid, block, 0, s, a);
    else if (vec && a.d <= 2048)
        hipLaunchKernelGGL((step_cell<TW, TX, true, 4>), grid, block, 0, s, a);
    else if (vec)
        hipLaunchKernelGGL((step_cell<TW, TX, true, 0>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((step_cell<TW, TX, false, 0>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const StepArgs &a, hipStream_t s)
{
    if (a.w_bf16)
        return a.x_bf16 ? step_launch<bf16_bits, bf16_bits>(a, s) : step_launch<bf16_bits, float>(a, s);
    return a.x_bf16 ? step_launch<float, bf16_bits>(a, s) : step_launch<float, float>(a, s);
}

}  // namespace sru
