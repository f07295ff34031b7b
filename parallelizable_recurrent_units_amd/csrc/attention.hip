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

hipError_t launch_softmax(const AttnArgs &a, const float *S, bf16_bits *P, hipStream_t s)
{
    const int64_t rows = a.B * a.L, Lk = a.Lm + a.L;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    const float scale = 1.0f / sqrtf((float)a.dp);
#define SRU_SOFTMAX(NR)                                                                        \
    hipLaunchKernelGGL((attn_softmax<NR>), grid, block, 0, s, S, P, rows, a.L, Lk, a.Lm,      \
                       a.causal, scale)
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

}  // namespace

size_t attention_workspace_bytes(int64_t L, int64_t B, int64_t dp, int64_t Lm)
{
    return ws_layout(L, B, dp, Lm).total;
}

hipError_t launch_attention_forward(const AttnArgs &a, hipStream_t s)
{
    const int64_t L = a.L, B = a.B, d = a.d, dp = a.dp, Lm = a.Lm, Lk = Lm + L, LB = L * B;
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
    {   // S_b [L, Lk] = Q~_b K_b^T for every sequence b (rows t*B + b)
        GemmArgs g;
        g.M = L, g.N = Lk, g.K = dp;
        g.A = a.Q, g.a_bf16 = false, g.lda = B * dp, g.sa = dp;
        g.Bm = KV, g.b_bf16 = true, g.b_kn = false, g.ldb = B * 2 * dp, g.sb = 2 * dp;
        g.C = S, g.ldc = Lk, g.sc = L * Lk, g.accumulate = false;
        g.batch = B;
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    if ((e = launch_softmax(a, S, P, s)) != hipSuccess) return e;
    {   // O_b [L, d'] (rows t*B + b of O) = P_b V_b
        GemmArgs g;
        g.M = L, g.N = dp, g.K = Lk;
        g.A = P, g.a_bf16 = true, g.lda = Lk, g.sa = L * Lk;
        g.Bm = KV + dp, g.b_bf16 = true, g.b_kn = true, g.ldb = B * 2 * dp, g.sb = 2 * dp;
        g.C = O, g.ldc = B * dp, g.sc = dp, g.accumulate = false;
        g.batch = B;
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    if ((e = launch_residual(a, O, s)) != hipSuccess) return e;
    {   // U [L*B, ndir*3d] = R~ Wo^T, fp32 or rounded to bf16
        GemmArgs g;
        g.M = LB, g.N = a.n3, g.K = dp;
        g.A = a.R, g.a_bf16 = false;
        g.Bm = a.Wo, g.b_bf16 = true, g.b_kn = false;
        g.C = (float *)a.U, g.accumulate = false;
        if ((e = a.u_bf16 ? launch_gemm_bf16_out(g, s) : launch_gemm(g, s)) != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace sru
