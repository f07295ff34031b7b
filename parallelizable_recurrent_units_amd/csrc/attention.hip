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

// ---- backward -----------------------------------------------------------

constexpr int kResRowsPerWave = 16;   // rows of attn_residual_bwd per wave (64 per block)

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

// dgamma, dbeta (when ln) and dalpha: the blocks' partial rows added in block
// order (bit-reproducible run to run).
__global__ __launch_bounds__(256) void attn_part_reduce(const float *__restrict__ part,
                                                        int64_t nblk, int64_t dp,
                                                        float *__restrict__ dgamma,
                                                        float *__restrict__ dbeta,
                                                        float *__restrict__ dalpha)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= 2 * dp + 1) return;
    float acc = 0.0f;
    for (int64_t b = 0; b < nblk; ++b) acc += part[b * (2 * dp + 1) + e];
    if (e < dp) {
        if (dgamma) dgamma[e] = acc;
    } else if (e < 2 * dp) {
        if (dbeta) dbeta[e - dp] = acc;
    } else {
        *dalpha = acc;
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
                  const bf16_bits *KV, float *S, bf16_bits *P, float *O, hipStream_t s)
{
    const int64_t Lk = Lm + L;
    hipError_t e;
    {
        GemmArgs g;
        g.M = L, g.N = Lk, g.K = dp;
        g.A = Q, g.a_bf16 = false, g.lda = B * dp, g.sa = dp;
        g.Bm = KV, g.b_bf16 = true, g.b_kn = false, g.ldb = B * 2 * dp, g.sb = 2 * dp;
        g.C = S, g.ldc = Lk, g.sc = L * Lk, g.accumulate = false;
        g.batch = B;
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    if ((e = launch_softmax(L, B, dp, Lm, causal, S, P, s)) != hipSuccess) return e;
    GemmArgs g;
    g.M = L, g.N = dp, g.K = Lk;
    g.A = P, g.a_bf16 = true, g.lda = Lk, g.sa = L * Lk;
    g.Bm = KV + dp, g.b_bf16 = true, g.b_kn = true, g.ldb = B * 2 * dp, g.sb = 2 * dp;
    g.C = O, g.ldc = B * dp, g.sc = dp, g.accumulate = false;
    g.batch = B;
    return launch_gemm(g, s);
}

// Workspace of the backward (bytes, each region 256-byte aligned).
struct BwdLayout {
    size_t s_off, p_off, dp_off, dsp_off, o_off, dr_off, dq_off, do_off, dkv_off, d_off,
        part_off, wg_off, total;
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
    w.dkv_off = take(LB * 2 * dp * 4);
    w.d_off = take(LB * 4);
    w.part_off = take((size_t)w.nblk * (size_t)(2 * dp + 1) * 4);
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
    float *dKV = (float *)(ws + w.dkv_off);
    float *D = (float *)(ws + w.d_off);
    float *part = (float *)(ws + w.part_off);
    float *wg = (float *)(ws + w.wg_off);
    const bf16_bits *KV = a.KV;
    hipError_t e;
    // the forward's weights and A, recomputed from Q and KV
    if ((e = attend(L, B, dp, Lm, a.causal, a.Q, KV, S, P, O, s)) != hipSuccess) return e;
    {   // dR [LB, d'] = dU Wo (Wo [n3, d'] read as [K, N])
        GemmArgs g;
        g.M = LB, g.N = dp, g.K = n3;
        g.A = a.dU, g.a_bf16 = a.du_bf16;
        g.Bm = a.Wo, g.b_bf16 = true, g.b_kn = true;
        g.C = dR, g.accumulate = false;
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    {   // dWo [n3, d'] = dU^T R~
        GemmArgs g;
        g.M = n3, g.N = dp, g.K = LB;
        g.A = a.dU, g.a_bf16 = a.du_bf16;
        g.Bm = a.R, g.b_bf16 = false;
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
        hipLaunchKernelGGL(attn_part_reduce, dim3((unsigned)((2 * dp + 1 + 255) / 256)), dim3(256),
                           0, s, part, w.nblk, dp, a.layernorm ? a.dgamma : nullptr,
                           a.layernorm ? a.dbeta : nullptr, a.dalpha);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {   // dP_b [L, Lk] = dO~_b V~_b^T
        GemmArgs g;
        g.M = L, g.N = Lk, g.K = dp;
        g.A = dO, g.a_bf16 = false, g.lda = B * dp, g.sa = dp;
        g.Bm = KV + dp, g.b_bf16 = true, g.b_kn = false, g.ldb = B * 2 * dp, g.sb = 2 * dp;
        g.C = dP, g.ldc = Lk, g.sc = L * Lk, g.accumulate = false;
        g.batch = B;
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    {   // dS' = p (dP - D) / sqrt(d') in bf16
        const int64_t rows = B * L;
        const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
        const float scale = 1.0f / sqrtf((float)dp);
#define SRU_SM_BWD(NR)                                                                           \
    hipLaunchKernelGGL((attn_softmax_bwd<NR>), grid, block, 0, s, S, dP, D, dSp, rows, L, B, Lk, \
                       Lm, a.causal, scale)
        if (Lk <= 256)
            SRU_SM_BWD(4);
        else if (Lk <= 512)
            SRU_SM_BWD(8);
        else if (Lk <= 1024)
            SRU_SM_BWD(16);
        else if (Lk <= 2048)
            SRU_SM_BWD(32);
        else
            SRU_SM_BWD(0);
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
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    {   // this segment's keys: dK_b [L, d'] = dS'_b[:, Lm:]^T Q~_b, into dKV[:, :d']
        GemmArgs g;
        g.M = L, g.N = dp, g.K = L;
        g.A = dSp + Lm, g.a_bf16 = true, g.lda = Lk, g.sa = L * Lk;
        g.Bm = a.Q, g.b_bf16 = false, g.ldb = B * dp, g.sb = dp;
        g.C = dKV, g.ldc = B * 2 * dp, g.sc = 2 * dp, g.accumulate = false;
        g.batch = B;
        if ((e = launch_gemm_tn(g, s)) != hipSuccess) return e;
    }
    {   // and values: dV_b [L, d'] = P_b[:, Lm:]^T dO~_b, into dKV[:, d':]
        GemmArgs g;
        g.M = L, g.N = dp, g.K = L;
        g.A = P + Lm, g.a_bf16 = true, g.lda = Lk, g.sa = L * Lk;
        g.Bm = dO, g.b_bf16 = false, g.ldb = B * dp, g.sb = dp;
        g.C = dKV + dp, g.ldc = B * 2 * dp, g.sc = 2 * dp, g.accumulate = false;
        g.batch = B;
        if ((e = launch_gemm_tn(g, s)) != hipSuccess) return e;
    }
    {   // dWkv [2d', d'] = [dK | dV]^T Q~
        GemmArgs g;
        g.M = 2 * dp, g.N = dp, g.K = LB;
        g.A = dKV, g.a_bf16 = false;
        g.Bm = a.Q, g.b_bf16 = false;
        g.C = a.dWkv, g.accumulate = false;
        if ((e = launch_gemm_wgrad(g, false, wg, s)) != hipSuccess) return e;
    }
    {   // dQ += [dK | dV] Wkv (Wkv [2d', d'] read as [K, N])
        GemmArgs g;
        g.M = LB, g.N = dp, g.K = 2 * dp;
        g.A = dKV, g.a_bf16 = false;
        g.Bm = a.Wkv, g.b_bf16 = true, g.b_kn = true;
        g.C = dQ, g.accumulate = true;
        if ((e = launch_gemm(g, s)) != hipSuccess) return e;
    }
    {   // dWq [d', d] = dQ^T X~
        GemmArgs g;
        g.M = dp, g.N = d, g.K = LB;
        g.A = dQ, g.a_bf16 = false;
        g.Bm = a.X, g.b_bf16 = a.x_bf16;
        g.C = a.dWq, g.accumulate = false;
        if ((e = launch_gemm_wgrad(g, false, wg, s)) != hipSuccess) return e;
    }
    // dX (+)= dQ Wq (Wq [d', d] read as [K, N])
    GemmArgs g;
    g.M = LB, g.N = d, g.K = dp;
    g.A = dQ, g.a_bf16 = false;
    g.Bm = a.Wq, g.b_bf16 = true, g.b_kn = true;
    g.C = a.dX, g.accumulate = a.dx_accumulate;
    return launch_gemm(g, s);
}

size_t attention_workspace_bytes(int64_t L, int64_t B, int64_t dp, int64_t Lm)
{
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
    if ((e = attend(L, B, dp, Lm, a.causal, a.Q, KV, S, P, O, s)) != hipSuccess) return e;
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
