/*
 * sru_oracle.c -- plain, slow, double-precision CPU oracle for one SRU layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * What it computes, and where that is defined:
 *
 *   Lei, "When Attention Meets Fast Recurrence: Training Language Models with
 *   Reduced Compute" (SRU++ paper), background section on the Simple Recurrent
 *   Unit, unnumbered cell equations and Eqs. 1-5:
 *     U^T = [W; W'; W''] X^T                          (Eq. 1, one projection)
 *     f[t] = sigma(U[t,0] + v  * c[t-1] + b )         (Eq. 2)
 *     r[t] = sigma(U[t,1] + v' * c[t-1] + b')         (Eq. 3)
 *     c[t] = f[t] * c[t-1] + (1 - f[t]) * U[t,2]      (Eq. 4)
 *     h[t] = r[t] * c[t] + (1 - r[t]) * x[t]          (Eq. 5)
 *   Every channel of every sequence is an independent chain once U is known
 *   (the remark after Eq. 5), so the oracle is written per chain.
 *   The projection's two gradients (input and weights) are the chain rule
 *   through Eq. 1.
 *   The factorised projection (same paper, Fig. 2(b)): U = W_o (W_q X) with a
 *   small inner dimension d'; it and its gradients are plain products
 *   (sru_oracle_matmul).
 *   The SRU++ attention that produces U (same paper, section on SRU++):
 *   Q = W_q X^T, K = W_k Q, V = W_v Q, A^T = softmax(Q^T K / sqrt(d')) V^T,
 *   U^T = W_o (Q + alpha A), optionally with layer normalisation of
 *   Q + alpha A (sru_oracle_attention, sru_oracle_layernorm, and products).
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - the highway input is scaled by a scalar alpha: (1 - r) * alpha * x;
 *     alpha = 1 gives Eq. 5 exactly;
 *   - c[-1] = c0 is an input (0 when absent);
 *   - a bidirectional layer is two independent directions; direction 1 walks
 *     t = L-1 .. 0 and its c0 is the state before t = L-1;
 *   - the backward pass is the chain rule applied to the equations above (the
 *     pages print none);
 *   - the linear mode ("Parallelizing Legendre Memory Unit Training",
 *     abstract: linear recurrences can be trained in parallel) is the same
 *     recurrence with v = v' = 0.  These are structural zeros: the gates do
 *     not see the state, so no v * c term is formed at all (with a NaN state,
 *     0 * NaN would be NaN although the linear cell's gates do not depend on
 *     it).  For finite values this is the v = 0 evaluation exactly.  The
 *     oracle evaluates it sequentially; it never chunks.
 *
 * All arithmetic is in double.  Inputs arrive as float (fp32, or bf16 values
 * widened exactly to fp32) and are widened once.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Logistic sigmoid in double; the two branches avoid overflow of exp. */
static double oracle_sigmoid(double z)
{
    if (z >= 0.0)
        return 1.0 / (1.0 + exp(-z));
    double e = exp(z);
    return e / (1.0 + e);
}

double sru_oracle_sigmoid(double z) { return oracle_sigmoid(z); }

/*
 * Round an fp32 value to the nearest bfloat16 (ties to even) and return it
 * widened back to fp32.  bfloat16 keeps the upper 16 bits of the fp32 pattern.
 * NaN stays NaN (quietened); infinities and zeros pass through.
 */
float sru_oracle_round_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u) {          /* inf or nan */
        if (u & 0x007fffffu)
            u |= 0x00400000u;                          /* quiet nan */
        u &= 0xffff0000u;
    } else {
        uint32_t lower = u & 0xffffu;
        uint32_t upper = u >> 16;
        if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
            upper += 1u;                               /* may carry into exponent */
        u = upper << 16;
    }
    float y;
    memcpy(&y, &u, sizeof y);
    return y;
}

/* sru_oracle_round_bf16 applied to n values. */
void sru_oracle_round_bf16_n(int64_t n, const float *in, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = sru_oracle_round_bf16(in[i]);
}

/*
 * Plain matrix product in double: C[m][n] = sum_{k<K} A(m, k) B(k, n), the
 * terms added in increasing k, with
 *   A(m, k) = A[m*K + k] (A stored [M, K]) or, when a_km, A[k*M + m] ([K, M]);
 *   B(k, n) = B[n*K + k] (B stored [N, K]) when b_nk, else B[k*N + n] ([K, N]).
 * The factorised projection of the SRU++ paper (Fig. 2(b): U = W_o (W_q X),
 * a small inner dimension d') and its gradients are products of this form.
 */
void sru_oracle_matmul(int64_t M, int64_t N, int64_t K, const double *A, int a_km,
                       const double *B, int b_nk, double *C)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double a = a_km ? A[k * M + m] : A[m * K + k];
                const double b = b_nk ? B[n * K + k] : B[k * N + n];
                s += a * b;
            }
            C[m * N + n] = s;
        }
    }
}

/*
 * The attention of an SRU++ layer (SRU++ paper, section on SRU++): single
 * head, scaled dot product.  For every sequence b and query step t:
 *   s_j = (Q[t] . K[j]) / sqrt(dp)  over the keys j the query may see,
 *   p_j = exp(s_j - max s) / sum_i exp(s_i - max s),
 *   A[t] = sum_j p_j V[j].
 * Keys and values are [Lk, B, dp] with Lk = Lm + L: the first Lm rows are the
 * previous segment's (context carried over, the paper's training setup) and
 * row Lm + t belongs to step t of this segment.  Without `causal` every query
 * sees all Lk keys; with it, query t sees keys j <= Lm + t.
 * round_p != 0: p_j is rounded to bf16 after normalisation, the value the
 * GPU path multiplies (the sum then uses the rounded weights).
 * Q [L, B, dp]; A [L, B, dp].  Every (b, t) is independent.
 */
void sru_oracle_attention(int64_t L, int64_t B, int64_t dp, int64_t Lm, int causal,
                          const double *Q, const double *K, const double *V, int round_p,
                          double *A)
{
    const int64_t Lk = Lm + L;
    const double scale = 1.0 / sqrt((double)dp);
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)Lk);
#pragma omp for schedule(static)
        for (int64_t bt = 0; bt < L * B; ++bt) {
            const int64_t t = bt / B, b = bt % B;
            const double *q = Q + (t * B + b) * dp;
            const int64_t nk = causal ? Lm + t + 1 : Lk;
            double mx = -INFINITY;
            for (int64_t j = 0; j < nk; ++j) {
                const double *k = K + (j * B + b) * dp;
                double s = 0.0;
                for (int64_t e = 0; e < dp; ++e)
                    s += q[e] * k[e];
                p[j] = s * scale;
                if (p[j] > mx)
                    mx = p[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                p[j] = exp(p[j] - mx);
                l += p[j];
            }
            for (int64_t j = 0; j < nk; ++j) {
                p[j] /= l;
                if (round_p)
                    p[j] = (double)sru_oracle_round_bf16((float)p[j]);
            }
            double *a = A + (t * B + b) * dp;
            for (int64_t e = 0; e < dp; ++e)
                a[e] = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                const double *v = V + (j * B + b) * dp;
                for (int64_t e = 0; e < dp; ++e)
                    a[e] += p[j] * v[e];
            }
        }
        free(p);
    }
}

/*
 * Layer normalisation over the last dimension (Ba et al.; the SRU++ paper
 * applies it to Q + alpha A before the output projection): for each of the
 * n rows of width w, y = gamma * (x - mean) / sqrt(var + eps) + beta with the
 * biased variance (mean of squared deviations).
 */
void sru_oracle_layernorm(int64_t n, int64_t w, const double *x, const double *gamma,
                          const double *beta, double eps, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const double *r = x + i * w;
        double mean = 0.0;
        for (int64_t e = 0; e < w; ++e)
            mean += r[e];
        mean /= (double)w;
        double var = 0.0;
        for (int64_t e = 0; e < w; ++e)
            var += (r[e] - mean) * (r[e] - mean);
        var /= (double)w;
        const double inv = 1.0 / sqrt(var + eps);
        for (int64_t e = 0; e < w; ++e)
            y[i * w + e] = gamma[e] * (r[e] - mean) * inv + beta[e];
    }
}

/*
 * Gradient of sru_oracle_attention with respect to Q, K and V, given the
 * gradient dA of its output (chain rule; the pages give no backward).  With
 * p the weights of query t and s the scaled scores:
 *   dV[j] += p_j dA[t]                       (A[t] = sum_j p_j V[j])
 *   g_j    = dA[t] . V[j],  D = sum_j p_j g_j
 *   ds_j   = p_j (g_j - D)                   (softmax Jacobian)
 *   dQ[t]  = sum_j ds_j K[j] / sqrt(dp),  dK[j] += ds_j Q[t] / sqrt(dp)
 * over the keys j the query sees (masked keys take no gradient).  Layouts as
 * in sru_oracle_attention; dQ [L, B, dp] is written, dK and dV [Lk, B, dp]
 * are written (summed over the queries that see each key).  Sequences are
 * independent: the loop over b runs in parallel, t and j in order.
 */
void sru_oracle_attention_backward(int64_t L, int64_t B, int64_t dp, int64_t Lm, int causal,
                                   const double *Q, const double *K, const double *V,
                                   const double *dA, double *dQ, double *dK, double *dV)
{
    const int64_t Lk = Lm + L;
    const double scale = 1.0 / sqrt((double)dp);
    for (int64_t i = 0; i < Lk * B * dp; ++i) {
        dK[i] = 0.0;
        dV[i] = 0.0;
    }
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)Lk);
        double *g = (double *)malloc(sizeof(double) * (size_t)Lk);
#pragma omp for schedule(static)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t t = 0; t < L; ++t) {
                const double *q = Q + (t * B + b) * dp;
                const double *da = dA + (t * B + b) * dp;
                const int64_t nk = causal ? Lm + t + 1 : Lk;
                double mx = -INFINITY;
                for (int64_t j = 0; j < nk; ++j) {
                    const double *k = K + (j * B + b) * dp;
                    double s = 0.0;
                    for (int64_t e = 0; e < dp; ++e)
                        s += q[e] * k[e];
                    p[j] = s * scale;
                    if (p[j] > mx)
                        mx = p[j];
                }
                double l = 0.0;
                for (int64_t j = 0; j < nk; ++j) {
                    p[j] = exp(p[j] - mx);
                    l += p[j];
                }
                double D = 0.0;
                for (int64_t j = 0; j < nk; ++j) {
                    p[j] /= l;
                    const double *v = V + (j * B + b) * dp;
                    double gj = 0.0;
                    for (int64_t e = 0; e < dp; ++e)
                        gj += da[e] * v[e];
                    g[j] = gj;
                    D += p[j] * gj;
                }
                double *dq = dQ + (t * B + b) * dp;
                for (int64_t e = 0; e < dp; ++e)
                    dq[e] = 0.0;
                for (int64_t j = 0; j < nk; ++j) {
                    const double ds = p[j] * (g[j] - D) * scale;
                    const double *k = K + (j * B + b) * dp;
                    double *dk = dK + (j * B + b) * dp;
                    double *dv = dV + (j * B + b) * dp;
                    for (int64_t e = 0; e < dp; ++e) {
                        dq[e] += ds * k[e];
                        dk[e] += ds * q[e];
                        dv[e] += p[j] * da[e];
                    }
                }
            }
        }
        free(p);
        free(g);
    }
}

/*
 * Gradient of sru_oracle_layernorm given dy: with xh = (x - mean) / sqrt(var
 * + eps) per row and dxh = dy * gamma,
 *   dx = (dxh - mean(dxh) - xh * mean(dxh * xh)) / sqrt(var + eps),
 *   dgamma = sum over rows of dy * xh,  dbeta = sum over rows of dy.
 * Rows in order (the parameter gradients are plain sums).
 */
void sru_oracle_layernorm_backward(int64_t n, int64_t w, const double *x, const double *gamma,
                                   double eps, const double *dy, double *dx, double *dgamma,
                                   double *dbeta)
{
    double *xh = (double *)malloc(sizeof(double) * (size_t)w);
    for (int64_t e = 0; e < w; ++e) {
        dgamma[e] = 0.0;
        dbeta[e] = 0.0;
    }
    for (int64_t i = 0; i < n; ++i) {
        const double *r = x + i * w;
        const double *g = dy + i * w;
        double mean = 0.0;
        for (int64_t e = 0; e < w; ++e)
            mean += r[e];
        mean /= (double)w;
        double var = 0.0;
        for (int64_t e = 0; e < w; ++e)
            var += (r[e] - mean) * (r[e] - mean);
        var /= (double)w;
        const double inv = 1.0 / sqrt(var + eps);
        double m1 = 0.0, m2 = 0.0;
        for (int64_t e = 0; e < w; ++e) {
            xh[e] = (r[e] - mean) * inv;
            const double dxh = g[e] * gamma[e];
            m1 += dxh;
            m2 += dxh * xh[e];
            dgamma[e] += g[e] * xh[e];
            dbeta[e] += g[e];
        }
        m1 /= (double)w;
        m2 /= (double)w;
        for (int64_t e = 0; e < w; ++e)
            dx[i * w + e] = (g[e] * gamma[e] - m1 - xh[e] * m2) * inv;
    }
    free(xh);
}

/*
 * Projection (Eq. 1) for a cross product of selected rows and columns:
 *   out[i][k] = sum_{q<K} Atilde[rows[i]][q] * W[cols[k]][q]
 * A is [M, K] row-major, W is [N, K] row-major (row n = output feature n).
 * Atilde = bf16-rounded A when round_a != 0, else A.  Sum in double, q in
 * increasing order.  Rows are independent and are spread over threads.
 */
void sru_oracle_project(int64_t M, int64_t N, int64_t K,
                        const float *A, int round_a, const float *W,
                        const int64_t *rows, int64_t n_rows,
                        const int64_t *cols, int64_t n_cols,
                        double *out)
{
    (void)M; (void)N;
#pragma omp parallel
    {
        double *arow = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n_rows; ++i) {
            const float *a = A + rows[i] * K;
            for (int64_t q = 0; q < K; ++q)
                arow[q] = round_a ? (double)sru_oracle_round_bf16(a[q]) : (double)a[q];
            for (int64_t k = 0; k < n_cols; ++k) {
                const float *w = W + cols[k] * K;
                double s = 0.0;
                for (int64_t q = 0; q < K; ++q)
                    s += arow[q] * (double)w[q];
                out[i * n_cols + k] = s;
            }
        }
        free(arow);
    }
}

/*
 * Backward-data projection: out[i][q] = sum_n G[rows[i]][n] * W[n][q] for all
 * q < K.  G is [M, N] row-major (the gradient of U), W is [N, K].  This is the
 * transpose of Eq. 1's map applied to the gradient (chain rule).
 */
void sru_oracle_project_bwd_data(int64_t M, int64_t N, int64_t K,
                                 const double *G, const float *W,
                                 const int64_t *rows, int64_t n_rows,
                                 double *out)
{
    (void)M;
    /* for every q the terms are added in increasing n */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_rows; ++i) {
        const double *g = G + rows[i] * N;
        double *o = out + i * K;
        for (int64_t q = 0; q < K; ++q)
            o[q] = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const float *w = W + n * K;
            for (int64_t q = 0; q < K; ++q)
                o[q] += g[n] * (double)w[q];
        }
    }
}

/*
 * Weight-gradient projection: out[n][q] = sum_m G[m][n] * Xt[m][q], with
 * Xt = bf16(X) when round_x (the operand the forward projection multiplies)
 * and X otherwise.  G is [M, N] row-major (the gradient of U), X is [M, K],
 * out is [N, K] (the layout of W).  This is the derivative of Eq. 1's
 * product with respect to its weights (chain rule); the terms of every
 * output are added in increasing m.
 */
void sru_oracle_project_bwd_weight(int64_t M, int64_t N, int64_t K,
                                   const double *G, const float *X, int round_x,
                                   double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double *o = out + n * K;
        for (int64_t q = 0; q < K; ++q)
            o[q] = 0.0;
        for (int64_t m = 0; m < M; ++m) {
            const double g = G[m * N + n];
            const float *x = X + m * K;
            for (int64_t q = 0; q < K; ++q) {
                const double xv = round_x ? (double)sru_oracle_round_bf16(x[q]) : (double)x[q];
                o[q] += g * xv;
            }
        }
    }
}

/*
 * One chain, forward.  All per-step arrays are indexed by the natural time
 * index t = 0..L-1.  dir = 0 walks t = 0..L-1, dir = 1 walks t = L-1..0.
 *   uf, ur, ux : the three slots of U for this channel (Eqs. 2, 3, 4)
 *   x          : the layer input for this channel (highway term, Eq. 5)
 * linear = 1: the linear mode (the gates do not see the state; vf, vr are
 * then ignored).
 * Outputs h[t], c[t] (the state after step t) and the final state.
 */
void sru_oracle_chain_forward(int64_t L, int dir, int linear, double alpha,
                              const double *uf, const double *ur,
                              const double *ux, const double *x,
                              double vf, double vr, double bf, double br,
                              double c0, double *h, double *c, double *c_last)
{
    double state = c0;
    for (int64_t s = 0; s < L; ++s) {
        int64_t t = dir ? (L - 1 - s) : s;
        double prev = state;
        double seen = linear ? 0.0 : prev;    /* the state the gates see */
        double f = oracle_sigmoid(uf[t] + vf * seen + bf);          /* Eq. 2 */
        double r = oracle_sigmoid(ur[t] + vr * seen + br);          /* Eq. 3 */
        state = f * prev + (1.0 - f) * ux[t];                       /* Eq. 4 */
        h[t] = r * state + (1.0 - r) * alpha * x[t];                /* Eq. 5 */
        c[t] = state;
    }
    *c_last = state;
}

/*
 * One chain, backward (chain rule through the forward above, in reverse
 * order of the direction's walk).  c[] is the forward state sequence, dh[]
 * the gradient of h, dc_last the gradient of the final state.  Outputs the
 * gradients of uf, ur, ux, of x through the highway term only, the chain's
 * contributions to dv, dv', db, db' and the gradient of c0.  linear as for
 * the forward: the state adjoint then has no terms through the gates.
 */
void sru_oracle_chain_backward(int64_t L, int dir, int linear, double alpha,
                               const double *uf, const double *ur,
                               const double *ux, const double *x,
                               double vf, double vr, double bf, double br,
                               double c0, const double *c, const double *dh,
                               double dc_last,
                               double *duf, double *dur, double *dux,
                               double *dx_hw, double *dvf, double *dvr,
                               double *dbf, double *dbr, double *dc0)
{
    double gc = dc_last;          /* dLoss/dc[t] arriving from later steps */
    double svf = 0.0, svr = 0.0, sbf = 0.0, sbr = 0.0;
    for (int64_t s = L - 1; s >= 0; --s) {
        int64_t t = dir ? (L - 1 - s) : s;
        double prev;
        if (s == 0)
            prev = c0;
        else
            prev = c[dir ? (t + 1) : (t - 1)];
        double seen = linear ? 0.0 : prev;
        double f = oracle_sigmoid(uf[t] + vf * seen + bf);
        double r = oracle_sigmoid(ur[t] + vr * seen + br);
        double ct = c[t];
        /* h = r*c + (1-r)*alpha*x */
        double dc = gc + dh[t] * r;
        double dr = dh[t] * (ct - alpha * x[t]);
        dx_hw[t] = dh[t] * (1.0 - r) * alpha;
        /* c = f*prev + (1-f)*ux */
        double df = dc * (prev - ux[t]);
        dux[t] = dc * (1.0 - f);
        /* through the sigmoids */
        double dzf = df * f * (1.0 - f);
        double dzr = dr * r * (1.0 - r);
        duf[t] = dzf;
        dur[t] = dzr;
        svf += dzf * prev;
        svr += dzr * prev;
        sbf += dzf;
        sbr += dzr;
        /* prev reaches the loss through c (via f*prev), f and r */
        gc = linear ? dc * f : dc * f + dzf * vf + dzr * vr;
    }
    *dvf = svf; *dvr = svr; *dbf = sbf; *dbr = sbr;
    *dc0 = gc;
}

/* ---------------------------------------------------------------------------
 * Whole-tensor routines.  Layouts (row-major, innermost last):
 *   U      [L, B, ndir, 3, d]   slot 0 = f, 1 = r, 2 = candidate (double:
 *                               given fp32/bf16 values widened, or the
 *                               oracle's own projection)
 *   x      [L, B, d]            shared by both directions
 *   v, b   [ndir, 2, d]         row 0 = f gate, row 1 = r gate; v NULL is
 *                               the linear mode (gates without the state)
 *   c0     [ndir, B, d]         NULL means zeros
 *   h, c   [L, B, ndir, d]
 *   c_last [ndir, B, d]
 *   dU     like U; dx_hw like x (sum over directions); dv, db like v;
 *   dc0    like c0
 * Chains are independent; OpenMP only spreads whole chains over threads and
 * the reductions over the batch are done afterwards in a fixed order.
 * ------------------------------------------------------------------------- */

static void gather_chain(int64_t L, int64_t B, int64_t d, int ndir,
                         int64_t dl, int64_t b, int64_t j,
                         const double *U, const float *x,
                         double *uf, double *ur, double *ux, double *xx)
{
    for (int64_t t = 0; t < L; ++t) {
        int64_t base = ((t * B + b) * ndir + dl) * 3 * d;
        uf[t] = U[base + 0 * d + j];
        ur[t] = U[base + 1 * d + j];
        ux[t] = U[base + 2 * d + j];
        xx[t] = x[(t * B + b) * d + j];
    }
}

void sru_oracle_forward(int64_t L, int64_t B, int64_t d, int ndir, double alpha,
                        const double *U, const float *x, const float *v,
                        const float *bias, const float *c0,
                        double *h, double *c, double *c_last)
{
    int64_t chains = (int64_t)ndir * B * d;
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * 6 * (size_t)L);
        double *uf = buf, *ur = buf + L, *ux = buf + 2 * L, *xx = buf + 3 * L;
        double *hh = buf + 4 * L, *cc = buf + 5 * L;
#pragma omp for schedule(static)
        for (int64_t ch = 0; ch < chains; ++ch) {
            int64_t dl = ch / (B * d), b = (ch / d) % B, j = ch % d;
            gather_chain(L, B, d, ndir, dl, b, j, U, x, uf, ur, ux, xx);
            double cl;
            sru_oracle_chain_forward(L, (int)dl, v == NULL, alpha, uf, ur, ux, xx,
                                     v ? v[(dl * 2 + 0) * d + j] : 0.0f,
                                     v ? v[(dl * 2 + 1) * d + j] : 0.0f,
                                     bias[(dl * 2 + 0) * d + j], bias[(dl * 2 + 1) * d + j],
                                     c0 ? (double)c0[(dl * B + b) * d + j] : 0.0,
                                     hh, cc, &cl);
            for (int64_t t = 0; t < L; ++t) {
                int64_t o = ((t * B + b) * ndir + dl) * d + j;
                h[o] = hh[t];
                c[o] = cc[t];
            }
            c_last[(dl * B + b) * d + j] = cl;
        }
        free(buf);
    }
}

/*
 * c is the oracle's own forward state sequence [L, B, ndir, d] (double).
 * dc_last may be NULL (zeros).  dv_part / db_part receive per-(dir, b)
 * partials [ndir, B, 2, d] that are then summed over b in increasing b.
 */
void sru_oracle_backward(int64_t L, int64_t B, int64_t d, int ndir, double alpha,
                         const double *U, const float *x, const float *v,
                         const float *bias, const float *c0, const double *c,
                         const float *dh, const float *dc_last,
                         double *dU, double *dx_hw, double *dv, double *db,
                         double *dc0)
{
    int64_t chains = (int64_t)ndir * B * d;
    double *dv_part = (double *)calloc((size_t)chains * 2, sizeof(double));
    double *db_part = (double *)calloc((size_t)chains * 2, sizeof(double));
    double *dxd = (double *)calloc((size_t)chains * (size_t)L, sizeof(double));
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * 11 * (size_t)L);
        double *uf = buf, *ur = buf + L, *ux = buf + 2 * L, *xx = buf + 3 * L;
        double *cc = buf + 4 * L, *gh = buf + 5 * L;
        double *duf = buf + 6 * L, *dur = buf + 7 * L, *dux = buf + 8 * L;
        double *dxx = buf + 9 * L;
#pragma omp for schedule(static)
        for (int64_t ch = 0; ch < chains; ++ch) {
            int64_t dl = ch / (B * d), b = (ch / d) % B, j = ch % d;
            gather_chain(L, B, d, ndir, dl, b, j, U, x, uf, ur, ux, xx);
            for (int64_t t = 0; t < L; ++t) {
                int64_t o = ((t * B + b) * ndir + dl) * d + j;
                cc[t] = c[o];
                gh[t] = dh[o];
            }
            double dvf, dvr, dbf, dbr, g0;
            sru_oracle_chain_backward(L, (int)dl, v == NULL, alpha, uf, ur, ux, xx,
                                      v ? v[(dl * 2 + 0) * d + j] : 0.0f,
                                      v ? v[(dl * 2 + 1) * d + j] : 0.0f,
                                      bias[(dl * 2 + 0) * d + j], bias[(dl * 2 + 1) * d + j],
                                      c0 ? (double)c0[(dl * B + b) * d + j] : 0.0,
                                      cc, gh,
                                      dc_last ? (double)dc_last[(dl * B + b) * d + j] : 0.0,
                                      duf, dur, dux, dxx, &dvf, &dvr, &dbf, &dbr, &g0);
            for (int64_t t = 0; t < L; ++t) {
                int64_t base = ((t * B + b) * ndir + dl) * 3 * d;
                dU[base + 0 * d + j] = duf[t];
                dU[base + 1 * d + j] = dur[t];
                dU[base + 2 * d + j] = dux[t];
                dxd[ch * L + t] = dxx[t];
            }
            dv_part[ch * 2 + 0] = dvf; dv_part[ch * 2 + 1] = dvr;
            db_part[ch * 2 + 0] = dbf; db_part[ch * 2 + 1] = dbr;
            dc0[(dl * B + b) * d + j] = g0;
        }
        free(buf);
    }
    /* highway gradient of x: sum over directions, direction 0 first */
    for (int64_t t = 0; t < L; ++t)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t j = 0; j < d; ++j) {
                double s = 0.0;
                for (int64_t dl = 0; dl < ndir; ++dl)
                    s += dxd[((dl * B + b) * d + j) * L + t];
                dx_hw[(t * B + b) * d + j] = s;
            }
    /* parameter gradients: sum over the batch, b increasing */
    for (int64_t dl = 0; dl < ndir; ++dl)
        for (int g = 0; g < 2; ++g)
            for (int64_t j = 0; j < d; ++j) {
                double sv = 0.0, sb = 0.0;
                for (int64_t b = 0; b < B; ++b) {
                    int64_t ch = (dl * B + b) * d + j;
                    sv += dv_part[ch * 2 + g];
                    sb += db_part[ch * 2 + g];
                }
                dv[(dl * 2 + g) * d + j] = sv;
                db[(dl * 2 + g) * d + j] = sb;
            }
    free(dv_part);
    free(db_part);
    free(dxd);
}

/* Sets the number of threads the routines above use from now on (n >= 1);
   the baseline timing runs them single-threaded and on every core. */
void sru_oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n < 1 ? 1 : n);
#else
    (void)n;
#endif
}

/* Number of threads the OpenMP runtime would use for the routines above. */
int sru_oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp master
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
