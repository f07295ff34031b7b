// linear_scan.hip -- the SRU recurrence with v = v' = 0 evaluated as a
// time-chunked parallel scan.
//
// With no c[t-1] term inside the gates ("Parallelizing Legendre Memory Unit
// Training", abstract: a network whose recurrent part is linear can be
// trained in parallel), Eq. 4 of the SRU++ paper becomes the first-order
// linear recurrence
//     c[t] = a[t] c[t-1] + (1 - a[t]) U[t,2],     a[t] = sigma(U[t,0] + b),
// i.e. a scan of the affine maps c -> a c + beta, whose composition is
//     (a1, beta1) then (a2, beta2)  =  (a2 a1, a2 beta1 + beta2).
// The sequence of each chain is cut into chunks of `chunk` steps:
//   1. aggregate: each (chain, chunk) folds its maps into (A, E) = the map of
//      the whole chunk (E is the chunk's state when started from 0);
//   2. carry: each chain folds the chunk maps in order, giving every chunk
//      its incoming state;
//   3. apply: each (chain, chunk) replays its steps from the incoming state
//      and writes h and c.
// The backward pass is the same construction in reverse time on the adjoint
//     gc[t-1] = a[t] (gc[t] + r[t] dh[t]),
// followed by the purely local gradients of each step.
//
// Phases 1 and 3 run one lane per (chain, chunk); at B*d = 16384 chains and
// 64 chunks that is a million independent lanes, which keeps every CU busy
// even though each chain alone is sequential.
#include "device_common.h"
#include "internal.h"

namespace sru {
namespace {

struct LinGeom {
    int64_t L, B, d, chunk, nC, chains;  // chains of one direction = B*d
    int ndir, dl;
};

__device__ __forceinline__ int64_t lin_t(const LinGeom &g, int64_t s)
{
    return g.dl ? (g.L - 1 - s) : s;
}

// ---------------------------------------------------------------- forward ---
template <typename TU>
__global__ __launch_bounds__(256) void lin_fwd_aggregate(LinGeom g, const TU *__restrict__ U,
                                                          const float *__restrict__ bias,
                                                          float *A, float *E)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.chains * g.nC) return;
    const int64_t ch = i % g.chains, k = i / g.chains;
    const int64_t j = ch % g.d, bb = ch / g.d;
    const float bf = bias[(g.dl * 2 + 0) * g.d + j];
    const int64_t s0 = k * g.chunk;
    const int64_t s1 = s0 + g.chunk < g.L ? s0 + g.chunk : g.L;
    float pa = 1.0f, e = 0.0f;
    for (int64_t s = s0; s < s1; ++s) {
        const int64_t ub = ((lin_t(g, s) * g.B + bb) * g.ndir + g.dl) * 3 * g.d + j;
        const Gate a = gate(load_as_f32(U + ub) + bf);
        const float ux = load_as_f32(U + ub + 2 * g.d);
        e = fmaf(a.g, e, a.gc * ux);
        pa *= a.g;
    }
    A[k * g.chains + ch] = pa;
    E[k * g.chains + ch] = e;
}

__global__ __launch_bounds__(256) void lin_fwd_carry(LinGeom g, const float *__restrict__ A,
                                                     const float *__restrict__ E,
                                                     const float *__restrict__ c0, float *cin)
{
    const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (ch >= g.chains) return;
    float c = c0 ? c0[g.dl * g.chains + ch] : 0.0f;
    for (int64_t k = 0; k < g.nC; ++k) {
        cin[k * g.chains + ch] = c;
        c = fmaf(A[k * g.chains + ch], c, E[k * g.chains + ch]);
    }
}

template <typename TU, typename TX>
__global__ __launch_bounds__(256) void lin_fwd_apply(LinGeom g, const TU *__restrict__ U,
                                                      const TX *__restrict__ X,
                                                      const float *__restrict__ bias,
                                                      float alpha, const float *__restrict__ cin,
                                                      float *h, float *c_seq, float *c_last)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.chains * g.nC) return;
    const int64_t ch = i % g.chains, k = i / g.chains;
    const int64_t j = ch % g.d, bb = ch / g.d;
    const float bf = bias[(g.dl * 2 + 0) * g.d + j], br = bias[(g.dl * 2 + 1) * g.d + j];
    const int64_t s0 = k * g.chunk;
    const int64_t s1 = s0 + g.chunk < g.L ? s0 + g.chunk : g.L;
    float c = cin[k * g.chains + ch];
    for (int64_t s = s0; s < s1; ++s) {
        const int64_t t = lin_t(g, s);
        const int64_t ub = ((t * g.B + bb) * g.ndir + g.dl) * 3 * g.d + j;
        const Gate a = gate(load_as_f32(U + ub) + bf);
        const Gate r = gate(load_as_f32(U + ub + g.d) + br);
        const float ux = load_as_f32(U + ub + 2 * g.d);
        const float ax = alpha * load_as_f32(X + (t * g.B + bb) * g.d + j);
        c = fmaf(a.g, c, a.gc * ux);
        const int64_t o = ((t * g.B + bb) * g.ndir + g.dl) * g.d + j;
        h[o] = fmaf(r.g, c, r.gc * ax);
        if (c_seq) c_seq[o] = c;
    }
    if (c_last && k == g.nC - 1) c_last[g.dl * g.chains + ch] = c;
}

// --------------------------------------------------------------- backward ---
template <typename TU>
__global__ __launch_bounds__(256) void lin_bwd_aggregate(LinGeom g, const TU *__restrict__ U,
                                                          const float *__restrict__ bias,
                                                          const float *__restrict__ dh,
                                                          float *A, float *G)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.chains * g.nC) return;
    const int64_t ch = i % g.chains, k = i / g.chains;
    const int64_t j = ch % g.d, bb = ch / g.d;
    const float bf = bias[(g.dl * 2 + 0) * g.d + j], br = bias[(g.dl * 2 + 1) * g.d + j];
    const int64_t s0 = k * g.chunk;
    const int64_t s1 = s0 + g.chunk < g.L ? s0 + g.chunk : g.L;
    float pa = 1.0f, gc = 0.0f;
    for (int64_t s = s1 - 1; s >= s0; --s) {
        const int64_t t = lin_t(g, s);
        const int64_t ub = ((t * g.B + bb) * g.ndir + g.dl) * 3 * g.d + j;
        const Gate a = gate(load_as_f32(U + ub) + bf);
        const Gate r = gate(load_as_f32(U + ub + g.d) + br);
        const float dhv = dh[((t * g.B + bb) * g.ndir + g.dl) * g.d + j];
        gc = a.g * fmaf(r.g, dhv, gc);
        pa *= a.g;
    }
    A[k * g.chains + ch] = pa;
    G[k * g.chains + ch] = gc;
}

__global__ __launch_bounds__(256) void lin_bwd_carry(LinGeom g, const float *__restrict__ A,
                                                     const float *__restrict__ G,
                                                     const float *__restrict__ dc_last,
                                                     float *gin)
{
    const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (ch >= g.chains) return;
    float gc = dc_last ? dc_last[g.dl * g.chains + ch] : 0.0f;
    for (int64_t k = g.nC - 1; k >= 0; --k) {
        gin[k * g.chains + ch] = gc;
        gc = fmaf(A[k * g.chains + ch], gc, G[k * g.chains + ch]);
    }
}

template <typename TU, typename TX>
__global__ __launch_bounds__(256) void lin_bwd_apply(LinGeom g, const TU *__restrict__ U,
                                                      const TX *__restrict__ X,
                                                      const float *__restrict__ bias,
                                                      float alpha, const float *__restrict__ c0,
                                                      const float *__restrict__ c_seq,
                                                      const float *__restrict__ dh,
                                                      const float *__restrict__ gin,
                                                      float *dU, float *dx, bool dx_acc,
                                                      float *dc0, float *dbpart)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.chains * g.nC) return;
    const int64_t ch = i % g.chains, k = i / g.chains;
    const int64_t j = ch % g.d, bb = ch / g.d;
    const float bf = bias[(g.dl * 2 + 0) * g.d + j], br = bias[(g.dl * 2 + 1) * g.d + j];
    const int64_t s0 = k * g.chunk;
    const int64_t s1 = s0 + g.chunk < g.L ? s0 + g.chunk : g.L;
    auto oidx = [&](int64_t t) { return ((t * g.B + bb) * g.ndir + g.dl) * g.d + j; };
    const float c0v = c0 ? c0[g.dl * g.chains + ch] : 0.0f;
    float gc = gin[k * g.chains + ch];
    float c = c_seq[oidx(lin_t(g, s1 - 1))];
    float sbf = 0.0f, sbr = 0.0f;
    for (int64_t s = s1 - 1; s >= s0; --s) {
        const int64_t t = lin_t(g, s);
        const float cp = s > 0 ? c_seq[oidx(lin_t(g, s - 1))] : c0v;
        const int64_t ub = ((t * g.B + bb) * g.ndir + g.dl) * 3 * g.d + j;
        const Gate a = gate(load_as_f32(U + ub) + bf);
        const Gate r = gate(load_as_f32(U + ub + g.d) + br);
        const float ux = load_as_f32(U + ub + 2 * g.d);
        const int64_t xi = (t * g.B + bb) * g.d + j;
        const float xv = load_as_f32(X + xi);
        const float dhv = dh[oidx(t)];
        const float D = fmaf(r.g, dhv, gc);
        const float dr = dhv * fmaf(-alpha, xv, c);
        float dxh = dhv * r.gc * alpha;
        if (dx_acc) dxh += dx[xi];
        const float dzf = D * (cp - ux) * (a.g * a.gc);
        const float dzr = dr * (r.g * r.gc);
        dU[ub] = dzf;
        dU[ub + g.d] = dzr;
        dU[ub + 2 * g.d] = D * a.gc;
        dx[xi] = dxh;
        sbf += dzf;
        sbr += dzr;
        gc = a.g * D;
        c = cp;
    }
    if (dc0 && k == 0) dc0[g.dl * g.chains + ch] = gc;
    dbpart[(k * 2 + 0) * g.chains + ch] = sbf;
    dbpart[(k * 2 + 1) * g.chains + ch] = sbr;
}

// db[dl, g, j] = sum over (b, chunk) of the per-(chain, chunk) partials.  A
// block of 256 threads owns 64 consecutive j of one gate: wave w sums the
// (b, chunk) pairs of index w mod 4 (pair index = b * nC + chunk), with loads
// in flight, and the four wave sums are added in wave order; the order depends
// only on the shape, so results are identical run to run.
__global__ __launch_bounds__(256) void lin_db_reduce(LinGeom g, const float *__restrict__ part,
                                                     float *db)
{
    __shared__ float red[4][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t jblocks = (g.d + 63) / 64;
    const int gg = (int)(blockIdx.x / jblocks);
    const int64_t j = (blockIdx.x % jblocks) * 64 + lane;
    const int64_t pairs = g.B * g.nC;
    float s = 0.0f;
    if (j < g.d) {
        auto at = [&](int64_t q) {
            const int64_t bb = q / g.nC, k = q % g.nC;
            return part[(k * 2 + gg) * g.chains + bb * g.d + j];
        };
        int64_t q = wv;
        for (; q + 12 < pairs; q += 16) {
            const float a0 = at(q), a1 = at(q + 4), a2 = at(q + 8), a3 = at(q + 12);
            s += a0;
            s += a1;
            s += a2;
            s += a3;
        }
        for (; q < pairs; q += 4) s += at(q);
    }
    red[wv][lane] = s;
    __syncthreads();
    if (wv == 0 && j < g.d)
        db[(g.dl * 2 + gg) * g.d + j] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

template <typename TU, typename TX>
hipError_t lin_forward_t(const LinArgs &a, hipStream_t s)
{
    const int64_t nC = (a.L + a.chunk - 1) / a.chunk;
    const int64_t chains = a.B * a.d;
    float *ws = (float *)a.ws;
    float *A = ws, *E = ws + nC * chains, *cin = ws + 2 * nC * chains;
    for (int dl = 0; dl < a.ndir; ++dl) {
        LinGeom g{a.L, a.B, a.d, a.chunk, nC, chains, a.ndir, dl};
        hipLaunchKernelGGL(lin_fwd_aggregate<TU>, dim3(blocks_for(chains * nC)), dim3(256), 0, s,
                           g, (const TU *)a.U, a.b, A, E);
        hipLaunchKernelGGL(lin_fwd_carry, dim3(blocks_for(chains)), dim3(256), 0, s, g, A, E,
                           a.c0, cin);
        hipLaunchKernelGGL((lin_fwd_apply<TU, TX>), dim3(blocks_for(chains * nC)), dim3(256), 0,
                           s, g, (const TU *)a.U, (const TX *)a.x, a.b, a.alpha, cin, a.h,
                           a.c_seq, a.c_last);
    }
    return hipGetLastError();
}

template <typename TU, typename TX>
hipError_t lin_backward_t(const LinArgs &a, hipStream_t s)
{
    const int64_t nC = (a.L + a.chunk - 1) / a.chunk;
    const int64_t chains = a.B * a.d;
    float *ws = (float *)a.ws;
    float *A = ws, *G = ws + nC * chains, *gin = ws + 2 * nC * chains;
    float *dbp = ws + 3 * nC * chains;  // [nC, 2, chains]
    for (int dl = a.ndir - 1; dl >= 0; --dl) {
        LinGeom g{a.L, a.B, a.d, a.chunk, nC, chains, a.ndir, dl};
        hipLaunchKernelGGL(lin_bwd_aggregate<TU>, dim3(blocks_for(chains * nC)), dim3(256), 0, s,
                           g, (const TU *)a.U, a.b, a.dh, A, G);
        hipLaunchKernelGGL(lin_bwd_carry, dim3(blocks_for(chains)), dim3(256), 0, s, g, A, G,
                           a.dc_last, gin);
        hipLaunchKernelGGL((lin_bwd_apply<TU, TX>), dim3(blocks_for(chains * nC)), dim3(256), 0,
                           s, g, (const TU *)a.U, (const TX *)a.x, a.b, a.alpha, a.c0, a.c_seq,
                           a.dh, gin, a.dU, a.dx, dl != a.ndir - 1, a.dc0, dbp);
        if (a.db)
            hipLaunchKernelGGL(lin_db_reduce, dim3((unsigned)(2 * ((a.d + 63) / 64))), dim3(256), 0,
                               s, g, dbp, a.db);
    }
    return hipGetLastError();
}

}  // namespace

size_t linear_workspace_bytes(int64_t L, int64_t B, int64_t d, int ndir, int64_t chunk,
                              bool backward)
{
    (void)ndir;  // directions are processed one after another and reuse it
    const int64_t nC = (L + chunk - 1) / chunk;
    const int64_t per = nC * B * d;
    const int64_t floats = backward ? 5 * per : 3 * per;
    return (size_t)floats * sizeof(float);
}

hipError_t launch_linear_forward(const LinArgs &a, hipStream_t s)
{
    if (a.u_bf16)
        return a.x_bf16 ? lin_forward_t<bf16_bits, bf16_bits>(a, s)
                        : lin_forward_t<bf16_bits, float>(a, s);
    return a.x_bf16 ? lin_forward_t<float, bf16_bits>(a, s) : lin_forward_t<float, float>(a, s);
}

hipError_t launch_linear_backward(const LinArgs &a, hipStream_t s)
{
    if (a.u_bf16)
        return a.x_bf16 ? lin_backward_t<bf16_bits, bf16_bits>(a, s)
                        : lin_backward_t<bf16_bits, float>(a, s);
    return a.x_bf16 ? lin_backward_t<float, bf16_bits>(a, s) : lin_backward_t<float, float>(a, s);
}

}  // namespace sru
