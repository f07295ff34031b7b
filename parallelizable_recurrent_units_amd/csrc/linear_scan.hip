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
#include "scan_common.h"

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
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
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

// ---------------------------------------------------------------------------
// Single-pass chunked scan (chunk = W * SEG steps, d % 64 == 0).
//
// A workgroup of W waves owns 64 consecutive chains and one chunk; wave w
// holds steps [w*SEG, (w+1)*SEG) of the chunk, so every input element is
// read from HBM once:
//   1. each lane folds its SEG steps into the segment map (A, E);
//   2. wave 0 folds the W segment maps into the chunk map, obtains the
//      chunk's incoming state from the previous chunk of the same chains,
//      publishes its own outgoing state, and hands every segment its
//      incoming state via LDS;
//   3. each lane replays its steps from that state and writes h and c.
// Chunks exchange states through the look-back of scan_common.h; tickets
// are handed out chain-major (ticket = chunk * tiles + tile).
// ---------------------------------------------------------------------------
template <typename TU, typename TX, int W, int SEG, int PB, int WPE>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(WPE))) void lin_fwd_fused(
    LinGeom g, const TU *__restrict__ U, const TX *__restrict__ X, const float *__restrict__ bias,
    float alpha, const float *__restrict__ c0, float *h, float *c_seq, float *c_last, Lookback lb)
{
    static_assert(SEG % PB == 0, "phase-3 batches must tile the segment");
    __shared__ float sA[W][64], sE[W][64], sC[W][64];
    __shared__ uint32_t s_ticket;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int64_t tiles = g.chains / 64;
    const int64_t tk = take_ticket(lb, &s_ticket);
    const int64_t k = tk / tiles, tile = tk % tiles;
    // a tile is 64 consecutive channels of one batch row (d % 64 == 0)
    const int64_t ch0 = tile * 64, ch = ch0 + lane;
    const int64_t j0 = ch0 % g.d, bb = ch0 / g.d, j = j0 + lane;
    const float bfs = bias[(g.dl * 2 + 0) * g.d + j] * kNegLog2e;
    const float brs = bias[(g.dl * 2 + 1) * g.d + j] * kNegLog2e;
    const int64_t s_lo = k * g.chunk + wv * SEG;
    const SegRows sr(g.L, g.dl != 0, s_lo, SEG);
    // uniform bases at row t0; per-lane part: lane * element size
    const int64_t ustride = g.B * g.ndir * 3 * g.d, xstride = g.B * g.d;
    const int64_t ostride = g.B * g.ndir * g.d;
    const char *ubase = (const char *)(U + sr.t0 * ustride + (bb * g.ndir + g.dl) * 3 * g.d + j0);
    const char *xbase = (const char *)(X + sr.t0 * xstride + bb * g.d + j0);
    const uint32_t urow = (uint32_t)(ustride * sizeof(TU)), xrow = (uint32_t)(xstride * sizeof(TX));
    const uint32_t orow = (uint32_t)(ostride * sizeof(float));
    const uint32_t ulane = (uint32_t)lane * sizeof(TU), xlane = (uint32_t)lane * sizeof(TX);
    const uint32_t olane = (uint32_t)lane * sizeof(float);
    const uint32_t ud = (uint32_t)(g.d * sizeof(TU));   // stream-to-stream distance in a row

    // phase 1: load the forget-gate and candidate streams of the segment and
    // fold them into (A, E); the map (a, beta) of each step stays in registers
    float ga[SEG], gb[SEG];
    float A = 1.0f, E = 0.0f;
    if (sr.nv1 >= 0) {
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            const uint32_t o = sr.row(i) * urow + ulane;
            ga[i] = ld_off<TU>(ubase, o);
            gb[i] = ld_off<TU>(ubase, o + 2 * ud);
        }
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            if (i <= sr.nv1) {
                const Gate a = gate_scaled(fmaf(ga[i], kNegLog2e, bfs));
                ga[i] = a.g;
                gb[i] = a.gc * gb[i];          // beta = (1 - a) u_cand
                E = fmaf(a.g, E, gb[i]);
                A *= a.g;
            }
        }
    }
    sA[wv][lane] = A;
    sE[wv][lane] = E;
    __syncthreads();

    // phase 2 (wave 0): chunk map, carry in, carry out, segment carries
    if (wv == 0) {
        float Ac = 1.0f, Ec = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            Ec = fmaf(sA[w][lane], Ec, sE[w][lane]);
            Ac *= sA[w][lane];
        }
        float cin;
        if (k == 0)
            cin = c0 ? c0[g.dl * g.chains + ch] : 0.0f;
        else
            cin = consume(lb, (k - 1) * g.chains + ch, lane);
        if (k + 1 < g.nC) publish(lb, k * g.chains + ch, fmaf(Ac, cin, Ec));
        float cc = cin;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            sC[w][lane] = cc;
            cc = fmaf(sA[w][lane], cc, sE[w][lane]);
        }
    }
    __syncthreads();
    if (sr.nv1 < 0) return;   // the whole segment lies past the end

    // phase 3: replay the segment PB steps at a time; the reset-gate and x
    // streams are loaded only now, next to the stores of h and c
    float c = sC[wv][lane];
    char *hbase = (char *)(h + sr.t0 * ostride + (bb * g.ndir + g.dl) * g.d + j0);
    char *cbase = c_seq ? (char *)(c_seq + sr.t0 * ostride + (bb * g.ndir + g.dl) * g.d + j0)
                        : nullptr;
#pragma unroll
    for (int i0 = 0; i0 < SEG; i0 += PB) {
        float ur[PB], xv[PB];
#pragma unroll
        for (int i = 0; i < PB; ++i) {
            const uint32_t r = sr.row(i0 + i);
            ur[i] = ld_off<TU>(ubase, r * urow + ulane + ud);
            xv[i] = ld_off<TX>(xbase, r * xrow + xlane);
        }
#pragma unroll
        for (int i = 0; i < PB; ++i) {
            if (i0 + i <= sr.nv1) {
                c = fmaf(ga[i0 + i], c, gb[i0 + i]);
                const Gate rg = gate_scaled(fmaf(ur[i], kNegLog2e, brs));
                const uint32_t o = sr.row(i0 + i) * orow + olane;
                st_off(hbase, o, fmaf(rg.g, c, rg.gc * (alpha * xv[i])));
                if (cbase) st_off(cbase, o, c);
            }
        }
    }
    if (c_last && s_lo + sr.nv1 == g.L - 1) c_last[g.dl * g.chains + ch] = c;
}

// Backward: the adjoint of the state runs from the last step to the first,
//   gc[t-1] = a[t] (gc[t] + r[t] dh[t]),
// so chunks are chained from the last one down (ticket chunk = nC - 1 -
// ticket / tiles) and each segment's map is g -> A g + G over its steps in
// reverse.  Phase 3 recomputes the gates from the register-held U values and
// writes dU, dx and the per-chunk partial sums of dU_f, dU_r (for db).
template <typename TU, typename TX, int W, int SEG, int PB, int WPE>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(WPE))) void lin_bwd_fused(
    LinGeom g, const TU *__restrict__ U, const TX *__restrict__ X, const float *__restrict__ bias,
    float alpha, const float *__restrict__ c0, const float *__restrict__ c_seq,
    const float *__restrict__ dh, const float *__restrict__ dc_last, float *dU, float *dx,
    bool dx_acc, float *dc0, float *dbpart, Lookback lb)
{
    static_assert(SEG % PB == 0, "phase-3 batches must tile the segment");
    __shared__ float sA[W][64], sG[W][64], sC[W][64];
    __shared__ float sbf_w[W][64], sbr_w[W][64];
    __shared__ uint32_t s_ticket;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int64_t tiles = g.chains / 64;
    const int64_t tk = take_ticket(lb, &s_ticket);
    const int64_t k = g.nC - 1 - tk / tiles, tile = tk % tiles;
    const int64_t ch0 = tile * 64, ch = ch0 + lane;     // see the forward kernel
    const int64_t j0 = ch0 % g.d, bb = ch0 / g.d, j = j0 + lane;
    const float bfs = bias[(g.dl * 2 + 0) * g.d + j] * kNegLog2e;
    const float brs = bias[(g.dl * 2 + 1) * g.d + j] * kNegLog2e;
    const int64_t s_lo = k * g.chunk + wv * SEG;
    const SegRows sr(g.L, g.dl != 0, s_lo, SEG);
    const int64_t ustride = g.B * g.ndir * 3 * g.d, xstride = g.B * g.d;
    const int64_t hstride = g.B * g.ndir * g.d;
    const int64_t uoff = (bb * g.ndir + g.dl) * 3 * g.d + j0, xoff = bb * g.d + j0;
    const int64_t hoff = (bb * g.ndir + g.dl) * g.d + j0;
    const char *ubase = (const char *)(U + sr.t0 * ustride + uoff);       // uniform bases
    const char *xbase = (const char *)(X + sr.t0 * xstride + xoff);
    const char *dhbase = (const char *)(dh + sr.t0 * hstride + hoff);
    const char *csbase = (const char *)(c_seq + sr.t0 * hstride + hoff);
    const uint32_t urow = (uint32_t)(ustride * sizeof(TU)), xrow = (uint32_t)(xstride * sizeof(TX));
    const uint32_t hrow = (uint32_t)(hstride * sizeof(float));
    const uint32_t frow = (uint32_t)(ustride * sizeof(float)), fxrow = (uint32_t)(xstride * sizeof(float));
    const uint32_t ulane = (uint32_t)lane * sizeof(TU), xlane = (uint32_t)lane * sizeof(TX);
    const uint32_t flane = (uint32_t)lane * sizeof(float);
    const uint32_t ud = (uint32_t)(g.d * sizeof(TU)), fd = (uint32_t)(g.d * sizeof(float));

    // phase 1: gates and dh of the segment, folded in reverse into (A, G)
    float uf[SEG], ur[SEG], dv[SEG];
    float A = 1.0f, G = 0.0f;
    if (sr.nv1 >= 0) {
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            const uint32_t r = sr.row(i);
            uf[i] = ld_off<TU>(ubase, r * urow + ulane);
            ur[i] = ld_off<TU>(ubase, r * urow + ulane + ud);
            dv[i] = ldf_off(dhbase, r * hrow + flane);
        }
#pragma unroll
        for (int i = SEG - 1; i >= 0; --i) {
            if (i <= sr.nv1) {
                const Gate a = gate_scaled(fmaf(uf[i], kNegLog2e, bfs));
                const Gate r = gate_scaled(fmaf(ur[i], kNegLog2e, brs));
                G = a.g * fmaf(r.g, dv[i], G);
                A *= a.g;
            }
        }
    }
    sA[wv][lane] = A;
    sG[wv][lane] = G;
    __syncthreads();

    if (wv == 0) {
        float Ac = 1.0f, Gc = 0.0f;
#pragma unroll
        for (int w = W - 1; w >= 0; --w) {
            Gc = fmaf(sA[w][lane], Gc, sG[w][lane]);
            Ac *= sA[w][lane];
        }
        float gin;
        if (k == g.nC - 1)
            gin = dc_last ? dc_last[g.dl * g.chains + ch] : 0.0f;
        else
            gin = consume(lb, (k + 1) * g.chains + ch, lane);
        if (k > 0) publish(lb, k * g.chains + ch, fmaf(Ac, gin, Gc));
        float gg = gin;
#pragma unroll
        for (int w = W - 1; w >= 0; --w) {
            sC[w][lane] = gg;
            gg = fmaf(sA[w][lane], gg, sG[w][lane]);
        }
    }
    __syncthreads();

    // phase 3: local gradients, last step of the segment first, PB steps at
    // a time; the candidate, x and state streams are loaded only now.  Each
    // batch also needs the state one step before it: the previous batch's
    // last row, or for the first batch the state entering the segment.
    float gc = sC[wv][lane];
    float sbf = 0.0f, sbr = 0.0f;
    if (sr.nv1 >= 0) {
        float c_enter;   // state before the segment's first step
        if (s_lo == 0)
            c_enter = c0 ? c0[g.dl * g.chains + ch] : 0.0f;
        else
            c_enter = c_seq[lin_t(g, s_lo - 1) * hstride + hoff + lane];
        char *dubase = (char *)(dU + sr.t0 * ustride + uoff);
        char *dxbase = (char *)(dx + sr.t0 * xstride + xoff);
#pragma unroll
        for (int i0 = SEG - PB; i0 >= 0; i0 -= PB) {
            float ux[PB], xv[PB], cv[PB + 1];   // cv[i + 1] = c at step i0 + i
#pragma unroll
            for (int i = 0; i < PB; ++i) {
                const uint32_t r = sr.row(i0 + i);
                ux[i] = ld_off<TU>(ubase, r * urow + ulane + 2 * ud);
                xv[i] = ld_off<TX>(xbase, r * xrow + xlane);
                cv[i + 1] = ldf_off(csbase, r * hrow + flane);
            }
            cv[0] = i0 == 0 ? c_enter : ldf_off(csbase, sr.row(i0 - 1) * hrow + flane);
#pragma unroll
            for (int i = PB - 1; i >= 0; --i) {
                if (i0 + i <= sr.nv1) {
                    const Gate a = gate_scaled(fmaf(uf[i0 + i], kNegLog2e, bfs));
                    const Gate r = gate_scaled(fmaf(ur[i0 + i], kNegLog2e, brs));
                    const float dvi = dv[i0 + i];
                    const float D = fmaf(r.g, dvi, gc);
                    const float dr = dvi * fmaf(-alpha, xv[i], cv[i + 1]);
                    const uint32_t row = sr.row(i0 + i);
                    const uint32_t xo = row * fxrow + flane, uo = row * frow + flane;
                    float dxh = dvi * r.gc * alpha;
                    if (dx_acc) dxh += ldf_off(dxbase, xo);
                    const float dzf = D * (cv[i] - ux[i]) * (a.g * a.gc);
                    const float dzr = dr * (r.g * r.gc);
                    st_off(dubase, uo, dzf);
                    st_off(dubase, uo + fd, dzr);
                    st_off(dubase, uo + 2 * fd, D * a.gc);
                    st_off(dxbase, xo, dxh);
                    sbf += dzf;
                    sbr += dzr;
                    gc = a.g * D;
                }
            }
        }
    }
    if (k == 0 && wv == 0 && dc0) dc0[g.dl * g.chains + ch] = gc;
    // per-(chunk, chain) partial sums of dz_f and dz_r, waves added in order
    sbf_w[wv][lane] = sbf;
    sbr_w[wv][lane] = sbr;
    __syncthreads();
    if (wv == 0) {
        float f = 0.0f, r = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            f += sbf_w[w][lane];
            r += sbr_w[w][lane];
        }
        dbpart[(k * 2 + 0) * g.chains + ch] = f;
        dbpart[(k * 2 + 1) * g.chains + ch] = r;
    }
}


constexpr int kFusedChunk = 256;
#ifndef SRU_LIN_FWD_W
#define SRU_LIN_FWD_W 16
#endif
#ifndef SRU_LIN_FWD_PB
#define SRU_LIN_FWD_PB 16
#endif
#ifndef SRU_LIN_FWD_WPE
#define SRU_LIN_FWD_WPE 4
#endif
#ifndef SRU_LIN_BWD_WPE
#define SRU_LIN_BWD_WPE 4
#endif
#ifndef SRU_LIN_BWD_W
#define SRU_LIN_BWD_W 16
#endif
#ifndef SRU_LIN_BWD_PB
#define SRU_LIN_BWD_PB 16
#endif
constexpr int kFwdW = SRU_LIN_FWD_W, kFwdSeg = kFusedChunk / kFwdW, kFwdPB = SRU_LIN_FWD_PB,
              kFwdWpe = SRU_LIN_FWD_WPE;
constexpr int kBwdW = SRU_LIN_BWD_W, kBwdSeg = kFusedChunk / kBwdW, kBwdPB = SRU_LIN_BWD_PB,
              kBwdWpe = SRU_LIN_BWD_WPE;
static_assert(kFwdW * kFwdSeg == kFusedChunk && kBwdW * kBwdSeg == kFusedChunk, "chunk split");

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

// Workspace layout of the single-pass kernels (in floats):
//   control block [kCtrlWords] (error word, ticket) |
//   published states [nC * chains] 64-bit words (2 floats each) |
//   backward only: db partials [2 * nC * chains]
// The ticket and the states are cleared before each direction's launch, the
// error word once per call (before the first direction).
struct FusedWs {
    Lookback lb;
    float *dbpart;
    uint32_t *ctrl;        // the control block; the cleared region starts here
    int64_t clear_words;
};

FusedWs fused_ws(const LinArgs &a, bool backward)
{
    const int64_t nC = (a.L + a.chunk - 1) / a.chunk;
    const int64_t chains = a.B * a.d;
    float *ws = (float *)a.ws;
    FusedWs f;
    f.ctrl = (uint32_t *)ws;
    f.lb.err = f.ctrl + kErrWord;
    f.lb.ticket = f.ctrl + kTicketWord;
    f.lb.carry = (uint64_t *)(ws + kCtrlWords);
    f.dbpart = backward ? ws + kCtrlWords + 2 * nC * chains : nullptr;
    f.clear_words = kCtrlWords + 2 * nC * chains;
    return f;
}

// Clears the control block and states before direction number `k` of a
// call (k = 0 first): the error word only before the first.
void fused_clear(const FusedWs &f, int k, hipStream_t s)
{
    const int64_t from = k == 0 ? 0 : kTicketWord;
    hipLaunchKernelGGL(scan_clear, dim3(scan_clear_blocks(f.clear_words - from)), dim3(256), 0, s,
                       f.ctrl + from, f.clear_words - from);
}

bool use_fused(const LinArgs &a)
{
    const int64_t chains = a.B * a.d;
    const int64_t seg = kFwdSeg > kBwdSeg ? kFwdSeg : kBwdSeg;
    // the kernels address a segment with 32-bit byte offsets from one base
    const int64_t seg_bytes = (seg + 1) * a.B * a.ndir * 3 * a.d * (int64_t)sizeof(float);
    return a.chunk == kFusedChunk && a.d % 64 == 0 && seg_bytes < (int64_t(1) << 31) &&
           (chains / 64) * ((a.L + a.chunk - 1) / a.chunk) < (int64_t(1) << 31);
}

template <typename TU, typename TX>
hipError_t lin_forward_fused(const LinArgs &a, hipStream_t s)
{
    const int64_t nC = (a.L + a.chunk - 1) / a.chunk;
    const int64_t chains = a.B * a.d;
    const FusedWs f = fused_ws(a, false);
    for (int dl = 0; dl < a.ndir; ++dl) {
        LinGeom g{a.L, a.B, a.d, a.chunk, nC, chains, a.ndir, dl};
        fused_clear(f, dl, s);
        hipLaunchKernelGGL((lin_fwd_fused<TU, TX, kFwdW, kFwdSeg, kFwdPB, kFwdWpe>), dim3((unsigned)(nC * (chains / 64))),
                           dim3(kFwdW * 64), 0, s, g, (const TU *)a.U, (const TX *)a.x, a.b, a.alpha,
                           a.c0, a.h, a.c_seq, a.c_last, f.lb);
    }
    return hipGetLastError();
}

template <typename TU, typename TX>
hipError_t lin_backward_fused(const LinArgs &a, hipStream_t s)
{
    const int64_t nC = (a.L + a.chunk - 1) / a.chunk;
    const int64_t chains = a.B * a.d;
    const FusedWs f = fused_ws(a, true);
    for (int dl = a.ndir - 1; dl >= 0; --dl) {
        LinGeom g{a.L, a.B, a.d, a.chunk, nC, chains, a.ndir, dl};
        fused_clear(f, a.ndir - 1 - dl, s);
        hipLaunchKernelGGL((lin_bwd_fused<TU, TX, kBwdW, kBwdSeg, kBwdPB, kBwdWpe>), dim3((unsigned)(nC * (chains / 64))),
                           dim3(kBwdW * 64), 0, s, g, (const TU *)a.U, (const TX *)a.x, a.b, a.alpha,
                           a.c0, a.c_seq, a.dh, a.dc_last, a.dU, a.dx, dl != a.ndir - 1, a.dc0,
                           f.dbpart, f.lb);
        if (a.db)
            hipLaunchKernelGGL(lin_db_reduce, dim3((unsigned)(2 * ((a.d + 63) / 64))), dim3(256), 0,
                               s, g, f.dbpart, a.db);
    }
    return hipGetLastError();
}

template <typename TU, typename TX>
hipError_t lin_forward_t(const LinArgs &a, hipStream_t s)
{
    if (use_fused(a)) return lin_forward_fused<TU, TX>(a, s);
    const int64_t nC = (a.L + a.chunk - 1) / a.chunk;
    const int64_t chains = a.B * a.d;
    float *ws = (float *)a.ws + kCtrlWords;
    float *A = ws, *E = ws + nC * chains, *cin = ws + 2 * nC * chains;
    // no look-back on this path: the error word is only cleared
    hipLaunchKernelGGL(scan_clear, dim3(1), dim3(256), 0, s, (uint32_t *)a.ws + kErrWord,
                       (int64_t)1);
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
    if (use_fused(a)) return lin_backward_fused<TU, TX>(a, s);
    const int64_t nC = (a.L + a.chunk - 1) / a.chunk;
    const int64_t chains = a.B * a.d;
    float *ws = (float *)a.ws + kCtrlWords;
    float *A = ws, *G = ws + nC * chains, *gin = ws + 2 * nC * chains;
    float *dbp = ws + 3 * nC * chains;  // [nC, 2, chains]
    // no look-back on this path: the error word is only cleared
    hipLaunchKernelGGL(scan_clear, dim3(1), dim3(256), 0, s, (uint32_t *)a.ws + kErrWord,
                       (int64_t)1);
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
    // the control block, then three-phase: 3 (fwd) or 5 (bwd) per-chunk
    // arrays; single pass: 64-bit published states (+ db partials)
    const int64_t floats = kCtrlWords + (backward ? 5 * per : 3 * per);
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
