// backward_scan.hip -- the backward pass of the SRU recurrence (chain rule
// through Eqs. 2-5 of the SRU++ paper's background section, Lei, "When
// Attention Meets Fast Recurrence") evaluated as a time-chunked scan.
//
// Given the forward's stored states c, every quantity of a reverse step is
// local except the adjoint gc of the state, and that adjoint is linear:
//     f  = sigma(U_f + v_f c_prev + b_f),  r = sigma(U_r + v_r c_prev + b_r)
//     dc = gc + r dh
//     dz_r = dh (c - alpha x) r (1 - r)            (gc-free)
//     dx   = dh (1 - r) alpha                      (gc-free)
//     m    = (c_prev - U_cand) f (1 - f)
//     dz_f = dc m,   dU_cand = dc (1 - f)
//     gc_prev = kappa dc + dz_r v_r,   kappa = f + m v_f
// so gc_prev = kappa gc + (kappa r dh + dz_r v_r): a first-order linear
// recurrence in reverse time.  It is evaluated like the linear mode's
// backward (single pass, decoupled look-back between chunks, scan_common.h),
// which gives chains x chunks x waves of parallelism instead of one lane per
// chain: a sequence of 512 steps over 32768 chains becomes 32768 waves
// instead of 512.
//
// A workgroup of W waves owns 64 consecutive channels of one batch row and
// one chunk of W * SEG steps; wave w holds SEG steps:
//   1. load the segment's U, x, c, dh (each element once), compute the
//      gc-free outputs (dU_r, dx) and store them, keep per step the five
//      numbers the adjoint needs, fold the segment into its map g -> A g + G;
//   2. wave 0 composes the W maps, takes the adjoint entering the chunk from
//      the chunk after it (look-back), publishes the adjoint leaving it, and
//      hands every segment its incoming adjoint;
//   3. replay the segment in reverse: dU_f, dU_cand, the v/b sums.
// Per-(chunk, chain) sums of dz_f c_prev, dz_r c_prev, dz_f, dz_r go to the
// workspace; param_reduce adds them over (chunk, batch row) in a fixed order.
#include "device_common.h"
#include "internal.h"
#include "scan_common.h"

namespace sru {
namespace {

struct BwdScanArgs {
    int64_t L, B, d, nC, chains;   // chains of one direction = B * d
    int ndir, dl, chunk;
    float alpha;
    const void *U;
    const void *x;
    const float *v, *b, *c0, *c_seq, *dh, *dc_last;
    float *dU, *dx, *dc0;
    bf16_bits_t *dU_lp;
    bool dx_acc;
    float *part;                   // [ndir, nC * B, 4, d]
    Lookback lb;
};

__device__ __forceinline__ void st_bf16_off(bf16_bits_t *base, uint32_t off, float v)
{
    *(bf16_bits_t *)((char *)base + off) = f32_to_bf16(v);
}

template <typename TU, typename TX, int W, int SEG, int WPE>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(WPE))) void bwd_scan(
    BwdScanArgs a)
{
    __shared__ float sA[W][64], sG[W][64], sC[W][64];
    __shared__ float sred[4][W][64];
    __shared__ uint32_t s_ticket;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int64_t tiles = a.chains / 64;
    // one chunk: no look-back, so no ticket either, and no wait can run out
    if (a.nC == 1 && blockIdx.x == 0 && threadIdx.x == 0) *a.lb.err = 0u;
    const int64_t tk = a.nC == 1 ? (int64_t)blockIdx.x : take_ticket(a.lb, &s_ticket);
    const int64_t k = a.nC - 1 - tk / tiles, tile = tk % tiles;       // last chunk first
    const int64_t ch0 = tile * 64, ch = ch0 + lane;
    const int64_t j0 = ch0 % a.d, bb = ch0 / a.d, j = j0 + lane;
    const int dl = a.dl;
    const float vf = a.v[(dl * 2 + 0) * a.d + j], vr = a.v[(dl * 2 + 1) * a.d + j];
    const float vfs = vf * kNegLog2e, vrs = vr * kNegLog2e;
    const float bfs = a.b[(dl * 2 + 0) * a.d + j] * kNegLog2e;
    const float brs = a.b[(dl * 2 + 1) * a.d + j] * kNegLog2e;
    const float alpha = a.alpha;
    const int64_t s_lo = k * a.chunk + wv * SEG;
    const SegRows sr(a.L, dl != 0, s_lo, SEG);

    // uniform bases at row t0 of the segment; the lane adds lane * size
    const int64_t ustride = a.B * a.ndir * 3 * a.d, xstride = a.B * a.d;
    const int64_t hstride = a.B * a.ndir * a.d;
    const int64_t uoff = (bb * a.ndir + dl) * 3 * a.d + j0, xoff = bb * a.d + j0;
    const int64_t hoff = (bb * a.ndir + dl) * a.d + j0;
    const char *ubase = (const char *)((const TU *)a.U + sr.t0 * ustride + uoff);
    const char *xbase = (const char *)((const TX *)a.x + sr.t0 * xstride + xoff);
    const char *cbase = (const char *)(a.c_seq + sr.t0 * hstride + hoff);
    const char *dhbase = (const char *)(a.dh + sr.t0 * hstride + hoff);
    char *dubase = (char *)(a.dU + sr.t0 * ustride + uoff);
    char *dxbase = (char *)(a.dx + sr.t0 * xstride + xoff);
    bf16_bits_t *lpbase = a.dU_lp ? a.dU_lp + sr.t0 * ustride + uoff : nullptr;
    const uint32_t urow = (uint32_t)(ustride * sizeof(TU)), xrow = (uint32_t)(xstride * sizeof(TX));
    const uint32_t hrow = (uint32_t)(hstride * sizeof(float));
    const uint32_t frow = (uint32_t)(ustride * sizeof(float)), fxrow = (uint32_t)(xstride * sizeof(float));
    const uint32_t lrow = (uint32_t)(ustride * sizeof(bf16_bits_t));
    const uint32_t ulane = (uint32_t)lane * sizeof(TU), xlane = (uint32_t)lane * sizeof(TX);
    const uint32_t flane = (uint32_t)lane * sizeof(float), llane = (uint32_t)lane * 2;
    const uint32_t ud = (uint32_t)(a.d * sizeof(TU)), fd = (uint32_t)(a.d * sizeof(float));
    const uint32_t ld = (uint32_t)(a.d * 2);

    // phase 1: everything that does not depend on the adjoint
    float kap[SEG], q[SEG], w[SEG], m[SEG], fgc[SEG], cp[SEG];
    float A = 1.0f, G = 0.0f;
    float svr = 0.0f, sbr = 0.0f;
    if (sr.nv1 >= 0) {
        float uf[SEG], ur[SEG], ux[SEG], xv[SEG], cc[SEG], dv[SEG];
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            const uint32_t r = sr.row(i);
            const uint32_t uo = r * urow + ulane;
            uf[i] = ld_off<TU>(ubase, uo);
            ur[i] = ld_off<TU>(ubase, uo + ud);
            ux[i] = ld_off<TU>(ubase, uo + 2 * ud);
            xv[i] = ld_off<TX>(xbase, r * xrow + xlane);
            cc[i] = ldf_off(cbase, r * hrow + flane);
            dv[i] = ldf_off(dhbase, r * hrow + flane);
        }
        // state before the segment's first step
        const float c_enter = s_lo == 0 ? (a.c0 ? a.c0[(dl * a.B + bb) * a.d + j] : 0.0f)
                                        : a.c_seq[(dl ? a.L - s_lo : s_lo - 1) * hstride + hoff + lane];
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            cp[i] = i == 0 ? c_enter : cc[i - 1];
            const Gate f = gate_scaled(fmaf(vfs, cp[i], fmaf(uf[i], kNegLog2e, bfs)));
            const Gate rg = gate_scaled(fmaf(vrs, cp[i], fmaf(ur[i], kNegLog2e, brs)));
            const float dzr = dv[i] * fmaf(-alpha, xv[i], cc[i]) * (rg.g * rg.gc);
            float dxh = dv[i] * rg.gc * alpha;
            q[i] = dv[i] * rg.g;
            m[i] = (cp[i] - ux[i]) * (f.g * f.gc);
            kap[i] = fmaf(m[i], vf, f.g);
            w[i] = dzr * vr;
            fgc[i] = f.gc;
            if (i <= sr.nv1) {
                const uint32_t r = sr.row(i);
                const uint32_t xo = r * fxrow + flane;
                if (a.dx_acc) dxh += ldf_off(dxbase, xo);
                st_off(dxbase, xo, dxh);
                st_off(dubase, r * frow + flane + fd, dzr);
                if (lpbase) st_bf16_off(lpbase, r * lrow + llane + ld, dzr);
                svr = fmaf(dzr, cp[i], svr);
                sbr += dzr;
            }
        }
#pragma unroll
        for (int i = SEG - 1; i >= 0; --i) {
            if (i <= sr.nv1) {
                G = fmaf(kap[i], G + q[i], w[i]);
                A *= kap[i];
            }
        }
    }
    sA[wv][lane] = A;
    sG[wv][lane] = G;
    __syncthreads();

    // phase 2 (wave 0): chunk map, adjoint in from the next chunk, out to the
    // previous one, and the incoming adjoint of every segment
    if (wv == 0) {
        float Ac = 1.0f, Gc = 0.0f;
#pragma unroll
        for (int s = W - 1; s >= 0; --s) {
            Gc = fmaf(sA[s][lane], Gc, sG[s][lane]);
            Ac *= sA[s][lane];
        }
        float gin;
        if (k == a.nC - 1)
            gin = a.dc_last ? a.dc_last[(dl * a.B + bb) * a.d + j] : 0.0f;
        else
            gin = consume(a.lb, (k + 1) * a.chains + ch, lane);
        if (k > 0) publish(a.lb, k * a.chains + ch, fmaf(Ac, gin, Gc));
        float gg = gin;
#pragma unroll
        for (int s = W - 1; s >= 0; --s) {
            sC[s][lane] = gg;
            gg = fmaf(sA[s][lane], gg, sG[s][lane]);
        }
    }
    __syncthreads();

    // phase 3: the adjoint-dependent outputs, last step of the segment first
    float gc = sC[wv][lane];
    float svf = 0.0f, sbf = 0.0f;
    if (sr.nv1 >= 0) {
#pragma unroll
        for (int i = SEG - 1; i >= 0; --i) {
            if (i <= sr.nv1) {
                const float dc = gc + q[i];
                const float dzf = dc * m[i];
                const float dux = dc * fgc[i];
                const uint32_t r = sr.row(i);
                const uint32_t uo = r * frow + flane;
                st_off(dubase, uo, dzf);
                st_off(dubase, uo + 2 * fd, dux);
                if (lpbase) {
                    const uint32_t lo = r * lrow + llane;
                    st_bf16_off(lpbase, lo, dzf);
                    st_bf16_off(lpbase, lo + 2 * ld, dux);
                }
                svf = fmaf(dzf, cp[i], svf);
                sbf += dzf;
                gc = fmaf(kap[i], dc, w[i]);
            }
        }
    }
    if (k == 0 && wv == 0 && a.dc0) a.dc0[(dl * a.B + bb) * a.d + j] = gc;

    // per-(chunk, chain) sums, the waves added in order
    sred[0][wv][lane] = svf;
    sred[1][wv][lane] = svr;
    sred[2][wv][lane] = sbf;
    sred[3][wv][lane] = sbr;
    __syncthreads();
    if (wv < 4) {
        float t = 0.0f;
#pragma unroll
        for (int s = 0; s < W; ++s) t += sred[wv][s][lane];
        a.part[((dl * a.nC * a.B + k * a.B + bb) * 4 + wv) * a.d + j] = t;
    }
}

// Workgroup shapes (waves x steps per wave): short sequences use short
// segments so that no wave idles; a chunk is never shorter than 64 steps,
// which bounds the workspace.
#ifndef SRU_BWDS_SHORT_L
#define SRU_BWDS_SHORT_L 256
#endif
#ifndef SRU_BWDS_SHORT_W
#define SRU_BWDS_SHORT_W 8
#endif
#ifndef SRU_BWDS_SHORT_SEG
#define SRU_BWDS_SHORT_SEG 8
#endif
#ifndef SRU_BWDS_LONG_W
#define SRU_BWDS_LONG_W 8
#endif
#ifndef SRU_BWDS_LONG_SEG
#define SRU_BWDS_LONG_SEG 8
#endif
constexpr int kShortW = SRU_BWDS_SHORT_W, kShortSeg = SRU_BWDS_SHORT_SEG;
constexpr int kLongW = SRU_BWDS_LONG_W, kLongSeg = SRU_BWDS_LONG_SEG;
static_assert(kShortW * kShortSeg >= 64 && kLongW * kLongSeg >= 64, "chunks of >= 64 steps");
constexpr int kMaxSeg = kShortSeg > kLongSeg ? kShortSeg : kLongSeg;


inline bool is_short(int64_t L) { return L <= SRU_BWDS_SHORT_L; }
inline int chunk_for(int64_t L) { return is_short(L) ? kShortW * kShortSeg : kLongW * kLongSeg; }

// 4 waves per SIMD: two 8-wave workgroups (or one 16-wave one) per CU
template <int W, int SEG, typename TU, typename TX>
void launch_cfg(const BwdScanArgs &a, unsigned grid, hipStream_t s)
{
    hipLaunchKernelGGL((bwd_scan<TU, TX, W, SEG, 4>), dim3(grid), dim3(W * 64), 0, s, a);
}

template <typename TU, typename TX>
void launch_typed(const BwdScanArgs &a, unsigned grid, hipStream_t s)
{
    if (is_short(a.L))
        launch_cfg<kShortW, kShortSeg, TU, TX>(a, grid, s);
    else
        launch_cfg<kLongW, kLongSeg, TU, TX>(a, grid, s);
}

}  // namespace

#ifndef SRU_BWDS_MIN_L
#define SRU_BWDS_MIN_L 129
#endif

bool backward_scan_ok(int64_t L, int64_t B, int64_t d, int ndir, bool fp32_inputs)
{
    // For short sequences of fp32 inputs the one-wave-per-64-chains kernel of
    // recurrence.hip streams better: the chunked form has few workgroups per
    // CU then, and their load and store phases barely overlap.
    if (d % 64 != 0 || (fp32_inputs && L < SRU_BWDS_MIN_L)) return false;
    // 32-bit byte offsets inside one segment of the widest stream
    const int64_t seg_bytes = (kMaxSeg + 1) * B * ndir * 3 * d * (int64_t)sizeof(float);
    const int64_t nC = (L + chunk_for(L) - 1) / chunk_for(L);
    return seg_bytes < (int64_t(1) << 31) && nC * (B * d / 64) < (int64_t(1) << 31);
}

size_t backward_scan_workspace_bytes(int64_t L, int64_t B, int64_t d, int ndir)
{
    // the control block + look-back states (64-bit) + partial sums; the
    // shortest chunk (64 steps) bounds the chunk count
    const int64_t nC = (L + 63) / 64;
    const int64_t floats = kCtrlWords + 2 * nC * B * d + (int64_t)ndir * nC * B * 4 * d;
    return (size_t)floats * sizeof(float);
}

hipError_t launch_backward_scan(const RecArgs &r, void *ws, float *dv, float *db, hipStream_t s)
{
    const int chunk = chunk_for(r.L);
    const int64_t nC = (r.L + chunk - 1) / chunk;
    const int64_t chains = r.B * r.d;
    float *wsf = (float *)ws;
    BwdScanArgs a{};
    a.L = r.L;
    a.B = r.B;
    a.d = r.d;
    a.nC = nC;
    a.chains = chains;
    a.ndir = r.ndir;
    a.chunk = chunk;
    a.alpha = r.alpha;
    a.U = r.U;
    a.x = r.x;
    a.v = r.v;
    a.b = r.b;
    a.c0 = r.c0;
    a.c_seq = r.c_seq_in;
    a.dh = r.dh;
    a.dc_last = r.dc_last;
    a.dU = r.dU;
    a.dx = r.dx;
    a.dc0 = r.dc0;
    a.dU_lp = r.dU_lp;
    // control block (error word, ticket), then the published adjoints, then
    // the partial sums.  The call's error word is r.err_word: the control
    // block's own, or one the caller keeps elsewhere.
    uint32_t *ctrl = (uint32_t *)wsf;
    a.lb.err = r.err_word ? r.err_word : ctrl + kErrWord;
    a.lb.ticket = ctrl + kTicketWord;
    if (nC > 1 && a.lb.err != ctrl + kErrWord)   // outside the region cleared below
        hipLaunchKernelGGL(scan_clear, dim3(1), dim3(256), 0, s, a.lb.err, (int64_t)1);
    a.lb.carry = (uint64_t *)(wsf + kCtrlWords);
    a.part = wsf + kCtrlWords + 2 * nC * chains;
    const int64_t clear_words = kCtrlWords + 2 * nC * chains;
    const unsigned grid = (unsigned)(nC * (chains / 64));
    // the highway dx sums both directions: the last direction writes it, the
    // one before adds to it (stream order serialises the launches)
    for (int dl = r.ndir - 1; dl >= 0; --dl) {
        a.dl = dl;
        a.dx_acc = dl != r.ndir - 1;
        // the error word is cleared once per call (before the first
        // direction), the ticket and the published adjoints before each
        const int64_t from = dl == r.ndir - 1 ? 0 : kTicketWord;
        if (nC > 1)
            hipLaunchKernelGGL(scan_clear, dim3(scan_clear_blocks(clear_words - from)), dim3(256),
                               0, s, ctrl + from, clear_words - from);
        if (r.u_bf16)
            r.x_bf16 ? launch_typed<bf16_bits, bf16_bits>(a, grid, s)
                     : launch_typed<bf16_bits, float>(a, grid, s);
        else
            r.x_bf16 ? launch_typed<float, bf16_bits>(a, grid, s)
                     : launch_typed<float, float>(a, grid, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !(dv || db)) return e;
    return launch_param_reduce(a.part, nC * r.B, r.d, r.ndir, dv, db, s);
}

}  // namespace sru
