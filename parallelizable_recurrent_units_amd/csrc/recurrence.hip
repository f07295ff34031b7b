// recurrence.hip -- forward and backward elementwise recurrence of one SRU
// layer on gfx950.
//
// Forward: Eqs. 2-5 of the SRU++ paper's background section (Lei, "When
// Attention Meets Fast Recurrence"), with the highway input scaled by alpha.
// Once U (Eq. 1) is known every (direction, batch, channel) chain is
// independent (the paper's remark after Eq. 5), so one lane owns one chain
// and keeps c in a register for the whole sequence.
//
// Backward: the chain rule through the same equations, walking each chain in
// reverse.  The gradient of c[t-1] is
//     gc = dc f + dz_f v_f + dz_r v_r,   dc = gc_next + dh r,
// and the per-chain sums over t of dz_f c[t-1], dz_r c[t-1], dz_f, dz_r (the
// parameter gradients of v and b) are kept in registers and reduced over the
// batch afterwards in a fixed order (bit-reproducible, no float atomics).
//
// Memory system design (HBM-bound, ~0.6 flop/byte):
//  * A wavefront owns 64 consecutive channels of one (direction, batch) row.
//    Per timestep it needs four 256-byte rows (U_f, U_r, U_cand, x).  Instead
//    of four 4-byte-per-lane loads, ONE 16-byte-per-lane load fetches all
//    four rows (lanes 0-15 U_f, 16-31 U_r, 32-47 U_cand, 48-63 x; for bf16
//    inputs one load covers two timesteps).  The packet is transposed through
//    a 1 KB LDS slot so each lane then reads its own channel.
//  * Packets for the next R timesteps stay in flight in a register ring, so
//    a wave keeps R KB of loads outstanding: the kernel is latency-bound at
//    the small grids of long sequences (e.g. 512 waves for B*d = 32768), and
//    bytes in flight per wave is what sets its bandwidth.
//  * Outputs are staged the same way and leave as 16-byte-per-lane stores.
//  * Each block is one wavefront, so the LDS slots are private to it and no
//    barrier is needed (LDS operations of one wave execute in order).
#include "device_common.h"
#include "internal.h"

namespace sru {
namespace {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Generic forward: one thread per chain, scalar loads.  Used for any d that is
// not a multiple of 64 and for mixed U/x dtypes.
// ---------------------------------------------------------------------------
template <typename TU, typename TX>
__global__ __launch_bounds__(256) void fwd_generic(RecArgs a)
{
    const int64_t chains = (int64_t)a.ndir * a.B * a.d;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= chains) return;
    const int64_t j = g % a.d;
    const int64_t bb = (g / a.d) % a.B;
    const int dl = (int)(g / (a.B * a.d));
    const TU *U = (const TU *)a.U;
    const TX *X = (const TX *)a.x;
    const float vf = a.v[(dl * 2 + 0) * a.d + j], vr = a.v[(dl * 2 + 1) * a.d + j];
    const float bf = a.b[(dl * 2 + 0) * a.d + j], br = a.b[(dl * 2 + 1) * a.d + j];
    float c = a.c0 ? a.c0[(dl * a.B + bb) * a.d + j] : 0.0f;
    for (int64_t s = 0; s < a.L; ++s) {
        const int64_t t = dl ? (a.L - 1 - s) : s;
        const int64_t ub = ((t * a.B + bb) * a.ndir + dl) * 3 * a.d + j;
        const float uf = load_as_f32(U + ub), ur = load_as_f32(U + ub + a.d);
        const float ux = load_as_f32(U + ub + 2 * a.d);
        const float xv = load_as_f32(X + (t * a.B + bb) * a.d + j);
        const Gate f = gate(fmaf(vf, c, uf + bf));
        const Gate r = gate(fmaf(vr, c, ur + br));
        c = fmaf(f.g, c, f.gc * ux);
        const float ax = a.alpha * xv;
        const int64_t o = ((t * a.B + bb) * a.ndir + dl) * a.d + j;
        a.h[o] = fmaf(r.g, c, r.gc * ax);
        if (a.c_seq) a.c_seq[o] = c;
    }
    if (a.c_last) a.c_last[(dl * a.B + bb) * a.d + j] = c;
}

// ---------------------------------------------------------------------------
// Fast forward: one wavefront per 64 channels, packet loads + register ring.
// BF16 = U and x both bf16 (a packet then carries two timesteps), else both
// fp32.  Requires d % 64 == 0 and 16-byte aligned tensors.
// ---------------------------------------------------------------------------
template <bool BF16, int R>
__global__ __launch_bounds__(kWave) void fwd_fast(RecArgs a)
{
    __shared__ uint4 in_slot[kWave];     // one packet, 1 KB
    __shared__ float out_slot[4 * kWave];  // h, c for two timesteps, 1 KB

    const int lane = threadIdx.x;
    const int64_t gpr = a.d / kWave;                 // wave groups per row
    const int64_t w = blockIdx.x;
    const int dl = (int)(w / (a.B * gpr));
    const int64_t rem = w % (a.B * gpr);
    const int64_t bb = rem / gpr;
    const int64_t j0 = (rem % gpr) * kWave;
    const int64_t j = j0 + lane;
    const int64_t L = a.L;

    // time index of direction-step s
    auto tix = [&](int64_t s) -> int64_t { return dl ? (L - 1 - s) : s; };

    // ---- input packet addressing (per lane) ----
    constexpr int SPP = BF16 ? 2 : 1;                // timesteps per packet
    constexpr int ESZ = BF16 ? 2 : 4;                // element bytes
    const int e_in = BF16 ? (lane >> 5) : 0;         // timestep within packet
    const int q_in = BF16 ? ((lane >> 3) & 3) : (lane >> 4);  // 0 Uf 1 Ur 2 Ux 3 x
    const int sub_in = BF16 ? (lane & 7) : (lane & 15);
    const int64_t cpl = 16 / ESZ;                    // channels per lane
    const char *in_base;
    int64_t in_row;   // element offset of this lane's data at time t = 0
    int64_t in_tstride;  // element stride per time index
    if (q_in < 3) {
        in_base = (const char *)a.U;
        in_row = (bb * a.ndir + dl) * 3 * a.d + q_in * a.d + j0 + cpl * sub_in;
        in_tstride = a.B * a.ndir * 3 * a.d;
    } else {
        in_base = (const char *)a.x;
        in_row = bb * a.d + j0 + cpl * sub_in;
        in_tstride = a.B * a.d;
    }
    const int64_t NP = (L + SPP - 1) / SPP;          // packets
    auto load_packet = [&](int64_t p) -> uint4 {
        int64_t s = p * SPP + e_in;
        s = s < L ? s : L - 1;                       // clamp: stays in bounds
        const int64_t off = (in_row + tix(s) * in_tstride) * ESZ;
        return *(const uint4 *)(in_base + off);
    };

    // ---- output addressing (per lane), two timesteps per flush ----
    const int e_out = lane >> 5;
    const int q_out = (lane >> 4) & 1;               // 0 h, 1 c
    const int sub_out = lane & 15;
    float *out_base = q_out ? a.c_seq : a.h;
    const int64_t out_row = (bb * a.ndir + dl) * a.d + j0 + 4 * sub_out;
    const int64_t out_tstride = a.B * a.ndir * a.d;
    const bool out_on = (out_base != nullptr);

    const float vf = a.v[(dl * 2 + 0) * a.d + j], vr = a.v[(dl * 2 + 1) * a.d + j];
    const float bf = a.b[(dl * 2 + 0) * a.d + j], br = a.b[(dl * 2 + 1) * a.d + j];
    const float alpha = a.alpha;
    float c = a.c0 ? a.c0[(dl * a.B + bb) * a.d + j] : 0.0f;

    uint4 ring[R];
#pragma unroll
    for (int i = 0; i < R; ++i) ring[i] = load_packet(i);

    const float *inf = (const float *)in_slot;
    const bf16_bits *inh = (const bf16_bits *)in_slot;

    auto step = [&](int e, int64_t s) {
        float uf, ur, ux, xv;
        if (BF16) {
            uf = bf16_to_f32(inh[e * 256 + 0 * 64 + lane]);
            ur = bf16_to_f32(inh[e * 256 + 1 * 64 + lane]);
            ux = bf16_to_f32(inh[e * 256 + 2 * 64 + lane]);
            xv = bf16_to_f32(inh[e * 256 + 3 * 64 + lane]);
        } else {
            uf = inf[0 * 64 + lane];
            ur = inf[1 * 64 + lane];
            ux = inf[2 * 64 + lane];
            xv = inf[3 * 64 + lane];
        }
        const Gate f = gate(fmaf(vf, c, uf + bf));
        const Gate r = gate(fmaf(vr, c, ur + br));
        c = fmaf(f.g, c, f.gc * ux);
        const float ax = alpha * xv;
        const int pe = (int)(s & 1);
        out_slot[pe * 128 + lane] = fmaf(r.g, c, r.gc * ax);
        out_slot[pe * 128 + 64 + lane] = c;
    };
    auto flush = [&](int64_t s_even) {
        // timesteps s_even and s_even + 1 (the latter only if < L)
        const float4 val = ((const float4 *)out_slot)[lane];
        const int64_t s = s_even + e_out;
        if (out_on && s < L) {
            *(float4 *)(out_base + out_row + tix(s) * out_tstride) = val;
        }
    };

    for (int64_t p0 = 0; p0 < NP; p0 += R) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t p = p0 + i;
            if (p < NP) {
                in_slot[lane] = ring[i];
                ring[i] = load_packet(p + R);
                if (BF16) {
                    const int64_t s = 2 * p;
                    step(0, s);
                    if (s + 1 < L) step(1, s + 1);
                    flush(s);
                } else {
                    step(0, p);
                    if ((p & 1) || p == L - 1) flush(p & ~(int64_t)1);
                }
            }
        }
    }
    if (a.c_last) a.c_last[(dl * a.B + bb) * a.d + j] = c;
}

// ---------------------------------------------------------------------------
// Generic backward (one direction per launch): one thread per chain.
// ---------------------------------------------------------------------------
template <typename TU, typename TX>
__global__ __launch_bounds__(256) void bwd_generic(RecArgs a)
{
    const int64_t chains = a.B * a.d;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= chains) return;
    const int dl = a.dir;
    const int64_t j = g % a.d;
    const int64_t bb = g / a.d;
    const TU *U = (const TU *)a.U;
    const TX *X = (const TX *)a.x;
    const float vf = a.v[(dl * 2 + 0) * a.d + j], vr = a.v[(dl * 2 + 1) * a.d + j];
    const float bf = a.b[(dl * 2 + 0) * a.d + j], br = a.b[(dl * 2 + 1) * a.d + j];
    const float c0 = a.c0 ? a.c0[(dl * a.B + bb) * a.d + j] : 0.0f;
    const float alpha = a.alpha;
    const int64_t L = a.L;
    auto tix = [&](int64_t s) -> int64_t { return dl ? (L - 1 - s) : s; };
    auto oidx = [&](int64_t t) -> int64_t { return ((t * a.B + bb) * a.ndir + dl) * a.d + j; };

    float gc = a.dc_last ? a.dc_last[(dl * a.B + bb) * a.d + j] : 0.0f;
    float c = a.c_seq_in[oidx(tix(L - 1))];
    float svf = 0.f, svr = 0.f, sbf = 0.f, sbr = 0.f;
    for (int64_t s = L - 1; s >= 0; --s) {
        const int64_t t = tix(s);
        const float cp = s > 0 ? a.c_seq_in[oidx(tix(s - 1))] : c0;
        const int64_t ub = ((t * a.B + bb) * a.ndir + dl) * 3 * a.d + j;
        const float uf = load_as_f32(U + ub), ur = load_as_f32(U + ub + a.d);
        const float ux = load_as_f32(U + ub + 2 * a.d);
        const int64_t xi = (t * a.B + bb) * a.d + j;
        const float xv = load_as_f32(X + xi);
        const float dhv = a.dh[oidx(t)];
        const Gate f = gate(fmaf(vf, cp, uf + bf));
        const Gate r = gate(fmaf(vr, cp, ur + br));
        const float dc = fmaf(dhv, r.g, gc);
        const float dr = dhv * fmaf(-alpha, xv, c);
        float dxh = dhv * r.gc * alpha;
        if (a.dx_accumulate) dxh += a.dx[xi];
        const float dux = dc * f.gc;
        const float df = dc * (cp - ux);
        const float dzf = df * (f.g * f.gc);
        const float dzr = dr * (r.g * r.gc);
        svf = fmaf(dzf, cp, svf);
        svr = fmaf(dzr, cp, svr);
        sbf += dzf;
        sbr += dzr;
        gc = fmaf(dc, f.g, fmaf(dzf, vf, dzr * vr));
        a.dU[ub] = dzf;
        a.dU[ub + a.d] = dzr;
        a.dU[ub + 2 * a.d] = dux;
        a.dx[xi] = dxh;
        c = cp;
    }
    if (a.dc0) a.dc0[(dl * a.B + bb) * a.d + j] = gc;
    float *pp = a.partials + ((int64_t)(dl * a.B + bb) * 4) * a.d + j;
    pp[0 * a.d] = svf;
    pp[1 * a.d] = svr;
    pp[2 * a.d] = sbf;
    pp[3 * a.d] = sbr;
}

// ---------------------------------------------------------------------------
// Fast backward (fp32 U and x, d % 64 == 0): one wavefront per 64 channels.
// Per timestep two input packets:
//   A: lanes 0-15 U_f, 16-31 U_r, 32-47 U_cand, 48-63 x          (time t)
//   B: lanes 0-15 c[t_prev], 16-31 dh[t], 32-47 dx[t] (accumulate), 48-63 idle
// and one output packet: lanes 0-15 dU_f, 16-31 dU_r, 32-47 dU_cand, 48-63 dx.
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(kWave) void bwd_fast(RecArgs a)
{
    __shared__ uint4 slot_a[kWave];
    __shared__ uint4 slot_b[kWave];
    __shared__ float out_slot[4 * kWave];

    const int lane = threadIdx.x;
    const int dl = a.dir;
    const int64_t gpr = a.d / kWave;
    const int64_t w = blockIdx.x;
    const int64_t bb = w / gpr;
    const int64_t j0 = (w % gpr) * kWave;
    const int64_t j = j0 + lane;
    const int64_t L = a.L;
    auto tix = [&](int64_t s) -> int64_t { return dl ? (L - 1 - s) : s; };

    const int q = lane >> 4;
    const int sub = lane & 15;
    // packet A
    const char *pa_base;
    int64_t pa_row, pa_ts;
    if (q < 3) {
        pa_base = (const char *)a.U;
        pa_row = (bb * a.ndir + dl) * 3 * a.d + q * a.d + j0 + 4 * sub;
        pa_ts = a.B * a.ndir * 3 * a.d;
    } else {
        pa_base = (const char *)a.x;
        pa_row = bb * a.d + j0 + 4 * sub;
        pa_ts = a.B * a.d;
    }
    // packet B
    const char *pb_base;
    int64_t pb_row, pb_ts, pb_soff;
    const bool dxacc = a.dx_accumulate;
    if (q == 0) {          // c at the previous direction-step
        pb_base = (const char *)a.c_seq_in;
        pb_row = (bb * a.ndir + dl) * a.d + j0 + 4 * sub;
        pb_ts = a.B * a.ndir * a.d;
        pb_soff = -1;
    } else if (q == 1) {   // dh
        pb_base = (const char *)a.dh;
        pb_row = (bb * a.ndir + dl) * a.d + j0 + 4 * sub;
        pb_ts = a.B * a.ndir * a.d;
        pb_soff = 0;
    } else {               // dx (read only when accumulating; lanes 48-63 reuse it)
        pb_base = (const char *)a.dx;
        pb_row = bb * a.d + j0 + 4 * sub;
        pb_ts = a.B * a.d;
        pb_soff = 0;
    }
    auto clampL = [&](int64_t s) -> int64_t { return s < 0 ? 0 : (s >= L ? L - 1 : s); };
    // direction-step s is processed at iteration k = L-1-s
    auto load_a = [&](int64_t k) -> uint4 {
        const int64_t s = clampL(L - 1 - k);
        return *(const uint4 *)(pa_base + (pa_row + tix(s) * pa_ts) * 4);
    };
    auto load_b = [&](int64_t k) -> uint4 {
        const int64_t s = clampL(L - 1 - k + pb_soff);
        if (q >= 2 && !dxacc) return make_uint4(0, 0, 0, 0);
        return *(const uint4 *)(pb_base + (pb_row + tix(s) * pb_ts) * 4);
    };

    // output packet
    float *po_base = q < 3 ? a.dU : a.dx;
    const int64_t po_row = q < 3 ? ((bb * a.ndir + dl) * 3 * a.d + q * a.d + j0 + 4 * sub)
                                 : (bb * a.d + j0 + 4 * sub);
    const int64_t po_ts = q < 3 ? a.B * a.ndir * 3 * a.d : a.B * a.d;

    const float vf = a.v[(dl * 2 + 0) * a.d + j], vr = a.v[(dl * 2 + 1) * a.d + j];
    const float bf = a.b[(dl * 2 + 0) * a.d + j], br = a.b[(dl * 2 + 1) * a.d + j];
    const float c0 = a.c0 ? a.c0[(dl * a.B + bb) * a.d + j] : 0.0f;
    const float alpha = a.alpha;
    float gc = a.dc_last ? a.dc_last[(dl * a.B + bb) * a.d + j] : 0.0f;
    float c = a.c_seq_in[((tix(L - 1) * a.B + bb) * a.ndir + dl) * a.d + j];
    float svf = 0.f, svr = 0.f, sbf = 0.f, sbr = 0.f;

    uint4 ring_a[R], ring_b[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        ring_a[i] = load_a(i);
        ring_b[i] = load_b(i);
    }
    const float *fa = (const float *)slot_a;
    const float *fb = (const float *)slot_b;

    for (int64_t k0 = 0; k0 < L; k0 += R) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t k = k0 + i;
            if (k < L) {
                const int64_t s = L - 1 - k;
                slot_a[lane] = ring_a[i];
                slot_b[lane] = ring_b[i];
                ring_a[i] = load_a(k + R);
                ring_b[i] = load_b(k + R);
                const float uf = fa[lane], ur = fa[64 + lane], ux = fa[128 + lane];
                const float xv = fa[192 + lane];
                const float cp = s > 0 ? fb[lane] : c0;
                const float dhv = fb[64 + lane];
                const Gate f = gate(fmaf(vf, cp, uf + bf));
                const Gate r = gate(fmaf(vr, cp, ur + br));
                const float dc = fmaf(dhv, r.g, gc);
                const float dr = dhv * fmaf(-alpha, xv, c);
                float dxh = dhv * r.gc * alpha;
                if (dxacc) dxh += fb[128 + lane];
                const float dux = dc * f.gc;
                const float df = dc * (cp - ux);
                const float dzf = df * (f.g * f.gc);
                const float dzr = dr * (r.g * r.gc);
                svf = fmaf(dzf, cp, svf);
                svr = fmaf(dzr, cp, svr);
                sbf += dzf;
                sbr += dzr;
                gc = fmaf(dc, f.g, fmaf(dzf, vf, dzr * vr));
                c = cp;
                out_slot[lane] = dzf;
                out_slot[64 + lane] = dzr;
                out_slot[128 + lane] = dux;
                out_slot[192 + lane] = dxh;
                const float4 val = ((const float4 *)out_slot)[lane];
                *(float4 *)(po_base + po_row + tix(s) * po_ts) = val;
            }
        }
    }
    if (a.dc0) a.dc0[(dl * a.B + bb) * a.d + j] = gc;
    float *pp = a.partials + ((int64_t)(dl * a.B + bb) * 4) * a.d + j;
    pp[0 * a.d] = svf;
    pp[1 * a.d] = svr;
    pp[2 * a.d] = sbf;
    pp[3 * a.d] = sbr;
}

// dv[dl, g, j] = sum_b partials[dl, b, g, j]; db[dl, g, j] likewise with rows
// 2, 3.  b increases, so the result does not depend on the launch shape.
__global__ __launch_bounds__(256) void param_reduce(const float *__restrict__ part, int64_t B,
                                                     int64_t d, int ndir, float *dv, float *db)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)ndir * 4 * d;
    if (i >= total) return;
    const int64_t j = i % d;
    const int g = (int)((i / d) % 4);
    const int dl = (int)(i / (4 * d));
    float s = 0.0f;
    for (int64_t bb = 0; bb < B; ++bb) s += part[((dl * B + bb) * 4 + g) * d + j];
    if (g < 2) {
        if (dv) dv[(dl * 2 + g) * d + j] = s;
    } else {
        if (db) db[(dl * 2 + (g - 2)) * d + j] = s;
    }
}

template <typename TU, typename TX>
hipError_t fwd_generic_launch(const RecArgs &a, hipStream_t s)
{
    const int64_t chains = (int64_t)a.ndir * a.B * a.d;
    const int64_t blocks = (chains + 255) / 256;
    hipLaunchKernelGGL((fwd_generic<TU, TX>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename TU, typename TX>
hipError_t bwd_generic_launch(const RecArgs &a, hipStream_t s)
{
    const int64_t chains = a.B * a.d;
    const int64_t blocks = (chains + 255) / 256;
    hipLaunchKernelGGL((bwd_generic<TU, TX>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

constexpr int kFwdRingF32 = 16;
constexpr int kFwdRingBF16 = 16;
constexpr int kBwdRing = 12;

hipError_t launch_forward(const RecArgs &a, hipStream_t s)
{
    const bool fast = (a.d % kWave == 0) && (a.u_bf16 == a.x_bf16);
    if (fast) {
        const int64_t waves = (int64_t)a.ndir * a.B * (a.d / kWave);
        if (a.u_bf16)
            hipLaunchKernelGGL((fwd_fast<true, kFwdRingBF16>), dim3((unsigned)waves),
                               dim3(kWave), 0, s, a);
        else
            hipLaunchKernelGGL((fwd_fast<false, kFwdRingF32>), dim3((unsigned)waves),
                               dim3(kWave), 0, s, a);
        return hipGetLastError();
    }
    if (a.u_bf16) {
        return a.x_bf16 ? fwd_generic_launch<bf16_bits, bf16_bits>(a, s)
                        : fwd_generic_launch<bf16_bits, float>(a, s);
    }
    return a.x_bf16 ? fwd_generic_launch<float, bf16_bits>(a, s)
                    : fwd_generic_launch<float, float>(a, s);
}

hipError_t launch_backward_dir(const RecArgs &a, hipStream_t s)
{
    const bool fast = (a.d % kWave == 0) && !a.u_bf16 && !a.x_bf16;
    if (fast) {
        const int64_t waves = a.B * (a.d / kWave);
        hipLaunchKernelGGL((bwd_fast<kBwdRing>), dim3((unsigned)waves), dim3(kWave), 0, s, a);
        return hipGetLastError();
    }
    if (a.u_bf16) {
        return a.x_bf16 ? bwd_generic_launch<bf16_bits, bf16_bits>(a, s)
                        : bwd_generic_launch<bf16_bits, float>(a, s);
    }
    return a.x_bf16 ? bwd_generic_launch<float, bf16_bits>(a, s)
                    : bwd_generic_launch<float, float>(a, s);
}

hipError_t launch_param_reduce(const float *partials, int64_t B, int64_t d, int ndir,
                               float *dv, float *db, hipStream_t s)
{
    const int64_t total = (int64_t)ndir * 4 * d;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(param_reduce, dim3((unsigned)blocks), dim3(256), 0, s, partials, B, d,
                       ndir, dv, db);
    return hipGetLastError();
}

}  // namespace sru
