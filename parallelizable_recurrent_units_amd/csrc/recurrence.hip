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
        const float yf = fmaf(vf, c, uf + bf) * kNegLog2e;
        const float yr = fmaf(vr, c, ur + br) * kNegLog2e;
        c = gate_blend(yf, c, ux);
        const int64_t o = ((t * a.B + bb) * a.ndir + dl) * a.d + j;
        a.h[o] = gate_blend(yr, c, a.alpha * xv);
        if (a.c_seq) a.c_seq[o] = c;
    }
    if (a.c_last) a.c_last[(dl * a.B + bb) * a.d + j] = c;
}

// ---------------------------------------------------------------------------
// Fast forward: one wavefront per 64 channels, packet loads + register ring.
// BF16 = U and x both bf16 (a packet then carries two timesteps), else both
// fp32.  Requires d % 64 == 0, 16-byte aligned tensors, every tensor below
// 2 GiB and time strides below 16 MiB (the host checks; addresses are then
// a loop-invariant per-lane pointer plus a 24-bit x 24-bit product).
//
// The sequence is walked in groups of G packets.  Per group the wave writes
// G packets to LDS, refills those ring slots with the packets R ahead, reads
// back every lane's own values, runs the G*SPP recurrence steps, and writes
// h and c as 16-byte stores: one LDS round trip per group instead of per
// step.  The loop body has no conditional memory operations (prefetch
// indices are clamped), so the compiler's wait counts stay exact; the last
// L mod (G*SPP) steps run in a short tail with direct loads.  With at most
// one wave per SIMD on long sequences, the instruction count per step bounds
// the kernel, so the gate constants are pre-scaled by -log2(e) (each gate is
// fma, fma, min, exp, add, rcp, mul).
// ---------------------------------------------------------------------------
template <bool BF16, int R, int G>
__global__ __launch_bounds__(kWave) void fwd_fast(RecArgs a)
{
    static_assert(R % G == 0, "ring holds whole groups");
    constexpr int SPP = BF16 ? 2 : 1;                // timesteps per packet
    constexpr int S = G * SPP;                       // timesteps per group
    static_assert(S % 2 == 0, "outputs leave two timesteps per store");
    __shared__ uint4 in_slot[G * kWave];             // G packets
    __shared__ float out_slot[S * 2 * kWave];        // h, c of S timesteps

    const int lane = threadIdx.x;
    const int64_t gpr = a.d / kWave;                 // wave groups per row
    const int64_t w = blockIdx.x;
    const int dl = (int)(w / (a.B * gpr));
    const int64_t rem = w % (a.B * gpr);
    const int64_t bb = rem / gpr;
    const int64_t j0 = (rem % gpr) * kWave;
    const int64_t j = j0 + lane;
    const int64_t L = a.L;
    auto tix = [&](int64_t s) -> int64_t { return dl ? (L - 1 - s) : s; };

    // ---- input packets: lane = (timestep in packet, stream, channels) ----
    constexpr int ESZ = BF16 ? 2 : 4;                // element bytes
    const int e_in = BF16 ? (lane >> 5) : 0;
    const int q_in = BF16 ? ((lane >> 3) & 3) : (lane >> 4);  // 0 Uf 1 Ur 2 Ux 3 x
    const int sub_in = BF16 ? (lane & 7) : (lane & 15);
    const int64_t cpl = 16 / ESZ;                    // channels per lane
    const char *in_ptr;
    uint32_t in_stride;                              // bytes per time index
    if (q_in < 3) {
        in_ptr = (const char *)a.U +
                 ((bb * a.ndir + dl) * 3 * a.d + q_in * a.d + j0 + cpl * sub_in) * ESZ;
        in_stride = (uint32_t)(a.B * a.ndir * 3 * a.d * ESZ);
    } else {
        in_ptr = (const char *)a.x + (bb * a.d + j0 + cpl * sub_in) * ESZ;
        in_stride = (uint32_t)(a.B * a.d * ESZ);
    }
    // packet p holds direction-steps p*SPP .. p*SPP + SPP - 1; this lane's
    // time index is tin(p) + e_in (direction 0) or tin(p) + 1 - e_in
    // (direction 1), tin uniform
    if (BF16) in_ptr += (int64_t)(dl ? 1 - e_in : e_in) * in_stride;
    const int64_t Pmax = L / SPP - 1;                // last packet fully inside
    auto load_packet = [&](int64_t p) -> uint4 {
        p = p < Pmax ? p : Pmax;                     // clamp: stays in bounds
        const uint32_t t = (uint32_t)(dl ? (L - SPP - p * SPP) : p * SPP);
        return *(const uint4 *)(in_ptr + __umul24(t, in_stride));
    };

    // ---- outputs: lane = (step parity, h|c, 4 channels), 2 steps per store
    const int e_out = lane >> 5;
    const int q_out = (lane >> 4) & 1;               // 0 h, 1 c
    const int sub_out = lane & 15;
    float *out_t = q_out ? a.c_seq : a.h;
    const bool out_on = (out_t != nullptr);
    const uint32_t out_stride = (uint32_t)(a.B * a.ndir * a.d * 4);
    char *out_ptr = out_on ? (char *)(out_t + (bb * a.ndir + dl) * a.d + j0 + 4 * sub_out) +
                                 (int64_t)(dl ? 1 - e_out : e_out) * out_stride
                           : nullptr;

    const float vfs = a.v[(dl * 2 + 0) * a.d + j] * kNegLog2e;
    const float vrs = a.v[(dl * 2 + 1) * a.d + j] * kNegLog2e;
    const float bfs = a.b[(dl * 2 + 0) * a.d + j] * kNegLog2e;
    const float brs = a.b[(dl * 2 + 1) * a.d + j] * kNegLog2e;
    const float alpha = a.alpha;
    float c = a.c0 ? a.c0[(dl * a.B + bb) * a.d + j] : 0.0f;

    auto cell = [&](float uf, float ur, float ux, float xv, float &h) {
        const float yf = fmaf(vfs, c, fmaf(uf, kNegLog2e, bfs));
        const float yr = fmaf(vrs, c, fmaf(ur, kNegLog2e, brs));
        c = gate_blend(yf, c, ux);                   // f c + (1 - f) U_cand
        h = gate_blend(yr, c, alpha * xv);           // r c + (1 - r) alpha x
    };

    const int64_t groups = L / S;                    // full groups
    if (groups > 0) {
        uint4 ring[R];
#pragma unroll
        for (int i = 0; i < R; ++i) ring[i] = load_packet(i);
        const float *inf = (const float *)in_slot;
        const bf16_bits *inh = (const bf16_bits *)in_slot;
        int64_t gi = 0;
        for (;;) {
#pragma unroll
            for (int rg = 0; rg < R / G; ++rg) {
                const int64_t p0 = (gi + rg) * G;    // first packet of this group
#pragma unroll
                for (int i = 0; i < G; ++i) in_slot[i * kWave + lane] = ring[rg * G + i];
#pragma unroll
                for (int i = 0; i < G; ++i) ring[rg * G + i] = load_packet(p0 + R + i);
                float uf[S], ur[S], ux[S], xv[S];
#pragma unroll
                for (int st = 0; st < S; ++st) {
                    if (BF16) {
                        const bf16_bits *hp = inh + (st / 2) * 512 + (st % 2) * 256 + lane;
                        uf[st] = bf16_to_f32(hp[0]);
                        ur[st] = bf16_to_f32(hp[64]);
                        ux[st] = bf16_to_f32(hp[128]);
                        xv[st] = bf16_to_f32(hp[192]);
                    } else {
                        const float *fp = inf + st * 256 + lane;
                        uf[st] = fp[0];
                        ur[st] = fp[64];
                        ux[st] = fp[128];
                        xv[st] = fp[192];
                    }
                }
#pragma unroll
                for (int st = 0; st < S; ++st) {
                    float h;
                    cell(uf[st], ur[st], ux[st], xv[st], h);
                    out_slot[st * 128 + lane] = h;
                    out_slot[st * 128 + 64 + lane] = c;
                }
                if (out_on) {
#pragma unroll
                    for (int m = 0; m < S / 2; ++m) {
                        const float4 val = ((const float4 *)out_slot)[m * 64 + lane];
                        const int64_t st0 = p0 * SPP + 2 * m;       // even step of the pair
                        const uint32_t t = (uint32_t)(dl ? (L - 2 - st0) : st0);
                        *(float4 *)(out_ptr + __umul24(t, out_stride)) = val;
                    }
                }
                if (gi + rg + 1 >= groups) goto tail;
            }
            gi += R / G;
        }
    }
tail:
    // remaining L mod S timesteps: direct per-lane loads
    for (int64_t st = groups * S; st < L; ++st) {
        const int64_t t = tix(st);
        const int64_t ub = ((t * a.B + bb) * a.ndir + dl) * 3 * a.d + j;
        float uf, ur, ux, xv;
        if (BF16) {
            const bf16_bits *U = (const bf16_bits *)a.U;
            uf = bf16_to_f32(U[ub]);
            ur = bf16_to_f32(U[ub + a.d]);
            ux = bf16_to_f32(U[ub + 2 * a.d]);
            xv = bf16_to_f32(((const bf16_bits *)a.x)[(t * a.B + bb) * a.d + j]);
        } else {
            const float *U = (const float *)a.U;
            uf = U[ub];
            ur = U[ub + a.d];
            ux = U[ub + 2 * a.d];
            xv = ((const float *)a.x)[(t * a.B + bb) * a.d + j];
        }
        float h;
        cell(uf, ur, ux, xv, h);
        const int64_t o = ((t * a.B + bb) * a.ndir + dl) * a.d + j;
        a.h[o] = h;
        if (a.c_seq) a.c_seq[o] = c;
    }
    if (a.c_last) a.c_last[(dl * a.B + bb) * a.d + j] = c;
}

// ---------------------------------------------------------------------------
// Two-wave forward (d % 64 == 0, same size limits as fwd_fast): a workgroup of
// two waves per (direction, batch row, 64 channels).  Wave 0 carries the
// state: it reads the U_f and U_cand rows and computes c (Eqs. 2 and 4),
// writing c_seq and c_last.  Wave 1 reads the U_r and x rows and computes h
// (Eqs. 3 and 5) one group of steps behind, taking c[t-1] and c[t] from an
// LDS ring the state wave fills.  Each wave issues about half the
// instructions of a step, so grids with fewer waves than SIMDs (long
// sequences over few chains, where one wave per 64 chains is limited by its
// own instruction issue) run twice as many waves at half the work each.
// Per wave, one 16-byte-per-lane load fetches its two streams for SPP steps
// (fp32 2, bf16 4): lanes 0-31 stream 0, lanes 32-63 stream 1.  Both waves
// walk the same loop (one barrier per group) and keep their packets in one
// register ring with the same slot sequence: at iteration g wave r works on
// group g - r.
// ---------------------------------------------------------------------------
template <bool BF16, int R, int G>
__global__ __launch_bounds__(2 * kWave) void fwd_split(RecArgs a)
{
    static_assert(R % G == 0, "ring holds whole groups");
    constexpr int ESZ = BF16 ? 2 : 4;
    constexpr int SPP = BF16 ? 4 : 2;                // steps per packet
    constexpr int S = G * SPP;                       // steps per group
    constexpr int NRG = R / G;                       // groups in the ring
    static_assert(S % 4 == 0, "outputs leave four steps per store");
    constexpr int LPS = 32 / SPP;                    // lanes per (stream, step)
    constexpr int CPL = 16 / ESZ;                    // channels per lane
    __shared__ uint4 slot_all[2][G * kWave];
    __shared__ float ostage_all[2][S * kWave];
    __shared__ float cring[2][S * kWave];

    const int role = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    uint4 *slot = slot_all[role];
    float *ostage = ostage_all[role];
    const int64_t gpr = a.d / kWave;
    const int64_t w = blockIdx.x;
    const int dl = (int)(w / (a.B * gpr));
    const int64_t rem = w % (a.B * gpr);
    const int64_t bb = rem / gpr;
    const int64_t j0 = (rem % gpr) * kWave;
    const int64_t j = j0 + lane;
    const int64_t L = a.L;
    auto tix = [&](int64_t s) -> int64_t { return dl ? (L - 1 - s) : s; };

    // ---- input packets: lane = (stream, step in packet, channels) ---------
    const int q_in = lane >> 5;                      // 0: U_f | U_r, 1: U_cand | x
    const int e_in = (lane & 31) / LPS;
    const int sub_in = lane % LPS;
    const char *in_ptr;
    uint32_t in_stride;
    const int64_t ch_off = j0 + (int64_t)CPL * sub_in;
    if (role == 0 || q_in == 0) {                    // a U row: f / cand or r
        const int gate = role == 0 ? 2 * q_in : 1;
        in_ptr = (const char *)a.U + ((bb * a.ndir + dl) * 3 * a.d + gate * a.d + ch_off) * ESZ;
        in_stride = (uint32_t)(a.B * a.ndir * 3 * a.d * ESZ);
    } else {                                         // the x row
        in_ptr = (const char *)a.x + (bb * a.d + ch_off) * ESZ;
        in_stride = (uint32_t)(a.B * a.d * ESZ);
    }
    // packet p holds direction-steps p*SPP .. p*SPP + SPP - 1; this lane's
    // time index is tin(p) + e_in (direction 0) or tin(p) + SPP-1 - e_in
    if (dl) in_ptr += (int64_t)(SPP - 1 - e_in) * in_stride;
    else in_ptr += (int64_t)e_in * in_stride;
    const int64_t Pmax = L / SPP - 1;                // last packet fully inside
    auto load_packet = [&](int64_t p) -> uint4 {
        p = p < 0 ? 0 : (p < Pmax ? p : Pmax);       // clamp: stays in bounds
        const uint32_t t = (uint32_t)(dl ? (L - SPP - p * SPP) : p * SPP);
        return *(const uint4 *)(in_ptr + __umul24(t, in_stride));
    };

    // ---- outputs (c_seq for wave 0, h for wave 1): four steps per store ----
    const int e_out = lane >> 4;                     // step in the quad
    const int sub_out = lane & 15;                   // 4 channels
    float *out_t = role == 0 ? a.c_seq : a.h;
    const bool out_on = (out_t != nullptr);
    const uint32_t out_stride = (uint32_t)(a.B * a.ndir * a.d * 4);
    char *out_ptr = out_on ? (char *)(out_t + (bb * a.ndir + dl) * a.d + j0 + 4 * sub_out)
                           : nullptr;

    const float vs = a.v[(dl * 2 + role) * a.d + j] * kNegLog2e;   // v_f | v_r
    const float bs = a.b[(dl * 2 + role) * a.d + j] * kNegLog2e;
    const float alpha = a.alpha;
    const float c0 = a.c0 ? a.c0[(dl * a.B + bb) * a.d + j] : 0.0f;
    float c = c0;                                    // wave 0: the state
    float cprev = c0;                                // wave 1: c[t-1]

    auto store_outputs = [&](int64_t st0) {          // S staged steps from st0
        if (!out_on) return;
#pragma unroll
        for (int m = 0; m < S / 4; ++m) {
            const float4 val = *(const float4 *)(ostage + (m * 4 + e_out) * kWave + 4 * sub_out);
            const uint32_t t = (uint32_t)tix(st0 + m * 4 + e_out);
            *(float4 *)(out_ptr + __umul24(t, out_stride)) = val;
        }
    };

    // The ring's packet clamp needs a whole packet inside the sequence, which
    // a whole group guarantees; shorter sequences run in the tail alone.
    const int64_t groups = L / S;
    if (groups > 0) {
        uint4 ring[R];
        // slot sequence: group g - role sits in ring slot (g % NRG)
#pragma unroll
        for (int u = 0; u < NRG; ++u)
#pragma unroll
            for (int i = 0; i < G; ++i) ring[u * G + i] = load_packet((u - role) * G + i);
        const float *inf = (const float *)slot;
        const bf16_bits *inh = (const bf16_bits *)slot;
        for (int64_t g0 = 0;; g0 += NRG) {
            bool done = false;
#pragma unroll
            for (int u = 0; u < NRG; ++u) {
                const int64_t g = g0 + u;
                if (done) break;
                const int64_t mine = g - role;       // the group this wave works on
                const bool work = mine >= 0 && mine < groups;
#pragma unroll
                for (int i = 0; i < G; ++i) slot[i * kWave + lane] = ring[u * G + i];
#pragma unroll
                for (int i = 0; i < G; ++i) ring[u * G + i] = load_packet((mine + NRG) * G + i);
                if (work) {
                    float u0[S], u1[S];
#pragma unroll
                    for (int st = 0; st < S; ++st) {
                        const int pk = st / SPP, e = st % SPP;
                        if (BF16) {
                            u0[st] = bf16_to_f32(inh[pk * 512 + e * 64 + lane]);
                            u1[st] = bf16_to_f32(inh[pk * 512 + 256 + e * 64 + lane]);
                        } else {
                            u0[st] = inf[pk * 256 + e * 64 + lane];
                            u1[st] = inf[pk * 256 + 128 + e * 64 + lane];
                        }
                    }
                    float *cr = cring[mine & 1];
                    if (role == 0) {
#pragma unroll
                        for (int st = 0; st < S; ++st) {
                            c = gate_blend(fmaf(vs, c, fmaf(u0[st], kNegLog2e, bs)), c, u1[st]);
                            cr[st * kWave + lane] = c;
                            ostage[st * kWave + lane] = c;
                        }
                    } else {
#pragma unroll
                        for (int st = 0; st < S; ++st) {
                            const float ct = cr[st * kWave + lane];
                            ostage[st * kWave + lane] = gate_blend(
                                fmaf(vs, cprev, fmaf(u0[st], kNegLog2e, bs)), ct, alpha * u1[st]);
                            cprev = ct;
                        }
                    }
                    store_outputs(mine * S);
                }
                __syncthreads();                     // hand the ring half over
                done = g >= groups;                  // wave 1 has done the last group
            }
            if (done) break;
        }
    }
    // remaining L mod S steps: direct per-lane loads, state wave first
    const int64_t st_tail = groups * S;
    float *cr = cring[0];
    if (role == 0) {
        for (int64_t st = st_tail; st < L; ++st) {
            const int64_t t = tix(st);
            const int64_t ub = ((t * a.B + bb) * a.ndir + dl) * 3 * a.d + j;
            float uf, ux;
            if (BF16) {
                const bf16_bits *U = (const bf16_bits *)a.U;
                uf = bf16_to_f32(U[ub]);
                ux = bf16_to_f32(U[ub + 2 * a.d]);
            } else {
                const float *U = (const float *)a.U;
                uf = U[ub];
                ux = U[ub + 2 * a.d];
            }
            c = gate_blend(fmaf(vs, c, fmaf(uf, kNegLog2e, bs)), c, ux);
            cr[(st - st_tail) * kWave + lane] = c;
            if (a.c_seq) a.c_seq[((t * a.B + bb) * a.ndir + dl) * a.d + j] = c;
        }
        if (a.c_last) a.c_last[(dl * a.B + bb) * a.d + j] = c;
    }
    __syncthreads();
    if (role == 1) {
        for (int64_t st = st_tail; st < L; ++st) {
            const int64_t t = tix(st);
            const int64_t ub = ((t * a.B + bb) * a.ndir + dl) * 3 * a.d + j;
            float ur, xv;
            if (BF16) {
                ur = bf16_to_f32(((const bf16_bits *)a.U)[ub + a.d]);
                xv = bf16_to_f32(((const bf16_bits *)a.x)[(t * a.B + bb) * a.d + j]);
            } else {
                ur = ((const float *)a.U)[ub + a.d];
                xv = ((const float *)a.x)[(t * a.B + bb) * a.d + j];
            }
            const float ct = cr[(st - st_tail) * kWave + lane];
            a.h[((t * a.B + bb) * a.ndir + dl) * a.d + j] =
                gate_blend(fmaf(vs, cprev, fmaf(ur, kNegLog2e, bs)), ct, alpha * xv);
            cprev = ct;
        }
    }
}

// ---------------------------------------------------------------------------
// Generic backward (one direction per launch): one thread per chain.
// ---------------------------------------------------------------------------
template <typename TU, typename TX>
__global__ __launch_bounds__(256) void bwd_generic(RecArgs a)
{
    const int64_t chains = a.B * a.d;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g == 0 && a.err_word) *a.err_word = 0u;   // no look-back here: no error
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
        if (a.dU_lp) {
            a.dU_lp[ub] = f32_to_bf16(dzf);
            a.dU_lp[ub + a.d] = f32_to_bf16(dzr);
            a.dU_lp[ub + 2 * a.d] = f32_to_bf16(dux);
        }
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
// Fast backward (fp32 U and x, d % 64 == 0, same size limits as the fast
// forward): one wavefront per 64 channels, walking its direction's steps in
// reverse.  Per timestep two input packets:
//   A: lanes 0-15 U_f, 16-31 U_r, 32-47 U_cand, 48-63 x          (time t)
//   B: lanes 0-15 c[t_prev], 16-31 dh[t], 32-47 dx[t] (read when
//      accumulating; otherwise these lanes and lanes 48-63 re-read dh)
// and one output packet: lanes 0-15 dU_f, 16-31 dU_r, 32-47 dU_cand, 48-63 dx
// (plus, optionally, the three dU rows rounded to bf16).  Steps are processed
// in groups of G with one LDS round trip per group, a branch-free main loop
// over whole groups and a direct-load tail, as in the forward kernel.
// ---------------------------------------------------------------------------
//
// BIDI: both directions of one (batch row, 64 channels) in one workgroup of
// two waves (wave w walks direction w).  The highway dx contributions of all
// L steps go into one LDS row per step, started at -0.0, to which each wave
// adds its term with an LDS float atomic (round to nearest even, denormals
// kept); at the end the workgroup writes the rows to dx once, so the two
// directions need no ordering between launches and dx is never re-read.
// -0.0 + a is a exactly, and fp32 addition of two terms is commutative, so
// the row ends as (direction 0) + (direction 1) whichever wave adds first:
// the sum the one-direction-per-launch path produces.  LDS: L * 64 floats,
// passed as dynamic shared memory.
template <int R, int G, bool BIDI>
__global__ __launch_bounds__(BIDI ? 2 * kWave : kWave) void bwd_fast(RecArgs a)
{
    static_assert(R % G == 0, "ring holds whole groups");
    constexpr int NW = BIDI ? 2 : 1;
    __shared__ uint4 slot_a_all[NW][G * kWave];
    __shared__ uint4 slot_b_all[NW][G * kWave];
    __shared__ float out_slot_all[NW][G * 4 * kWave];
    extern __shared__ float dxbuf[];                 // BIDI: [L][64]

    const int wv = BIDI ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
    const int lane = threadIdx.x & 63;
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.err_word)
        *a.err_word = 0u;                            // no look-back here: no error
    uint4 *slot_a = slot_a_all[wv];
    uint4 *slot_b = slot_b_all[wv];
    float *out_slot = out_slot_all[wv];
    const int dl = BIDI ? wv : a.dir;
    const int64_t gpr = a.d / kWave;
    const int64_t w = blockIdx.x;
    const int64_t bb = w / gpr;
    const int64_t j0 = (w % gpr) * kWave;
    const int64_t j = j0 + lane;
    const int64_t L = a.L;
    auto tix = [&](int64_t s) -> int64_t { return dl ? (L - 1 - s) : s; };

    const int q = lane >> 4;
    const int sub = lane & 15;
    const bool dxacc = !BIDI && a.dx_accumulate;
    const uint32_t u_stride = (uint32_t)(a.B * a.ndir * 3 * a.d * 4);
    const uint32_t x_stride = (uint32_t)(a.B * a.d * 4);
    const uint32_t h_stride = (uint32_t)(a.B * a.ndir * a.d * 4);
    const int64_t u_row = (bb * a.ndir + dl) * 3 * a.d + q * a.d + j0 + 4 * sub;
    const int64_t x_row = bb * a.d + j0 + 4 * sub;
    const int64_t h_row = (bb * a.ndir + dl) * a.d + j0 + 4 * sub;
    // packet A
    const char *pa_ptr = q < 3 ? (const char *)a.U + u_row * 4 : (const char *)a.x + x_row * 4;
    const uint32_t pa_stride = q < 3 ? u_stride : x_stride;
    // packet B
    const bool b_is_dx = (q == 2 && dxacc);
    const char *pb_ptr = q == 0   ? (const char *)a.c_seq_in + h_row * 4
                         : b_is_dx ? (const char *)a.dx + x_row * 4
                                   : (const char *)a.dh + h_row * 4;
    const uint32_t pb_stride = b_is_dx ? x_stride : h_stride;
    const bool pb_prev = (q == 0);                   // c at the previous direction-step
    // output packet
    char *po_ptr = q < 3 ? (char *)a.dU + u_row * 4 : (char *)a.dx + x_row * 4;
    const uint32_t po_stride = pa_stride;
    const bool lp_on = a.dU_lp != nullptr && q < 3;
    char *lp_ptr = lp_on ? (char *)a.dU_lp + u_row * 2 : nullptr;
    const uint32_t lp_stride = u_stride / 2;

    // time index of reverse iteration k (direction-step L-1-k), clamped
    auto t_of = [&](int64_t k) -> uint32_t {
        const int64_t kk = k < L ? k : L - 1;
        return (uint32_t)(dl ? kk : L - 1 - kk);
    };
    auto tprev_of = [&](int64_t k) -> uint32_t {    // direction-step L-2-k, clamped
        const int64_t kk = k < L - 1 ? k : L - 2;
        if (kk < 0) return 0u;                       // L == 1: never used
        return (uint32_t)(dl ? kk + 1 : L - 2 - kk);
    };
    auto load_a = [&](int64_t k) -> uint4 {
        return *(const uint4 *)(pa_ptr + __umul24(t_of(k), pa_stride));
    };
    auto load_b = [&](int64_t k) -> uint4 {
        const uint32_t t = pb_prev ? tprev_of(k) : t_of(k);
        return *(const uint4 *)(pb_ptr + __umul24(t, pb_stride));
    };

    const float vf = a.v[(dl * 2 + 0) * a.d + j], vr = a.v[(dl * 2 + 1) * a.d + j];
    const float vfs = vf * kNegLog2e, vrs = vr * kNegLog2e;
    const float bfs = a.b[(dl * 2 + 0) * a.d + j] * kNegLog2e;
    const float brs = a.b[(dl * 2 + 1) * a.d + j] * kNegLog2e;
    const float c0 = a.c0 ? a.c0[(dl * a.B + bb) * a.d + j] : 0.0f;
    const float alpha = a.alpha;
    float gc = a.dc_last ? a.dc_last[(dl * a.B + bb) * a.d + j] : 0.0f;
    float c = a.c_seq_in[((tix(L - 1) * a.B + bb) * a.ndir + dl) * a.d + j];
    float svf = 0.f, svr = 0.f, sbf = 0.f, sbr = 0.f;
    // adds one direction's highway dx term to row t of the shared rows
    auto dx_add = [&](uint32_t t, float v) {
        __hip_atomic_fetch_add(dxbuf + t * kWave + lane, v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    if constexpr (BIDI) {
        for (int64_t idx = threadIdx.x; idx < L * 16; idx += 2 * kWave)
            *(float4 *)(dxbuf + 4 * idx) = make_float4(-0.0f, -0.0f, -0.0f, -0.0f);
        __syncthreads();
    }

    // one reverse step; returns dU_f, dU_r, dU_cand, dx (highway part)
    auto cell = [&](float uf, float ur, float ux, float xv, float cp, float dhv, float &o0,
                    float &o1, float &o2, float &o3) {
        const Gate f = gate_scaled(fmaf(vfs, cp, fmaf(uf, kNegLog2e, bfs)));
        const Gate r = gate_scaled(fmaf(vrs, cp, fmaf(ur, kNegLog2e, brs)));
        const float dc = fmaf(dhv, r.g, gc);
        const float dr = dhv * fmaf(-alpha, xv, c);
        o3 = dhv * r.gc * alpha;
        o2 = dc * f.gc;
        const float df = dc * (cp - ux);
        o0 = df * (f.g * f.gc);
        o1 = dr * (r.g * r.gc);
        svf = fmaf(o0, cp, svf);
        svr = fmaf(o1, cp, svr);
        sbf += o0;
        sbr += o1;
        gc = fmaf(dc, f.g, fmaf(o0, vf, o1 * vr));
        c = cp;
    };

    const int64_t groups = L / G;
    if (groups > 0) {
        uint4 ring_a[R], ring_b[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            ring_a[i] = load_a(i);
            ring_b[i] = load_b(i);
        }
        const float *fa = (const float *)slot_a;
        const float *fb = (const float *)slot_b;
        int64_t gi = 0;
        for (;;) {
#pragma unroll
            for (int rg = 0; rg < R / G; ++rg) {
                const int64_t k0 = (gi + rg) * G;
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    slot_a[i * kWave + lane] = ring_a[rg * G + i];
                    slot_b[i * kWave + lane] = ring_b[rg * G + i];
                }
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    ring_a[rg * G + i] = load_a(k0 + R + i);
                    ring_b[rg * G + i] = load_b(k0 + R + i);
                }
                float uf[G], ur[G], ux[G], xv[G], cp[G], dhv[G], dxi[G];
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    uf[i] = fa[i * 256 + lane];
                    ur[i] = fa[i * 256 + 64 + lane];
                    ux[i] = fa[i * 256 + 128 + lane];
                    xv[i] = fa[i * 256 + 192 + lane];
                    cp[i] = fb[i * 256 + lane];
                    dhv[i] = fb[i * 256 + 64 + lane];
                    dxi[i] = fb[i * 256 + 128 + lane];
                }
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const int64_t s = L - 1 - (k0 + i);
                    float o0, o1, o2, o3;
                    cell(uf[i], ur[i], ux[i], xv[i], s > 0 ? cp[i] : c0, dhv[i], o0, o1, o2, o3);
                    if (BIDI) dx_add(t_of(k0 + i), o3);
                    out_slot[i * 256 + lane] = o0;
                    out_slot[i * 256 + 64 + lane] = o1;
                    out_slot[i * 256 + 128 + lane] = o2;
                    out_slot[i * 256 + 192 + lane] = dxacc ? o3 + dxi[i] : o3;
                }
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const float4 val = ((const float4 *)out_slot)[i * 64 + lane];
                    const uint32_t t = t_of(k0 + i);
                    if (!BIDI || q < 3)   // BIDI: dx went to the LDS rows
                        *(float4 *)(po_ptr + __umul24(t, po_stride)) = val;
                    if (lp_on) {     // lanes of the three dU rows also write bf16
                        uint2 pk;
                        pk.x = pack_bf16x2(val.x, val.y);
                        pk.y = pack_bf16x2(val.z, val.w);
                        *(uint2 *)(lp_ptr + __umul24(t, lp_stride)) = pk;
                    }
                }
                if (gi + rg + 1 >= groups) goto tail;
            }
            gi += R / G;
        }
    }
tail:
    for (int64_t k = groups * G; k < L; ++k) {
        const int64_t s = L - 1 - k;
        const int64_t t = tix(s);
        const int64_t ub = ((t * a.B + bb) * a.ndir + dl) * 3 * a.d + j;
        const float *U = (const float *)a.U;
        const int64_t xi = (t * a.B + bb) * a.d + j;
        const float cpv =
            s > 0 ? a.c_seq_in[((tix(s - 1) * a.B + bb) * a.ndir + dl) * a.d + j] : c0;
        float o0, o1, o2, o3;
        cell(U[ub], U[ub + a.d], U[ub + 2 * a.d], ((const float *)a.x)[xi], cpv,
             a.dh[((t * a.B + bb) * a.ndir + dl) * a.d + j], o0, o1, o2, o3);
        a.dU[ub] = o0;
        a.dU[ub + a.d] = o1;
        a.dU[ub + 2 * a.d] = o2;
        if (a.dU_lp) {
            a.dU_lp[ub] = f32_to_bf16(o0);
            a.dU_lp[ub + a.d] = f32_to_bf16(o1);
            a.dU_lp[ub + 2 * a.d] = f32_to_bf16(o2);
        }
        if (BIDI)
            dx_add((uint32_t)t, o3);
        else
            a.dx[xi] = dxacc ? o3 + a.dx[xi] : o3;
    }
    if (a.dc0) a.dc0[(dl * a.B + bb) * a.d + j] = gc;
    float *pp = a.partials + ((int64_t)(dl * a.B + bb) * 4) * a.d + j;
    pp[0 * a.d] = svf;
    pp[1 * a.d] = svr;
    pp[2 * a.d] = sbf;
    pp[3 * a.d] = sbr;
    if constexpr (BIDI) {
        // dx[t, bb, j0 .. j0 + 63] = direction 0 + direction 1, 16-byte stores
        __syncthreads();
        for (int64_t idx = threadIdx.x; idx < L * 16; idx += 2 * kWave) {
            const int64_t t = idx >> 4;
            const int c = (int)(idx & 15) * 4;
            *(float4 *)(a.dx + (t * a.B + bb) * a.d + j0 + c) =
                *(const float4 *)(dxbuf + t * kWave + c);
        }
    }
}

// dv[dl, g, j] = sum_b partials[dl, b, g, j]; db[dl, g, j] likewise with rows
// 2, 3.  A block of 16 waves owns 64 consecutive j of one (dl, g): wave w sums
// the b of residue w (mod 16) in increasing order, sixteen (then eight) loads
// in flight at a time, then the 16 partial sums are added in wave order.  The
// summation order depends only on B, so results are identical run to run.
constexpr int kReduceWaves = 16;

__global__ __launch_bounds__(64 * kReduceWaves) void param_reduce(const float *__restrict__ part,
                                                                 int64_t B, int64_t d, float *dv,
                                                                 float *db)
{
    constexpr int NWv = kReduceWaves;
    __shared__ float red[NWv][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t jblocks = (d + 63) / 64;
    const int64_t row = blockIdx.x / jblocks;           // dl * 4 + g
    const int64_t j = (blockIdx.x % jblocks) * 64 + lane;
    const int g = (int)(row % 4), dl = (int)(row / 4);
    float s = 0.0f;
    if (j < d) {
        const float *p = part + ((int64_t)dl * B * 4 + g) * d + j;
        const int64_t stride = 4 * d;                   // next b
        int64_t bb = wv;
        // U rows of this wave's residue per batch of loads, added in order
        auto batch = [&](auto u_const) {
            constexpr int U = decltype(u_const)::value;
            for (; bb + (U - 1) * NWv < B; bb += U * NWv) {
                float v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = p[(bb + u * NWv) * stride];
#pragma unroll
                for (int u = 0; u < U; ++u) s += v[u];
            }
        };
        batch(std::integral_constant<int, 16>());
        batch(std::integral_constant<int, 8>());
        for (; bb < B; bb += NWv) s += p[bb * stride];
    }
    red[wv][lane] = s;
    __syncthreads();
    if (wv == 0 && j < d) {
        float t = red[0][lane];
#pragma unroll
        for (int w = 1; w < NWv; ++w) t += red[w][lane];
        if (g < 2) {
            if (dv) dv[(dl * 2 + g) * d + j] = t;
        } else {
            if (db) db[(dl * 2 + (g - 2)) * d + j] = t;
        }
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

#ifndef SRU_FWD_RING_F32
#define SRU_FWD_RING_F32 16
#endif
#ifndef SRU_FWD_GROUP_F32
#define SRU_FWD_GROUP_F32 8
#endif
#ifndef SRU_FWD_RING_BF16
#define SRU_FWD_RING_BF16 32
#endif
#ifndef SRU_FWD_GROUP_BF16
#define SRU_FWD_GROUP_BF16 8
#endif
#ifndef SRU_FWD_SPLIT
#define SRU_FWD_SPLIT 1
#endif
// fwd_split rings: bf16 inputs keep two groups of 8 packets (measured at
// L = 1024, B = 16, d = 2048: 88 us against 91-97 us for 8-24 packets in
// groups of 4 and 24-32 in groups of 8); fp32 two groups of 4.
#ifndef SRU_SPLIT_RING_F32
#define SRU_SPLIT_RING_F32 8
#endif
#ifndef SRU_SPLIT_RING_BF16
#define SRU_SPLIT_RING_BF16 16
#endif
#ifndef SRU_SPLIT_GROUP_F32
#define SRU_SPLIT_GROUP_F32 4
#endif
#ifndef SRU_SPLIT_GROUP_BF16
#define SRU_SPLIT_GROUP_BF16 8
#endif
// below this many 64-channel waves (the SIMD count) the forward splits each
// block's work over two waves
constexpr int64_t kSplitBelowWaves = 1024;
#ifndef SRU_BWD_RING
#define SRU_BWD_RING 8
#endif
#ifndef SRU_BWD_GROUP
#define SRU_BWD_GROUP 4
#endif

// Longest sequence whose dx rows (L * 256 bytes) the two-direction backward
// keeps in LDS.
constexpr int64_t kBidiMaxL = 64;

// The fast kernels address with 32-bit byte offsets built from 24-bit
// products: every tensor below 2 GiB and every time stride below 16 MiB.
static bool fast_sizes_ok(const RecArgs &a)
{
    const int64_t esz = a.u_bf16 ? 2 : 4;
    const int64_t u_bytes = a.L * a.B * a.ndir * 3 * a.d * 4;   // fp32 bound covers bf16
    const int64_t ustride = a.B * a.ndir * 3 * a.d * esz;
    return u_bytes < (int64_t(1) << 31) && ustride < (int64_t(1) << 24) && a.L < (int64_t(1) << 24);
}

hipError_t launch_forward(const RecArgs &a, hipStream_t s)
{
    const bool fast = (a.d % kWave == 0) && (a.u_bf16 == a.x_bf16) && fast_sizes_ok(a);
    if (fast) {
        const int64_t waves = (int64_t)a.ndir * a.B * (a.d / kWave);
        if (SRU_FWD_SPLIT && waves < kSplitBelowWaves) {   // fewer waves than SIMDs
            if (a.u_bf16)
                hipLaunchKernelGGL((fwd_split<true, SRU_SPLIT_RING_BF16, SRU_SPLIT_GROUP_BF16>),
                                   dim3((unsigned)waves), dim3(2 * kWave), 0, s, a);
            else
                hipLaunchKernelGGL((fwd_split<false, SRU_SPLIT_RING_F32, SRU_SPLIT_GROUP_F32>),
                                   dim3((unsigned)waves), dim3(2 * kWave), 0, s, a);
            return hipGetLastError();
        }
        if (a.u_bf16)
            hipLaunchKernelGGL((fwd_fast<true, SRU_FWD_RING_BF16, SRU_FWD_GROUP_BF16>),
                               dim3((unsigned)waves), dim3(kWave), 0, s, a);
        else
            hipLaunchKernelGGL((fwd_fast<false, SRU_FWD_RING_F32, SRU_FWD_GROUP_F32>),
                               dim3((unsigned)waves), dim3(kWave), 0, s, a);
        return hipGetLastError();
    }
    if (a.u_bf16) {
        return a.x_bf16 ? fwd_generic_launch<bf16_bits, bf16_bits>(a, s)
                        : fwd_generic_launch<bf16_bits, float>(a, s);
    }
    return a.x_bf16 ? fwd_generic_launch<float, bf16_bits>(a, s)
                    : fwd_generic_launch<float, float>(a, s);
}

bool backward_bidi_ok(const RecArgs &a)
{
    return a.ndir == 2 && a.L <= kBidiMaxL && (a.d % kWave == 0) && !a.u_bf16 && !a.x_bf16 &&
           fast_sizes_ok(a);
}

hipError_t launch_backward_bidi(const RecArgs &a, hipStream_t s)
{
    const int64_t blocks = a.B * (a.d / kWave);
    const size_t lds = (size_t)a.L * kWave * sizeof(float);
    hipLaunchKernelGGL((bwd_fast<SRU_BWD_RING, SRU_BWD_GROUP, true>), dim3((unsigned)blocks),
                       dim3(2 * kWave), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_backward_dir(const RecArgs &a, hipStream_t s)
{
    const bool fast = (a.d % kWave == 0) && !a.u_bf16 && !a.x_bf16 && fast_sizes_ok(a);
    if (fast) {
        const int64_t waves = a.B * (a.d / kWave);
        hipLaunchKernelGGL((bwd_fast<SRU_BWD_RING, SRU_BWD_GROUP, false>), dim3((unsigned)waves),
                           dim3(kWave), 0, s, a);
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
    const int64_t blocks = (int64_t)ndir * 4 * ((d + 63) / 64);
    hipLaunchKernelGGL(param_reduce, dim3((unsigned)blocks), dim3(64 * kReduceWaves), 0, s,
                       partials, B, d, dv, db);
    return hipGetLastError();
}

}  // namespace sru
