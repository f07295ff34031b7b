// scan_common.h -- device helpers shared by the single-pass chunked scans
// (linear mode, and the nonlinear backward evaluated as a linear scan of its
// adjoint): the look-back between chunks, per-segment row addressing, and a
// clearing kernel.
#pragma once
#include "device_common.h"

namespace sru {
namespace {

// A chunk's outgoing state is published as one 64-bit word per (chunk,
// chain): the float's bits in the low half and a ready mark in the high
// half, written and read with single relaxed device-scope atomics.  Value
// and mark travel together, so no fence (and none of the L2 write-back /
// invalidate a device-scope fence costs) is needed.  Chunks take dynamic
// tickets in order, so a chunk only ever waits for a chunk that started
// before it and progress is guaranteed.  The wait is bounded; if the bound is
// ever hit the kernel stops waiting and raises the error word.
struct Lookback {
    uint64_t *carry;     // [nC, chains]  published outgoing state of each chunk
    uint32_t *ticket;    // dynamic chunk ticket
    uint32_t *err;       // set if a wait ran out
};

constexpr uint32_t kSpinLimit = 1u << 22;
constexpr uint64_t kReady = uint64_t(1) << 32;

__device__ __forceinline__ void publish(Lookback lb, int64_t idx, float v)
{
    __hip_atomic_store(lb.carry + idx, kReady | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float consume(Lookback lb, int64_t idx, int lane)
{
    uint64_t w = __hip_atomic_load(lb.carry + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    while (!__all((w & kReady) != 0)) {
        if (++spins > kSpinLimit) {
            if (lane == 0)
                __hip_atomic_store(lb.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
        w = __hip_atomic_load(lb.carry + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return __uint_as_float((uint32_t)w);
}

__device__ __forceinline__ int64_t take_ticket(Lookback lb, uint32_t *s_ticket)
{
    if (threadIdx.x == 0) *s_ticket = atomicAdd(lb.ticket, 1u);
    __syncthreads();
    // the same value in every lane: keep it (and every index derived from
    // it) in scalar registers
    return (int64_t)__builtin_amdgcn_readfirstlane(*s_ticket);
}

// Rows of one wave's segment.  Step i of the segment (i = 0..SEG-1, in the
// direction's own order) lives at time t0 + row(i); steps past the end of
// the sequence are clamped onto the segment's last valid step, so every
// load stays in bounds.  t0 is the segment's lowest time index, so every
// row offset is a small non-negative number: with one uniform 64-bit base
// per stream, an access costs a 32-bit offset instead of 64-bit address
// arithmetic per step.
struct SegRows {
    int64_t t0;   // lowest time index the segment touches
    int nv1;      // index of the segment's last valid step (-1: none)
    bool rev;     // reverse direction: time decreases along the segment

    // L: sequence length; rev: direction 1; s_lo: the segment's first
    // step in the direction's order; seg: steps per segment
    __device__ SegRows(int64_t L, bool reverse, int64_t s_lo, int seg)
    {
        const int64_t left = L - 1 - s_lo;
        nv1 = (int)(left < 0 ? -1 : (left < seg - 1 ? left : seg - 1));
        rev = reverse;
        t0 = rev ? L - 1 - (s_lo + (nv1 < 0 ? 0 : nv1)) : s_lo;
    }
    __device__ __forceinline__ uint32_t row(int i) const
    {
        const int r = i < nv1 ? i : nv1;
        return (uint32_t)(rev ? nv1 - r : r);
    }
};

template <typename T> __device__ __forceinline__ float ld_off(const char *base, uint32_t off)
{
    return load_as_f32((const T *)(base + off));
}
__device__ __forceinline__ void st_off(char *base, uint32_t off, float v)
{
    *(float *)(base + off) = v;
}
__device__ __forceinline__ float ldf_off(const char *base, uint32_t off)
{
    return *(const float *)(base + off);
}


// Clears look-back states, ticket and error word before a launch (a plain
// kernel, so the sequence can also be captured in a graph).
// Zeroes n 32-bit words at p (16-byte aligned): one 16-byte store per thread,
// the words of a last partial quad one by one.
__global__ __launch_bounds__(256) void scan_clear(uint32_t *p, int64_t n)
{
    const int64_t w = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
    if (w + 3 < n)
        *(uint4 *)(p + w) = make_uint4(0u, 0u, 0u, 0u);
    else
        for (int64_t k = w; k < n; ++k) p[k] = 0u;
}

inline unsigned scan_clear_blocks(int64_t n) { return (unsigned)(((n + 3) / 4 + 255) / 256); }

}  // namespace
}  // namespace sru
