// device_common.h -- small device helpers shared by the libsru kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sru {

typedef uint16_t bf16_bits;

// bf16 -> fp32 is exact: the bf16 pattern is the upper half of the fp32 one.
__device__ __forceinline__ float bf16_to_f32(bf16_bits h)
{
    return __uint_as_float(uint32_t(h) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_bits f32_to_bf16(float f)
{
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(bf16_bits, b);
}

// Two fp32 values -> two bf16 (nearest even) in one dword, low half first
// (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <typename T> __device__ __forceinline__ float load_as_f32(const T *p);
template <> __device__ __forceinline__ float load_as_f32<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float load_as_f32<bf16_bits>(const bf16_bits *p)
{
    return bf16_to_f32(*p);
}

// A gate and its complement: g = sigma(z) = 1 / (1 + e^-z) and
// gc = 1 - g = sigma(-z) = e^-z g, both to a few ulp, using the hardware
// base-2 exponential and reciprocal (v_exp_f32, v_rcp_f32).  The complement
// is never formed as 1 - g: with g close to 1 (e.g. forget gates at
// sigma(8) = 0.9997) the subtraction would keep only ~11 significant bits.
//
// gate_scaled takes y = -z log2(e) (callers fold -log2(e) into their
// parameters once).  y is capped at 64 so that 2^y g stays finite: for very
// negative z, g = 2^-64 and gc = 1.  The cap is the IEEE 754-2019 minimum
// (one v_minimum3_f32), which returns NaN for a NaN operand, so a NaN
// pre-activation gives a NaN gate, as sigma(NaN) does, rather than a closed
// one (fminf would return the cap).
struct Gate {
    float g, gc;
};

constexpr float kNegLog2e = -1.4426950408889634f;

__device__ __forceinline__ float cap_exponent(float y)
{
    return __builtin_elementwise_minimum(y, 64.0f);
}

__device__ __forceinline__ Gate gate_scaled(float y)
{
    const float e = __builtin_amdgcn_exp2f(cap_exponent(y));
    const float g = __builtin_amdgcn_rcpf(1.0f + e);
    return {g, e * g};
}

__device__ __forceinline__ Gate gate(float z) { return gate_scaled(z * kNegLog2e); }

// The gate's blend g p + (1 - g) q for y = -z log2(e), evaluated as
// g (p + e q) with e = 2^y and g = 1 / (1 + e): the complement is carried by
// e (never 1 - g), and the fma runs beside 1 + e and the reciprocal, so a
// recurrence through p waits on exp, add, rcp and one multiply.  The cap on
// y is that of gate_scaled; e q stays finite for |q| < 2^64.
__device__ __forceinline__ float gate_blend(float y, float p, float q)
{
    const float e = __builtin_amdgcn_exp2f(cap_exponent(y));
    const float g = __builtin_amdgcn_rcpf(1.0f + e);
    return g * fmaf(e, q, p);
}

// ---- memory-to-LDS copies (global_load_lds_dwordx4) ----------------------

// Wait until at most N_ of this wave's vector memory requests are in flight
// (the copies below count as such requests until their data is in LDS).
template <int N_> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N_ >= 0 && N_ < 64, "vmcnt is 6 bits");
    // vmcnt[3:0] | expcnt[6:4] = 7 | lgkmcnt[11:8] = 15 | vmcnt[5:4] at [15:14]
    __builtin_amdgcn_s_waitcnt((N_ & 15) | (7 << 4) | (15 << 8) | ((N_ >> 4) << 14));
}

// Wait for every LDS access of this wave.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// 16 bytes per lane from gptr into LDS at lds_base + 16 * lane (lds_base is
// wave-uniform; M0 carries it).  The instruction has no register result; the
// caller accounts for its completion with wait_vmcnt.
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(gptr)
                 : "memory");
}

// The same with the address split into a wave-uniform base (SGPR pair) and a
// per-lane unsigned 32-bit byte offset: no 64-bit address arithmetic per lane.
// The base must be wave-uniform; it is read from the first lane so that it
// can live in scalar registers.
__device__ __forceinline__ void dma16s(const void *sbase, uint32_t voff, uint32_t lds_base)
{
    // (readfirstlane returns int: each half goes through uint32_t, so the low
    // half is zero-extended, never sign-extended into the high half)
    const uint64_t p = (uint64_t)(uintptr_t)sbase;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"((const void *)(uintptr_t)u)
                 : "memory");
}

}  // namespace sru
