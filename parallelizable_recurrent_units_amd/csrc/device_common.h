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
// e^-z is capped at 2^64 so that e^-z * g stays finite (g = 2^-64, gc = 1
// for very negative z); NaN passes through.
struct Gate {
    float g, gc;
};

__device__ __forceinline__ Gate gate(float z)
{
    float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
    e = e > 0x1p64f ? 0x1p64f : e;
    const float g = __builtin_amdgcn_rcpf(1.0f + e);
    return {g, e * g};
}

}  // namespace sru
