// qsa_device.h -- device helpers shared by the QSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Order-preserving map from an fp32 score to an unsigned key: a larger score
// gives a larger key.  -0 is folded onto +0 so the two compare equal (equal
// scores are then ranked by cell index).  Every finite score maps to a key
// >= 0x00800000, so 0 never names a real score.
__device__ __forceinline__ uint32_t score_key(float s)
{
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return (float)v;
}

__device__ __forceinline__ half2_t as_half2(uint32_t u)
{
    half2_t v;
    __builtin_memcpy(&v, &u, 4);
    return v;
}

// Sign-extended byte e (0..3) of a packed word, as float (one SDWA convert).
__device__ __forceinline__ float sbyte_to_float(int w, int e)
{
    return (float)(int8_t)(w >> (8 * e));
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace qsa
