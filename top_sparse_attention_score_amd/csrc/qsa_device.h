// qsa_device.h -- device helpers shared by the QSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

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

// Signed bytes 2*half_sel and 2*half_sel+1 of w as an exact fp16 pair:
// (b + 128) is placed in the low mantissa byte of 1024.0 (0x6400), giving
// 1024 + 128 + b exactly, and 1152 is subtracted in packed fp16.
__device__ __forceinline__ half2_t int8_pair_to_half2(int w, int half_sel)
{
    const uint32_t u = (uint32_t)w ^ 0x80808080u;
    const uint32_t sel = half_sel ? 0x04030402u : 0x04010400u;
    const uint32_t bits = __builtin_amdgcn_perm(0x64646464u, u, sel);
    return as_half2(bits) - half2_t{(_Float16)1152.0f, (_Float16)1152.0f};
}

// Orders this wave's LDS accesses: every earlier LDS access has completed and
// all lanes of the wave have reached this point.  Used where the waves of a
// workgroup never share LDS, so no workgroup barrier is needed.
__device__ __forceinline__ void wave_lds_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
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
