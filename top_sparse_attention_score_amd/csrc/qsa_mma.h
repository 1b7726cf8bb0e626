// qsa_mma.h -- helpers shared by the matrix-core attention kernels (gfx950,
// v_mfma_f32_16x16x32_f16 operand preparation, DPP row reductions).
#pragma once

#include "qsa_device.h"

namespace qsa {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef int int2v_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) int2v_t lds_int2v_t;

constexpr int kMmaCells = 32;     // cells per tile
constexpr float kWScale = 16.f;   // weights are carried at 2^4 times their value
constexpr float kLazyMax = 2.7f;  // reference max slack (natural log units, < ln 16)

__device__ __forceinline__ float4_t mfma16(half8_t a, half8_t b, float4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Eight int8 codes (bytes of w0 then w1) as exact fp16 values.
__device__ __forceinline__ half8_t codes_to_half8(uint32_t w0, uint32_t w1)
{
    const half2_t a = int8_pair_to_half2((int)w0, 0), b = int8_pair_to_half2((int)w0, 1);
    const half2_t c = int8_pair_to_half2((int)w1, 0), d = int8_pair_to_half2((int)w1, 1);
    const half4_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const half4_t cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// fp16 half `hi` (0 = low, 1 = high) of a packed word, as float.
__device__ __forceinline__ float half_of(uint32_t w, int hi)
{
    return half_bits_to_float((uint16_t)(hi ? (w >> 16) : (w & 0xffffu)));
}

// a * (fp16 half HI of w) in one mixed-precision FMA: the fp16 operand is
// widened exactly and the product rounded once to fp32.
template <int HI>
__device__ __forceinline__ float mul_by_half(float a, uint32_t w)
{
    float r;
    if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
            : "=v"(r) : "v"(a), "v"(w));
    else
        asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,0,0] op_sel_hi:[0,1,0]"
            : "=v"(r) : "v"(a), "v"(w));
    return r;
}

// Splits eight fp32 values into fp16 hi (round toward zero) and lo = x - hi
// (exact in fp32, then rounded toward zero to fp16).
__device__ __forceinline__ void split8(const float* x, half8_t& hi, half8_t& lo)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto h = __builtin_amdgcn_cvt_pkrtz(x[2 * i], x[2 * i + 1]);
        const auto l = __builtin_amdgcn_cvt_pkrtz(x[2 * i] - (float)h[0], x[2 * i + 1] - (float)h[1]);
        hi[2 * i] = (_Float16)h[0];
        hi[2 * i + 1] = (_Float16)h[1];
        lo[2 * i] = (_Float16)l[0];
        lo[2 * i + 1] = (_Float16)l[1];
    }
}

// Max / sum over the 16 lanes of a DPP row (rotations by 8, 4, 2, 1: every
// lane ends with the row's result).
__device__ __forceinline__ float row16_max(float v)
{
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false)));
    return v;
}

__device__ __forceinline__ float row16_sum(float v)
{
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));
    return v;
}

// The query operand of block blk for this lane: head hq (zero beyond G),
// elements 32*blk + 8*q4 .. +7, as fp16 hi and lo halves.
template <int G, int D, bool QF16>
__device__ __forceinline__ void load_q_block(const void* q, size_t prow, int hq, int q4, int blk,
                                             half8_t& hi, half8_t& lo)
{
    const bool hv = hq < G;
    const size_t off = (prow + (hv ? hq : 0)) * D + 32 * blk + 8 * q4;
    if constexpr (QF16) {
        const half8_t v = *(const half8_t*)((const _Float16*)q + off);
        hi = hv ? v : half8_t{};
        lo = half8_t{};
    } else {
        const float4* qr = (const float4*)((const float*)q + off);
        const float4 a = qr[0], b = qr[1];
        const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const _Float16 h = (_Float16)x[e];
            const _Float16 l = (_Float16)(x[e] - (float)h);
            hi[e] = hv ? h : (_Float16)0.f;
            lo[e] = hv ? l : (_Float16)0.f;
        }
    }
}

}  // namespace qsa
