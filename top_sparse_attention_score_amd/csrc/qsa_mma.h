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
// Query shift target: the largest |q| of an item is carried in [2^14, 2^15).
constexpr int kQShiftLo = 14;
// V-scale shift target: the largest V scale of a tile is carried in
// [2^6, 2^7), so weight (<= e^kLazyMax < 15) x kWScale x scale < 2^15 stays
// finite in fp16 and the lo half of every large term stays normal.
constexpr int kVShiftLo = 6;

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

// a * (fp16 half HI of w) - (fp16 half LO of h) in one mixed-precision FMA:
// both fp16 operands are widened exactly, the result is rounded once.
template <int HI, int LO>
__device__ __forceinline__ float fma_half_minus_half(float a, uint32_t w, uint32_t h)
{
    float r;
    if constexpr (HI && LO)
        asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[0,1,1] op_sel_hi:[0,1,1]"
            : "=v"(r) : "v"(a), "v"(w), "v"(h));
    else if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[0,1,0] op_sel_hi:[0,1,1]"
            : "=v"(r) : "v"(a), "v"(w), "v"(h));
    else if constexpr (LO)
        asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]"
            : "=v"(r) : "v"(a), "v"(w), "v"(h));
    else
        asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[0,0,0] op_sel_hi:[0,1,1]"
            : "=v"(r) : "v"(a), "v"(w), "v"(h));
    return r;
}

// The eight products x_e = a_e * s_e (s_e the fp16 half HI of w_e) as fp16
// hi + lo: hi = fp16(fp32(x_e)) rounded toward zero, lo = fp16(x_e - hi)
// rounded toward zero, with x_e - hi formed from the exact product in one
// mixed FMA.  hi + lo carries x_e to 22 significant bits.
template <int HI>
__device__ __forceinline__ void split8_prod(const float* a, const uint32_t* w, half8_t& hi,
                                            half8_t& lo)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto h = __builtin_amdgcn_cvt_pkrtz(mul_by_half<HI>(a[2 * i], w[2 * i]),
                                                  mul_by_half<HI>(a[2 * i + 1], w[2 * i + 1]));
        const uint32_t hb = __builtin_bit_cast(uint32_t, h);
        const auto l = __builtin_amdgcn_cvt_pkrtz(fma_half_minus_half<HI, 0>(a[2 * i], w[2 * i], hb),
                                                  fma_half_minus_half<HI, 1>(a[2 * i + 1],
                                                                            w[2 * i + 1], hb));
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

// Largest |x| of this lane's eight fp32 query elements of block blk (head
// hq, elements 32*blk + 8*q4 .. +7; 0 for the padded heads hq >= G).
template <int G, int D>
__device__ __forceinline__ float q_block_absmax(const void* q, size_t prow, int hq, int q4,
                                                int blk)
{
    if (hq >= G)
        return 0.f;
    const float4* qr = (const float4*)((const float*)q + (prow + hq) * D + 32 * blk + 8 * q4);
    const float4 a = qr[0], b = qr[1];
    return fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                 fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
}

// Power-of-two shift e that brings a positive finite amax into [2^lo, 2^(lo+1))
// as amax * 2^-e (0 for amax = 0, infinite or NaN).
__device__ __forceinline__ int pow2_shift(float amax, int lo)
{
    if (!(amax > 0.f) || amax == __builtin_inff())
        return 0;
    return __builtin_amdgcn_frexp_expf(amax) - 1 - lo;  // floor(log2 amax) - lo
}

// Wave-wide max (every lane gets it): DPP within rows of 16, then the four
// row results.
__device__ __forceinline__ float wave_max16x4(float v)
{
    v = row16_max(v);
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The query operand of block blk for this lane: head hq (zero beyond G),
// elements 32*blk + 8*q4 .. +7, as fp16 hi and lo halves of x * 2^-eq
// (fp32 queries; the exact power-of-two shift keeps both halves normal and
// finite, and the logits are scaled back by 2^eq).  fp16 queries are used
// as given (eq ignored).
template <int G, int D, bool QF16>
__device__ __forceinline__ void load_q_block(const void* q, size_t prow, int hq, int q4, int blk,
                                             int eq, half8_t& hi, half8_t& lo)
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
            const float xs = __builtin_amdgcn_ldexpf(x[e], -eq);
            const _Float16 h = (_Float16)xs;
            const _Float16 l = (_Float16)(xs - (float)h);
            hi[e] = hv ? h : (_Float16)0.f;
            lo[e] = hv ? l : (_Float16)0.f;
        }
    }
}

}  // namespace qsa
