// qsa_append.h -- KV append (device code shared by the append kernel and the
// single-launch decode window): quantise new tokens' K and V rows into int8
// codes with one fp16 scale per 32 elements, and their index keys into fp16
// (the cache format of "opus r20 track A: MTP map mlock + qsa_attn /
// qsa_merge decode tweaks", section 3).
//
// Quantiser (absmax reading; the pages name only the format): per block of
// 32 elements a = max |x|, s = fp16(a / 127), c = clamp(round(x / s), +-127),
// rounding to nearest-even on the exact values.  The scale comes from an
// fp32 quotient rounded to fp16 and is then decided against its two fp16
// neighbours with exact products (127 times an fp16 value has 18 significant
// bits, and its difference with a, when it matters, is exact by Sterbenz);
// the code quotient is formed in double, whose error (< 2^-46) is far below
// the smallest distance of a float / fp16 quotient to a half-integer, so
// rounding it to the nearest even integer gives the exact decision.
//
// Eight lanes per 32-element block of K or V (4 floats in, 4 codes out each;
// the scale is written by the first) and one lane per 4 index-key elements.
#pragma once

#include <math.h>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

__device__ __forceinline__ uint16_t f16_bits(_Float16 h)
{
    uint16_t u;
    __builtin_memcpy(&u, &h, 2);
    return u;
}

// Value of a non-negative binary16 pattern (0x7c00 and up: infinity).
__device__ __forceinline__ float f16_value(uint16_t u)
{
    return u >= 0x7c00u ? INFINITY : half_bits_to_float(u);
}

// fp16 pattern nearest to a / 127 for finite a >= 0, ties to the even
// pattern, never infinity (saturates at 65504).
__device__ __forceinline__ uint16_t scale_bits(float a)
{
    const uint16_t h = f16_bits((_Float16)(a / 127.0f));
    uint16_t best = h;
    float best_err = fabsf(a - 127.0f * f16_value(h));
    const uint16_t cand[2] = {(uint16_t)(h > 0 ? h - 1 : 0), (uint16_t)(h < 0x7c00u ? h + 1 : h)};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float err = fabsf(a - 127.0f * f16_value(cand[i]));
        if (err < best_err || (err == best_err && (cand[i] & 1u) == 0 && (best & 1u) == 1)) {
            best = cand[i];
            best_err = err;
        }
    }
    return best;
}

// Lane w of the quantisation items: 8 lanes per 32-element block of K or
// V, 4 elements each.
// w = ((((b * T + t) * Hkv + g) * NB + sb32) * 2 + which) * 8 + sub
struct QuantLane {
    int b, t, g, sb32, which, sub;
};

__device__ __forceinline__ QuantLane quant_lane(const AppendLaunch& a, long long w)
{
    const int NB = a.D / 32;
    QuantLane q;
    q.sub = (int)(w & 7);
    long long r = w >> 3;
    q.which = (int)(r & 1);
    r >>= 1;
    q.sb32 = (int)(r % NB);  // 32-element block of the row
    r /= NB;
    q.g = (int)(r % a.Hkv);
    r /= a.Hkv;
    q.t = (int)(r % a.T);
    q.b = (int)(r / a.T);
    return q;
}

// The lane's 4 new fp32 elements.
__device__ __forceinline__ float4 append_quant_load(const AppendLaunch& a, long long w)
{
    const QuantLane q = quant_lane(a, w);
    const float* src = (q.which ? a.v_new : a.k_new) +
                       (((size_t)q.b * a.T + q.t) * a.Hkv + q.g) * a.D + 32 * q.sb32 + 4 * q.sub;
    return *(const float4*)src;
}

// Quantise and store the lane's 4 elements v: the block maximum is combined
// over the 8 consecutive lanes of the block, so all 8 lanes of a group must
// call this together; `live` false makes a lane take part in the shuffles
// only.
__device__ __forceinline__ void append_quant_store(const AppendLaunch& a, long long w, float4 v,
                                                   bool live)
{
    const int NB = a.D / 32;
    const QuantLane q = quant_lane(a, w);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
    for (int o = 1; o < 8; o <<= 1)
        amax = fmaxf(amax, __shfl_xor(amax, o, 8));
    if (!live)
        return;
    const uint16_t sb = scale_bits(amax);
    const double s = (double)half_bits_to_float(sb);
    const float x[4] = {v.x, v.y, v.z, v.w};
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        int c = 0;
        if (s > 0.0) {
            const double qv = rint((double)x[e] / s);
            c = (int)fmin(fmax(qv, -127.0), 127.0);
        }
        word |= ((uint32_t)(uint8_t)(int8_t)c) << (8 * e);
    }
    const long long cell = (long long)(a.pos0 + q.t);
    int8_t* codes = (q.which ? a.Vq : a.Kq) + (long long)q.b * (q.which ? a.vq_bs : a.kq_bs) +
                    cell * (q.which ? a.vq_cs : a.kq_cs) + (long long)q.g * a.D + 32 * q.sb32 +
                    4 * q.sub;
    *(uint32_t*)codes = word;
    if (q.sub == 0) {
        char* sc = (char*)(q.which ? a.Vsc : a.Ksc) +
                   (long long)q.b * (q.which ? a.vsc_bs : a.ksc_bs) +
                   cell * (q.which ? a.vsc_cs : a.ksc_cs) + ((long long)q.g * NB + q.sb32) * 2;
        *(uint16_t*)sc = sb;
    }
}

// Both steps for lane w (see above).
__device__ __forceinline__ void append_quant_lane(const AppendLaunch& a, long long w, bool live)
{
    const float4 v = live ? append_quant_load(a, w) : make_float4(0.f, 0.f, 0.f, 0.f);
    append_quant_store(a, w, v, live);
}

// fp16 bits of two floats (nearest, ties to even), the first in the low half.
__device__ __forceinline__ uint32_t pack_half2_rne(float lo, float hi)
{
    return (uint32_t)f16_bits((_Float16)lo) | ((uint32_t)f16_bits((_Float16)hi) << 16);
}

// Lane r of the index-key items: 4 elements of (b, t), r = (b * T + t) *
// (DI / 4) + i.
__device__ __forceinline__ void append_index_lane(const AppendLaunch& a, long long r)
{
    const int per = a.DI / 4;
    const int i = (int)(r % per);
    const long long bt = r / per;
    const int t = (int)(bt % a.T);
    const int b = (int)(bt / a.T);
    const float4 v = ((const float4*)(a.kidx_new + (size_t)bt * a.DI))[i];
    uint16_t* dst = a.K_idx + ((size_t)b * a.N + a.pos0 + t) * a.DI + 4 * i;
    ((uint2*)dst)[0] = make_uint2(pack_half2_rne(v.x, v.y), pack_half2_rne(v.z, v.w));
}

// Items: the quantisation lanes, then one lane per 4 index-key elements.
// Blocks occupy whole 8-lane groups, so the shuffles stay inside a group.
// Workgroup blk of nblk (256 threads each) takes every nblk-th group of 256
// items.
__device__ __forceinline__ void append_blocks(const AppendLaunch& a, long long q_lanes,
                                              long long n_quant, long long n_idx, int blk,
                                              int nblk)
{
    const long long total = n_quant + n_idx;  // n_quant: q_lanes rounded up to 256
    const long long stride = (long long)nblk * 256;
    for (long long w0 = (long long)blk * 256; w0 < total; w0 += stride) {
        const long long w = w0 + threadIdx.x;
        if (w0 < n_quant) {
            // The whole workgroup is in the quantisation range (n_quant is a
            // multiple of 256), so every lane reaches the shuffles.
            append_quant_lane(a, w, w < q_lanes);
        } else if (w < total) {
            // index keys (n_quant is a multiple of 256, so this whole
            // workgroup is in the index range)
            append_index_lane(a, w - n_quant);
        }
    }
}

// The items of problem b only, by the `nthreads` threads of one workgroup
// (a multiple of 8): its T tokens' K and V blocks, then their index keys
// (when kidx_new is given).
__device__ __forceinline__ void append_problem(const AppendLaunch& a, int b, int nthreads)
{
    const long long nq = (long long)a.T * a.Hkv * (a.D / 32) * 16;  // a multiple of 16
    for (long long l = threadIdx.x; l < nq; l += nthreads)
        append_quant_lane(a, (long long)b * nq + l, true);
    if (a.kidx_new) {
        const long long ni = (long long)a.T * (a.DI / 4);
        for (long long l = threadIdx.x; l < ni; l += nthreads)
            append_index_lane(a, (long long)b * ni + l);
    }
}

}  // namespace qsa
