// qsa_append.hip -- KV append: quantise new tokens' K and V rows into int8
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
// One thread per 32-element block of K or V (32 floats in, 32 codes and a
// scale out) and one per 4 index-key elements.
#include <math.h>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

namespace {

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

__global__ __launch_bounds__(256) void k_kv_append(AppendLaunch a, long long n_quant,
                                                   long long n_idx)
{
    const int NB = a.D / 32;
    const long long total = n_quant + n_idx;
    for (long long w = (long long)blockIdx.x * blockDim.x + threadIdx.x; w < total;
         w += (long long)gridDim.x * blockDim.x) {
        if (w < n_quant) {
            // w = (((b * T + t) * Hkv + g) * NB + blk) * 2 + which
            const int which = (int)(w & 1);
            long long r = w >> 1;
            const int blk = (int)(r % NB);
            r /= NB;
            const int g = (int)(r % a.Hkv);
            r /= a.Hkv;
            const int t = (int)(r % a.T);
            const int b = (int)(r / a.T);
            const float* src = (which ? a.v_new : a.k_new) +
                               (((size_t)b * a.T + t) * a.Hkv + g) * a.D + 32 * blk;
            float x[32];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 v = ((const float4*)src)[i];
                x[4 * i] = v.x;
                x[4 * i + 1] = v.y;
                x[4 * i + 2] = v.z;
                x[4 * i + 3] = v.w;
            }
            float amax = 0.f;
#pragma unroll
            for (int e = 0; e < 32; ++e)
                amax = fmaxf(amax, fabsf(x[e]));
            const uint16_t sb = scale_bits(amax);
            const double s = (double)half_bits_to_float(sb);
            uint32_t word[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t wv = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    int c = 0;
                    if (s > 0.0) {
                        const double qv = rint((double)x[4 * i + e] / s);
                        c = (int)fmin(fmax(qv, -127.0), 127.0);
                    }
                    wv |= ((uint32_t)(uint8_t)(int8_t)c) << (8 * e);
                }
                word[i] = wv;
            }
            const long long cell = (long long)(a.pos0 + t);
            int8_t* codes = (which ? a.Vq : a.Kq) + (long long)b * (which ? a.vq_bs : a.kq_bs) +
                            cell * (which ? a.vq_cs : a.kq_cs) + (long long)g * a.D + 32 * blk;
            ((uint4*)codes)[0] = make_uint4(word[0], word[1], word[2], word[3]);
            ((uint4*)codes)[1] = make_uint4(word[4], word[5], word[6], word[7]);
            char* sc = (char*)(which ? a.Vsc : a.Ksc) + (long long)b * (which ? a.vsc_bs : a.ksc_bs) +
                       cell * (which ? a.vsc_cs : a.ksc_cs) + ((long long)g * NB + blk) * 2;
            *(uint16_t*)sc = sb;
        } else {
            // index keys: 4 elements of (b, t)
            const long long r = w - n_quant;
            const int per = a.DI / 4;
            const int i = (int)(r % per);
            const long long bt = r / per;
            const int t = (int)(bt % a.T);
            const int b = (int)(bt / a.T);
            const float4 v = ((const float4*)(a.kidx_new + (size_t)bt * a.DI))[i];
            const uint16_t h0 = f16_bits((_Float16)v.x), h1 = f16_bits((_Float16)v.y);
            const uint16_t h2 = f16_bits((_Float16)v.z), h3 = f16_bits((_Float16)v.w);
            uint16_t* dst = a.K_idx + ((size_t)b * a.N + a.pos0 + t) * a.DI + 4 * i;
            ((uint2*)dst)[0] = make_uint2((uint32_t)h0 | ((uint32_t)h1 << 16),
                                          (uint32_t)h2 | ((uint32_t)h3 << 16));
        }
    }
}

}  // namespace

hipError_t launch_kv_append(const AppendLaunch& a, hipStream_t s)
{
    const long long n_quant = (long long)a.B * a.T * a.Hkv * (a.D / 32) * 2;
    const long long n_idx = a.kidx_new ? (long long)a.B * a.T * (a.DI / 4) : 0;
    const long long total = n_quant + n_idx;
    const long long blocks = (total + 255) / 256;
    k_kv_append<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, s>>>(a, n_quant, n_idx);
    return hipGetLastError();
}

}  // namespace qsa
