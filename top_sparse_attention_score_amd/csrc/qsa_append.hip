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
// Eight lanes per 32-element block of K or V (4 floats in, 4 codes out each;
// the scale is written by the first) and one lane per 4 index-key elements.
#include <math.h>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

static __device__ __forceinline__ uint16_t f16_bits(_Float16 h)
{
    uint16_t u;
    __builtin_memcpy(&u, &h, 2);
    return u;
}

// Value of a non-negative binary16 pattern (0x7c00 and up: infinity).
static __device__ __forceinline__ float f16_value(uint16_t u)
{
    return u >= 0x7c00u ? INFINITY : half_bits_to_float(u);
}

// fp16 pattern nearest to a / 127 for finite a >= 0, ties to the even
// pattern, never infinity (saturates at 65504).
static __device__ __forceinline__ uint16_t scale_bits(float a)
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

// Items: 8 lanes per 32-element block of K or V (4 elements each; the
// block maximum is combined over the 8 consecutive lanes), then one lane per
// 4 index-key elements.  Blocks occupy whole 8-lane groups, so the shuffles
// stay inside a group.
__global__ __launch_bounds__(256) void k_kv_append(AppendLaunch a, long long q_lanes,
                                                   long long n_quant, long long n_idx)
{
    const int NB = a.D / 32;
    const long long total = n_quant + n_idx;  // n_quant: q_lanes rounded up to 256
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long w0 = (long long)blockIdx.x * blockDim.x; w0 < total; w0 += stride) {
        const long long w = w0 + threadIdx.x;
        if (w0 < n_quant) {
            // The whole workgroup is in the quantisation range (n_quant is a
            // multiple of 256), so every lane reaches the shuffles.
            // w = ((((b * T + t) * Hkv + g) * NB + blk) * 2 + which) * 8 + sub
            const int sub = (int)(w & 7);
            long long r = w >> 3;
            const int which = (int)(r & 1);
            r >>= 1;
            const int blk = (int)(r % NB);
            r /= NB;
            const int g = (int)(r % a.Hkv);
            r /= a.Hkv;
            const int t = (int)(r % a.T);
            const int b = (int)(r / a.T);
            const bool live = w < q_lanes;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (live) {
                const float* src = (which ? a.v_new : a.k_new) +
                                   (((size_t)b * a.T + t) * a.Hkv + g) * a.D + 32 * blk + 4 * sub;
                v = *(const float4*)src;
            }
            float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
            for (int o = 1; o < 8; o <<= 1)
                amax = fmaxf(amax, __shfl_xor(amax, o, 8));
            if (!live)
                continue;
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
            const long long cell = (long long)(a.pos0 + t);
            int8_t* codes = (which ? a.Vq : a.Kq) + (long long)b * (which ? a.vq_bs : a.kq_bs) +
                            cell * (which ? a.vq_cs : a.kq_cs) + (long long)g * a.D + 32 * blk +
                            4 * sub;
            *(uint32_t*)codes = word;
            if (sub == 0) {
                char* sc = (char*)(which ? a.Vsc : a.Ksc) +
                           (long long)b * (which ? a.vsc_bs : a.ksc_bs) +
                           cell * (which ? a.vsc_cs : a.ksc_cs) + ((long long)g * NB + blk) * 2;
                *(uint16_t*)sc = sb;
            }
        } else if (w < total) {
            // index keys: 4 elements of (b, t) (n_quant is a multiple of 256,
            // so this whole workgroup is in the index range)
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

hipError_t launch_kv_append(const AppendLaunch& a, hipStream_t s)
{
    // Quantisation lanes rounded up to whole workgroups, so no workgroup
    // mixes the two kinds of items (the extra lanes are idle).
    const long long q_lanes = (long long)a.B * a.T * a.Hkv * (a.D / 32) * 2 * 8;
    const long long n_quant = (q_lanes + 255) / 256 * 256;
    const long long n_idx = a.kidx_new ? (long long)a.B * a.T * (a.DI / 4) : 0;
    const long long blocks = (n_quant + n_idx + 255) / 256;
    k_kv_append<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, s>>>(a, q_lanes, n_quant,
                                                                          n_idx);
    return hipGetLastError();
}

}  // namespace qsa
