// qsa_merge.h -- the log-sum-exp merge of split-KV partials as a device
// function of one (virtual) workgroup, shared by the merge kernel and the
// single-launch decode window ("opus r20 track A: MTP map mlock + qsa_attn /
// qsa_merge decode tweaks", section 2 "qsa.metal", qsa_merge: rescale each
// chunk by exp(m_c - M), fma in chunk order, then one division).
#pragma once

#include <math.h>

#include "qsa_device.h"

namespace qsa {

constexpr int kMergeWaves = 4;

// The merge of EPL consecutive output elements of one (token, query head)
// row over its P chunks, in the order the merge formula fixes: M = max_c
// m_c, then over the chunks in order e = exp(m_c - M) (0 for an empty
// chunk), L = fma(l_c, e, L), y = fma(o_c, e, y), and one division.  An
// empty chunk has l = o = 0, so its zero weight leaves L and y bitwise
// unchanged.  Chunk c's m and l are at m[c * ms] and l[c * ms], its elements
// at o + c * os (global memory for the merge kernel, LDS for the fused
// attention epilogue: both run this same sequence, so their results agree
// bit for bit).
template <int EPL>
__device__ __forceinline__ void merge_elems(const float* m, const float* l, int ms,
                                            const float* o, long long os, int P, float res[EPL])
{
    float M = -INFINITY;
    for (int c = 0; c < P; ++c)
        M = fmaxf(M, m[(long long)c * ms]);
    float L = 0.f;
    float y[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        y[e] = 0.f;
    if (M != -INFINITY) {
#pragma unroll 8
        for (int c = 0; c < P; ++c) {
            const float mc = m[(long long)c * ms];
            const float w = (mc == -INFINITY) ? 0.f : expf(mc - M);
            L = fmaf(l[(long long)c * ms], w, L);
            if constexpr (EPL == 4) {
                const float4 v = *(const float4*)(o + c * os);
                y[0] = fmaf(v.x, w, y[0]);
                y[1] = fmaf(v.y, w, y[1]);
                y[2] = fmaf(v.z, w, y[2]);
                y[3] = fmaf(v.w, w, y[3]);
            } else {
                y[0] = fmaf(o[c * os], w, y[0]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        res[e] = (L > 0.f) ? y[e] / L : 0.f;
}

// Output gate and store of EPL merged elements at element offset `off` of
// out; the gate values are at element offset `goff` of `gate` (fp16 when
// gate_f16, else fp32; the gate has the layout of q, and the fused attention
// epilogue passes a copy in LDS): with a gate, each result is multiplied by
// 1 / (1 + exp(-g)) in fp32, then rounded to fp16 (nearest even) when
// OUTF16.
template <int EPL, bool OUTF16>
__device__ __forceinline__ void gate_store(float res[EPL], const void* __restrict__ gate,
                                           int gate_f16, long long goff, void* __restrict__ out,
                                           long long off)
{
    if (gate) {
        float gv[EPL];
        if (gate_f16) {
            const _Float16* gp = (const _Float16*)gate + goff;
            if constexpr (EPL == 4) {
                const half4_t g4 = *(const half4_t*)gp;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    gv[e] = (float)g4[e];
            } else {
                gv[0] = (float)gp[0];
            }
        } else {
            const float* gp = (const float*)gate + goff;
            if constexpr (EPL == 4) {
                const float4 g4 = *(const float4*)gp;
                gv[0] = g4.x;
                gv[1] = g4.y;
                gv[2] = g4.z;
                gv[3] = g4.w;
            } else {
                gv[0] = gp[0];
            }
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            res[e] *= 1.f / (1.f + expf(-gv[e]));
    }
    if constexpr (OUTF16) {
        _Float16* dst = (_Float16*)out + off;
        if constexpr (EPL == 4)
            *(half4_t*)dst = half4_t{(_Float16)res[0], (_Float16)res[1], (_Float16)res[2],
                                     (_Float16)res[3]};
        else
            dst[0] = (_Float16)res[0];
    } else {
        float* dst = (float*)out + off;
        if constexpr (EPL == 4)
            *(float4*)dst = make_float4(res[0], res[1], res[2], res[3]);
        else
            dst[0] = res[0];
    }
}

// EPL (4 or 1) consecutive output elements per lane, D/EPL lanes per (token,
// query head) row; a wave covers 64/(D/EPL) rows (EPL = 1 spreads rows with
// many chunks over more waves).
template <int D, int EPL, bool OUTF16>
__device__ __forceinline__ void merge_block(int blk, const float* __restrict__ pm,
                                            const float* __restrict__ pl,
                                            const float* __restrict__ po,
                                            void* __restrict__ out, int P, long long rows,
                                            const void* __restrict__ gate, int gate_f16)
{
    constexpr int LPR = D / EPL;   // lanes per row
    constexpr int RPW = 64 / LPR;  // rows per wave (D = 64, EPL = 1: one row per wave)
    static_assert(LPR <= 64 || LPR % 64 == 0, "rows map to whole lane groups or waves");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    long long r;
    int de;  // first element of this lane
    if constexpr (LPR <= 64) {
        r = ((long long)blk * kMergeWaves + wave) * RPW + lane / LPR;
        de = EPL * (lane % LPR);
    } else {
        constexpr int WPR = LPR / 64;  // waves per row
        r = ((long long)blk * kMergeWaves + wave) / WPR;
        de = EPL * (64 * (wave % WPR) + lane);
    }
    if (r >= rows)
        return;
    float res[EPL];
    merge_elems<EPL>(pm + r * P, pl + r * P, 1, po + r * P * D + de, D, P, res);
    gate_store<EPL, OUTF16>(res, gate, gate_f16, r * D + de, out, r * D + de);
}

}  // namespace qsa
