// qsa_attend.hip -- split-KV attention over the kept cells, and the merge of
// the chunk partials (gfx950, wave64).
//
// Method ("opus r20 track A: MTP map mlock + qsa_attn / qsa_merge decode
// tweaks", section 2 "qsa.metal"): each chunk of a token's kept cells yields
// the exact max of its logits, the sum of exp(logit - max) and the
// unnormalised exp-weighted sum of V rows; an absent cell contributes p = 0;
// V is read as int8 codes times an fp16 scale per 32 elements (section 3),
// and every V row loaded feeds a per-head FMA chain (the query heads that
// share a KV head).  The merge rescales each chunk by exp(m_c - M), sums
// l_c e_c and o_c e_c with fma in chunk order, then divides once.
//
// k_attend: one wave per (token, chunk, KV head); its G query heads share
// every K and V row it gathers (GQA).  Cells are taken 64 at a time:
//   QK  lane i owns cell i of the tile and streams that cell's int8 K row
//       (D bytes) and fp16 scales; the G query rows are wave-uniform and are
//       read from SGPRs (scalar loads), so each int8 code is converted once
//       (one SDWA convert) and used by G fp32 FMAs.  The per-32 block scale
//       multiplies the block's partial dot product.
//   softmax  tile max and sum over lanes with butterfly reductions; a running
//       (max, sum) pair rescales earlier tiles when a chunk spans several.
//   PV  lane owns D/64 consecutive output elements of all G heads; each kept
//       cell's V row is read once, coalesced across the wave, scaled, and
//       accumulated into G*D/64 fp32 FMAs with the weights broadcast from LDS.
#include <math.h>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

// Loads N consecutive wave-uniform 32-bit words starting at element `off`.
// The offset passes through an empty asm so the loads stay where they are
// written (they are not merged with, or hoisted next to, other heads' loads).
template <int N, typename T>
__device__ __forceinline__ void load_uniform(const T* __restrict__ base, size_t off, T* dst)
{
    asm volatile("" : "+s"(off));
#pragma unroll
    for (int e = 0; e < N; ++e)
        dst[e] = base[off + e];
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

template <int G, int D, bool QF16>
__global__ __launch_bounds__(64) void k_attend(
    const void* __restrict__ q, const int8_t* __restrict__ Kq, const uint8_t* __restrict__ Ksc,
    const int8_t* __restrict__ Vq, const uint8_t* __restrict__ Vsc, long long kq_cs,
    long long ksc_cs, long long vq_cs, long long vsc_cs, long long kq_bs, long long ksc_bs,
    long long vq_bs, long long vsc_bs, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ n_sel, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ po, int T, int Hq, int P, int cap, int N, float scale)
{
    constexpr int NB = D / 32;        // scale blocks per head row
    constexpr int DPL = D / 64;       // output elements per lane
    constexpr int GP = (G + 3) & ~3;  // LDS row pitch of the tile weights
    __shared__ float p_s[64 * GP];

    const int bt = blockIdx.x, c = blockIdx.y, g = blockIdx.z;
    const int b = bt / T;
    const int lane = threadIdx.x;
    const size_t prow = (size_t)bt * Hq + (size_t)g * G;  // row of head g*G

    const int ns = min(n_sel[bt], cap);
    const int S = (ns + P - 1) / P;
    const int beg = c * S;
    const int end = min(beg + S, ns);

    if (beg >= end) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (lane == 0) {
                pm[(prow + h) * P + c] = -INFINITY;
                pl[(prow + h) * P + c] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                po[((prow + h) * P + c) * D + lane * DPL + e] = 0.f;
        }
        return;
    }

    const char* Kb = (const char*)Kq + (long long)b * kq_bs + (long long)g * D;
    const char* Ksb = (const char*)Ksc + (long long)b * ksc_bs + (long long)g * NB * 2;
    const char* Vb = (const char*)Vq + (long long)b * vq_bs + (long long)g * D;
    const char* Vsb = (const char*)Vsc + (long long)b * vsc_bs + (long long)g * NB * 2;
    const int32_t* idr = ids + (size_t)bt * cap;

    float m_run[G], l_run[G], o[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            o[h][e] = 0.f;
    }

#pragma unroll 1
    for (int t0 = beg; t0 < end; t0 += 64) {
        const int nt = min(64, end - t0);
        const bool valid = lane < nt;
        // Ids outside [0, N) are undefined input; clamping keeps every
        // gather inside the cache.
        const int j = min((unsigned)idr[t0 + (valid ? lane : 0)], (unsigned)(N - 1));

        // ---- QK: lane = cell ------------------------------------------
        const char* kr = Kb + (long long)j * kq_cs;
        const uint32_t* ksr = (const uint32_t*)(Ksb + (long long)j * ksc_cs);
        float ksc[NB];
#pragma unroll
        for (int w = 0; w < NB / 2; ++w) {
            const uint32_t two = ksr[w];
            ksc[2 * w] = half_bits_to_float((uint16_t)(two & 0xffffu));
            ksc[2 * w + 1] = half_bits_to_float((uint16_t)(two >> 16));
        }
        float x[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
            x[h] = 0.f;
        // The G x D query values are wave-uniform and are scalar-loaded one
        // head (32 values of one scale block) ahead of use; sched_barrier
        // fences keep the compiler from hoisting all of them at once, which
        // would overflow the SGPR file.
        int4 wa0 = *(const int4*)(kr);
        int4 wa1 = *(const int4*)(kr + 16);
#pragma unroll 1
        for (int blk = 0; blk < NB; ++blk) {
            const int nblk = min(blk + 1, NB - 1);
            const int4 wb0 = *(const int4*)(kr + nblk * 32);  // next block's codes
            const int4 wb1 = *(const int4*)(kr + nblk * 32 + 16);
            const int ww[8] = {wa0.x, wa0.y, wa0.z, wa0.w, wa1.x, wa1.y, wa1.z, wa1.w};
            if constexpr (!QF16) {
                float kf[32];
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    kf[e] = sbyte_to_float(ww[e >> 2], e & 3);
                const float* qf = (const float*)q;
                float qc[32], qn[32];
                load_uniform<32>(qf, prow * D + blk * 32, qc);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    if (h + 1 < G)
                        load_uniform<32>(qf, (prow + h + 1) * D + blk * 32, qn);
                    __builtin_amdgcn_sched_barrier(0);
                    float part = 0.f;
#pragma unroll
                    for (int e = 0; e < 32; ++e)
                        part = fmaf(qc[e], kf[e], part);
                    x[h] = fmaf(ksc[blk], part, x[h]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int e = 0; e < 32; ++e)
                        qc[e] = qn[e];
                }
            } else {
                // fp16 queries: int8 codes become exact fp16 pairs and each
                // v_dot2 takes two fp16 x fp16 products (exact) into the fp32
                // accumulator.
                half2_t k2[16];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    k2[2 * i] = int8_pair_to_half2(ww[i], 0);
                    k2[2 * i + 1] = int8_pair_to_half2(ww[i], 1);
                }
                const uint32_t* q2 = (const uint32_t*)q;
                uint32_t qc[16], qn[16];
                load_uniform<16>(q2, (prow * D + blk * 32) / 2, qc);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    if (h + 1 < G)
                        load_uniform<16>(q2, ((prow + h + 1) * D + blk * 32) / 2, qn);
                    __builtin_amdgcn_sched_barrier(0);
                    float part = 0.f;
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        part = __builtin_amdgcn_fdot2(as_half2(qc[e]), k2[e], part, false);
                    x[h] = fmaf(ksc[blk], part, x[h]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        qc[e] = qn[e];
                }
            }
            wa0 = wb0;
            wa1 = wb1;
        }

        // ---- softmax over the tile, folded into the running pair -------
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float xs = valid ? x[h] * scale : -INFINITY;
            const float mn = fmaxf(m_run[h], wave_max(xs));
            const float alpha = __builtin_amdgcn_exp2f((m_run[h] - mn) * kLog2e);
            const float p = valid ? __builtin_amdgcn_exp2f((xs - mn) * kLog2e) : 0.f;
            l_run[h] = fmaf(l_run[h], alpha, wave_sum(p));
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                o[h][e] *= alpha;
            m_run[h] = mn;
            p_s[lane * GP + h] = p;
        }
        __syncthreads();

        // ---- PV: lane = DPL output elements, loop over the tile's cells --
        const int dsc = (lane * DPL) >> 5;  // scale block of this lane's elements
#pragma unroll 4
        for (int i = 0; i < nt; ++i) {
            const int jj = __builtin_amdgcn_readlane(j, i);
            const char* vr = Vb + (long long)jj * vq_cs + lane * DPL;
            const float vs = half_bits_to_float(
                *(const uint16_t*)(Vsb + (long long)jj * vsc_cs + dsc * 2));
            float vf[DPL];
            if constexpr (DPL == 4) {
                const int w = *(const int*)vr;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    vf[e] = sbyte_to_float(w, e) * vs;
            } else if constexpr (DPL == 2) {
                const int w = (int)*(const uint16_t*)vr;
                vf[0] = sbyte_to_float(w, 0) * vs;
                vf[1] = sbyte_to_float(w, 1) * vs;
            } else {
                vf[0] = (float)(*(const int8_t*)vr) * vs;
            }
            const float* pr = p_s + i * GP;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pv = pr[h];
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    o[h][e] = fmaf(pv, vf[e], o[h][e]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int h = 0; h < G; ++h) {
        if (lane == 0) {
            pm[(prow + h) * P + c] = m_run[h];
            pl[(prow + h) * P + c] = l_run[h];
        }
        float* dst = po + ((prow + h) * P + c) * D + lane * DPL;
        if constexpr (DPL == 4) {
            *(float4*)dst = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
        } else {
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                dst[e] = o[h][e];
        }
    }
}

// One workgroup of D threads per (token, query head) row; thread d merges
// output element d.
template <int D, bool OUTF16>
__global__ __launch_bounds__(D) void k_merge(const float* __restrict__ pm,
                                             const float* __restrict__ pl,
                                             const float* __restrict__ po,
                                             void* __restrict__ out, int P)
{
    const size_t r = blockIdx.x;
    const int d = threadIdx.x;
    const float* m = pm + r * P;
    const float* l = pl + r * P;
    const float* o = po + r * P * D + d;
    float M = -INFINITY;
    for (int c = 0; c < P; ++c)
        M = fmaxf(M, m[c]);
    float L = 0.f, y = 0.f;
    if (M != -INFINITY) {
        for (int c = 0; c < P; ++c) {
            const float mc = m[c];
            if (mc == -INFINITY)
                continue;  // empty chunk: weight 0
            const float e = expf(mc - M);
            L = fmaf(l[c], e, L);
            y = fmaf(o[(size_t)c * D], e, y);
        }
    }
    const float res = (L > 0.f) ? y / L : 0.f;
    if constexpr (OUTF16)
        ((_Float16*)out)[r * D + d] = (_Float16)res;
    else
        ((float*)out)[r * D + d] = res;
}

// ------------------------------------------------------------- launch ---

template <int G, int D>
static void launch_attend_gd(const AttnLaunch& a, hipStream_t s)
{
    dim3 grid((unsigned)(a.B * a.T), (unsigned)a.P, (unsigned)a.Hkv);
#define QSA_ATTEND_ARGS                                                                      \
    a.q, a.Kq, (const uint8_t*)a.Ksc, a.Vq, (const uint8_t*)a.Vsc, a.kq_cs, a.ksc_cs, a.vq_cs, \
        a.vsc_cs, a.kq_bs, a.ksc_bs, a.vq_bs, a.vsc_bs, a.ids, a.n_sel, a.pm, a.pl, a.po, a.T, \
        a.Hq, a.P, a.cap, a.N, a.scale
    if (a.q_f16)
        k_attend<G, D, true><<<grid, 64, 0, s>>>(QSA_ATTEND_ARGS);
    else
        k_attend<G, D, false><<<grid, 64, 0, s>>>(QSA_ATTEND_ARGS);
#undef QSA_ATTEND_ARGS
}

template <int D>
static bool launch_attend_d(const AttnLaunch& a, int G, hipStream_t s)
{
    switch (G) {
    case 1: launch_attend_gd<1, D>(a, s); return true;
    case 2: launch_attend_gd<2, D>(a, s); return true;
    case 4: launch_attend_gd<4, D>(a, s); return true;
    case 8: launch_attend_gd<8, D>(a, s); return true;
    case 12: launch_attend_gd<12, D>(a, s); return true;
    case 16: launch_attend_gd<16, D>(a, s); return true;
    default: return false;
    }
}

bool attend_supported(int G, int D)
{
    const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8 || G == 12 || G == 16;
    return g_ok && (D == 64 || D == 256);
}

hipError_t launch_attend(const AttnLaunch& a, hipStream_t s)
{
    const int G = a.Hq / a.Hkv;
    const bool ok = (a.D == 64) ? launch_attend_d<64>(a, G, s) : launch_attend_d<256>(a, G, s);
    if (!ok)
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_merge(const AttnLaunch& a, hipStream_t s)
{
    const unsigned rows = (unsigned)(a.B * a.T * a.Hq);
    if (a.D == 64) {
        if (a.out_f16)
            k_merge<64, true><<<rows, 64, 0, s>>>(a.pm, a.pl, a.po, a.out, a.P);
        else
            k_merge<64, false><<<rows, 64, 0, s>>>(a.pm, a.pl, a.po, a.out, a.P);
    } else {
        if (a.out_f16)
            k_merge<256, true><<<rows, 256, 0, s>>>(a.pm, a.pl, a.po, a.out, a.P);
        else
            k_merge<256, false><<<rows, 256, 0, s>>>(a.pm, a.pl, a.po, a.out, a.P);
    }
    return hipGetLastError();
}

}  // namespace qsa
