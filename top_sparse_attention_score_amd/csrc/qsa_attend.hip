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
// k_attend: one wave per (token, chunk, KV head), four consecutive (token,
// chunk) items per workgroup, so chunks of one token share its query rows in
// the scalar cache; a wave's G query heads share every K and V row it
// gathers (GQA).
// Cells are taken 64 at a time:
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
#include "qsa_merge.h"

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

// Copies the V codes (D bytes) and V scales (D/16 bytes) of the tile's 64
// cells from the cache straight into LDS (gfx950 global_load_lds, no VGPR
// round trip).  Row-major: cell i's codes at v_s[i*D], scales at vsc_s[i*D/32].
// `j` is this lane's cell (lane = cell); tail lanes hold a valid duplicate.
template <int D>
__device__ __forceinline__ void dma_v_tile(const char* Vb, long long vq_cs, const char* Vsb,
                                           long long vsc_cs, int j, int8_t* v_s,
                                           uint16_t* vsc_s)
{
    constexpr int LPC = D / 16;   // lanes per cell row (16 bytes each)
    constexpr int CPI = 64 / LPC; // cells per instruction
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 64 / CPI; ++i) {
        const int cell = i * CPI + lane / LPC;
        const int jj = __shfl(j, cell, 64);
        const char* src = Vb + (long long)jj * vq_cs + (lane % LPC) * 16;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(v_s + i * CPI * D), 16,
                                         0, 0);
    }
    const char* ssrc = Vsb + (long long)j * vsc_cs;
    if constexpr (D / 16 == 16)
        __builtin_amdgcn_global_load_lds((const void*)ssrc, (lds_void_t*)vsc_s, 16, 0, 0);
    else
        __builtin_amdgcn_global_load_lds((const void*)ssrc, (lds_void_t*)vsc_s, 4, 0, 0);
}

constexpr int kAttendWaves = 4;  // chunks of one (token, KV head) per workgroup

template <int G, int D, bool QF16>
__global__ __launch_bounds__(64 * kAttendWaves) void k_attend(
    const void* __restrict__ q, const int8_t* __restrict__ Kq, const uint8_t* __restrict__ Ksc,
    const int8_t* __restrict__ Vq, const uint8_t* __restrict__ Vsc, long long kq_cs,
    long long ksc_cs, long long vq_cs, long long vsc_cs, long long kq_bs, long long ksc_bs,
    long long vq_bs, long long vsc_bs, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ n_sel, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ po, int T, int Hq, int P, int cap, int N, int BT, float scale)
{
    constexpr int NB = D / 32;        // scale blocks per head row
    constexpr int DPL = D / 64;       // output elements per lane
    constexpr int GP = (G + 3) & ~3;  // LDS row pitch of the tile weights
    constexpr int KC = D / 16;        // 16-byte chunks per K row
    constexpr int SW = NB / 2;        // 32-bit words of scales per head row
    __shared__ __align__(16) int8_t v_all[kAttendWaves][64 * D];
    __shared__ __align__(16) uint16_t vsc_all[kAttendWaves][64 * NB];
    __shared__ __align__(16) float p_all[kAttendWaves][64 * GP];

    // Each wave takes one (token, chunk) item; consecutive items are the
    // chunks of one token, so for P >= 4 the waves of a workgroup share the
    // token's query rows, and for small P no wave of a workgroup idles.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const long long item = (long long)blockIdx.x * kAttendWaves + wave;
    if (item >= (long long)BT * P)
        return;
    const int bt = (int)(item / P), c = (int)(item % P), g = blockIdx.y;
    int8_t* v_s = v_all[wave];
    uint16_t* vsc_s = vsc_all[wave];
    float* p_s = p_all[wave];
    const int b = bt / T;
    const int lane = threadIdx.x & 63;
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

    // Lane = cell of the current 64-cell tile.  Ids outside [0, N) are
    // undefined input; clamping keeps every gather inside the cache.  Tail
    // lanes duplicate the tile's first cell so every load stays valid.
    int t0 = beg;
    int nt = min(64, end - t0);
    int j = min((unsigned)idr[t0 + (lane < nt ? lane : 0)], (unsigned)(N - 1));
    uint4 krow[KC];
    uint32_t ksw[SW];
    {
        const uint4* kr = (const uint4*)(Kb + (long long)j * kq_cs);
#pragma unroll
        for (int i = 0; i < KC; ++i)
            krow[i] = kr[i];
        const uint32_t* ks = (const uint32_t*)(Ksb + (long long)j * ksc_cs);
#pragma unroll
        for (int w = 0; w < SW; ++w)
            ksw[w] = ks[w];
    }

#pragma unroll 1
    for (;;) {
        const bool valid = lane < nt;
        const int t1 = t0 + 64;
        const bool more = t1 < end;
        const int nt1 = more ? min(64, end - t1) : 0;
        int jn = 0;
        // Settle the K row (loaded during the previous PV phase) before any
        // copy of this tile is issued: after this no K use waits on memory,
        // so the V copy below overlaps the whole QK phase.
#pragma unroll
        for (int i = 0; i < KC; ++i)
            asm volatile("" : "+v"(krow[i].x), "+v"(krow[i].y), "+v"(krow[i].z),
                         "+v"(krow[i].w));
#pragma unroll
        for (int w = 0; w < SW; ++w)
            asm volatile("" : "+v"(ksw[w]));
        dma_v_tile<D>(Vb, vq_cs, Vsb, vsc_cs, j, v_s, vsc_s);
        if (more)
            jn = idr[t1 + (lane < nt1 ? lane : 0)];

        // ---- QK: lane = cell, K row in VGPRs, queries in SGPRs --------
        // The query row offset is re-derived each tile (empty asm) so the
        // per-segment offsets below are computed inside the loop instead of
        // being precomputed and held for every segment.
        size_t qrow = prow * D;
        asm volatile("" : "+s"(qrow));
        float x[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
            x[h] = 0.f;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const uint4 w0 = krow[2 * blk], w1 = krow[2 * blk + 1];
            const int ww[8] = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w,
                               (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
            const uint32_t sw = ksw[blk / 2];
            const float ksc = half_bits_to_float((uint16_t)((blk & 1) ? (sw >> 16) : (sw & 0xffffu)));

            if constexpr (!QF16) {
                float kf[32];
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    kf[e] = sbyte_to_float(ww[e >> 2], e & 3);
                // One head's 32 query values of this block at a time; the next
                // head's are scalar-loaded while these are used.
                const float* qf = (const float*)q;
                float qc[32], qn[32];
                load_uniform<32>(qf, qrow + blk * 32, qc);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    if (h + 1 < G)
                        load_uniform<32>(qf, qrow + (h + 1) * D + blk * 32, qn);
                    __builtin_amdgcn_sched_barrier(0);
                    float part = 0.f;
#pragma unroll
                    for (int e = 0; e < 32; ++e)
                        part = fmaf(qc[e], kf[e], part);
                    x[h] = fmaf(ksc, part, x[h]);
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
                load_uniform<16>(q2, (qrow + blk * 32) / 2, qc);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    if (h + 1 < G)
                        load_uniform<16>(q2, (qrow + (h + 1) * D + blk * 32) / 2, qn);
                    __builtin_amdgcn_sched_barrier(0);
                    float part = 0.f;
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        part = __builtin_amdgcn_fdot2(as_half2(qc[e]), k2[e], part, false);
                    x[h] = fmaf(ksc, part, x[h]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        qc[e] = qn[e];
                }
            }
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

        // ---- V copy complete; next tile's K rows in flight during PV ----
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("" : "+v"(jn));   // keep the use of the prefetched ids here
        int j1 = j;
        if (more) {
            j1 = min((unsigned)jn, (unsigned)(N - 1));
            const uint4* kr = (const uint4*)(Kb + (long long)j1 * kq_cs);
#pragma unroll
            for (int i = 0; i < KC; ++i)
                krow[i] = kr[i];
            const uint32_t* ks = (const uint32_t*)(Ksb + (long long)j1 * ksc_cs);
#pragma unroll
            for (int w = 0; w < SW; ++w)
                ksw[w] = ks[w];
        }
        wave_lds_sync();   // p_s written; V tile landed in LDS

        // ---- PV: lane = DPL output elements, cells from LDS -------------
        const int dsc = (lane * DPL) >> 5;  // scale block of this lane's elements
#pragma unroll 4
        for (int i = 0; i < nt; ++i) {
            const float vs = half_bits_to_float(vsc_s[i * NB + dsc]);
            float vf[DPL];
            if constexpr (DPL == 4) {
                const int w = *(const int*)(v_s + i * D + lane * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    vf[e] = sbyte_to_float(w, e) * vs;
            } else if constexpr (DPL == 2) {
                const int w = (int)*(const uint16_t*)(v_s + i * D + lane * 2);
                vf[0] = sbyte_to_float(w, 0) * vs;
                vf[1] = sbyte_to_float(w, 1) * vs;
            } else {
                vf[0] = (float)v_s[i * D + lane] * vs;
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
        wave_lds_sync();   // LDS reads done before the next tile's copies
        if (!more)
            break;
        t0 = t1;
        nt = nt1;
        j = j1;
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

template <int D, int EPL, bool OUTF16>
__global__ __launch_bounds__(64 * kMergeWaves) void k_merge(const float* __restrict__ pm,
                                                            const float* __restrict__ pl,
                                                            const float* __restrict__ po,
                                                            void* __restrict__ out, int P,
                                                            long long rows,
                                                            const void* __restrict__ gate,
                                                            int gate_f16)
{
    merge_block<D, EPL, OUTF16>(blockIdx.x, pm, pl, po, out, P, rows, gate, gate_f16);
}

// ------------------------------------------------------------- launch ---

template <int G, int D>
static void launch_attend_gd(const AttnLaunch& a, hipStream_t s)
{
    const long long items = (long long)a.B * a.T * a.P;
    dim3 grid((unsigned)((items + kAttendWaves - 1) / kAttendWaves), (unsigned)a.Hkv);
#define QSA_ATTEND_ARGS                                                                      \
    a.q, a.Kq, (const uint8_t*)a.Ksc, a.Vq, (const uint8_t*)a.Vsc, a.kq_cs, a.ksc_cs, a.vq_cs, \
        a.vsc_cs, a.kq_bs, a.ksc_bs, a.vq_bs, a.vsc_bs, a.ids, a.n_sel, a.pm, a.pl, a.po, a.T, \
        a.Hq, a.P, a.cap, a.N, a.B * a.T, a.scale
    if (a.q_f16)
        k_attend<G, D, true><<<grid, 64 * kAttendWaves, 0, s>>>(QSA_ATTEND_ARGS);
    else
        k_attend<G, D, false><<<grid, 64 * kAttendWaves, 0, s>>>(QSA_ATTEND_ARGS);
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
    bool ok;
    if (a.algo == 2)  // vector fp32 kernel
        ok = (a.D == 64) ? launch_attend_d<64>(a, G, s) : launch_attend_d<256>(a, G, s);
    else
        ok = launch_attend_mma(a, s);
    if (!ok)
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int D, int EPL>
static void launch_merge_de(const AttnLaunch& a, long long rows, hipStream_t s)
{
    const long long lanes = rows * (D / EPL);
    const unsigned grid = (unsigned)((lanes + 64 * kMergeWaves - 1) / (64 * kMergeWaves));
    const int gate_f16 = a.q_f16 ? 1 : 0;
    if (a.out_f16)
        k_merge<D, EPL, true><<<grid, 64 * kMergeWaves, 0, s>>>(a.pm, a.pl, a.po, a.out, a.P, rows,
                                                               a.gate, gate_f16);
    else
        k_merge<D, EPL, false><<<grid, 64 * kMergeWaves, 0, s>>>(a.pm, a.pl, a.po, a.out, a.P,
                                                                rows, a.gate, gate_f16);
}

hipError_t launch_merge(const AttnLaunch& a, hipStream_t s)
{
    const long long rows = (long long)a.B * a.T * a.Hq;
    // Many chunks per row: one element per lane (four times the waves).
    const bool wide = a.P >= 32;
    if (a.D == 64) {
        if (wide)
            launch_merge_de<64, 1>(a, rows, s);
        else
            launch_merge_de<64, 4>(a, rows, s);
    } else {
        if (wide)
            launch_merge_de<256, 1>(a, rows, s);
        else
            launch_merge_de<256, 4>(a, rows, s);
    }
    return hipGetLastError();
}

}  // namespace qsa
