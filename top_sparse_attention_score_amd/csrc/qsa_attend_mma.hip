// qsa_attend_mma.hip -- split-KV attention partials on the gfx950 matrix
// cores (v_mfma_f32_16x16x32_f16).
//
// Same contract as the vector kernel in qsa_attend.hip ("opus r20 track A:
// MTP map mlock + qsa_attn / qsa_merge decode tweaks", section 2
// "qsa.metal", qsa_attn): for one (token, chunk, KV head) it produces, per
// query head, the max logit m, the sum l of exp(logit - m) and the
// unnormalised sum o of exp(logit - m) * V over the chunk's kept cells, with
// K and V read as int8 codes times an fp16 scale per 32 elements (section 3).
//
// Both products are dense contractions of a 16-row head block against 32
// cells, so they run on the matrix cores; the fp32 arithmetic of the
// definition is kept by exact fp16 operands:
//   - an int8 code is exact in fp16;
//   - an fp32 query element x is split as hi = fp16(x), lo = fp16(x - hi),
//     so hi + lo carries 22 significant bits, and each product is issued
//     twice (hi, then lo) into the same fp32 accumulator;
//   - a softmax weight times a V scale is split the same way (rounding toward
//     zero for hi, so x - hi is exact), carried at 2^8 times its value so the
//     lo half stays clear of the fp16 subnormal range.
// fp16 products are exact in fp32, so the remaining error is fp32
// accumulation order plus the 2^-22 split residue.
//
// Mapping (one wave per (token, chunk) item, four items per workgroup, KV
// head = blockIdx.y; a tile is 32 consecutive kept cells):
//   QK  C[h][cell] = sum_d q[h][d] K[cell][d] per 32-element scale block;
//       A = q (row h = lane%16, elements 8*(lane/16)..+7 of the block, held
//       in registers for the whole chunk), B = K codes (column = cell
//       lane%16 of a 16-cell half, the same 8 elements, one 8-byte gather per
//       lane), so each lane's accumulator covers one cell and four heads and
//       the block's K scale is that lane's own scalar.
//   softmax  per head over the tile's cells: two halves in-lane, then DPP
//       rotations across the 16 lanes of a row.  Weights go to LDS as a
//       head x cell table (the operand layouts of QK and PV differ).
//   PV  O^T[d][h] = sum_cell V[cell][d] (p[h][cell] vsc[cell][d/32]); A = V
//       codes read from LDS with the transpose read ds_read_b64_tr_b8 (each
//       16-lane group gets an 8-cell x 16-element block, one column per
//       lane), B = weights x V scale for 8 cells of head lane%16.  The
//       accumulator of a lane then holds head lane%16 only, so the running
//       rescale is a per-lane scalar.
// V codes reach LDS with global_load_lds (no register round trip) in rows
// padded by one 16-byte chunk, so the transpose reads of 8 cells hit
// distinct banks; V scales land as a [scale pair][cell] table.
#include <math.h>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef int int2v_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) int2v_t lds_int2v_t;

constexpr int kMmaWaves = 4;     // (token, chunk) items per workgroup
constexpr int kMmaCells = 32;    // cells per tile
constexpr float kWScale = 256.f; // weights are carried at 2^8 times their value
#ifndef QSA_MMA_MIN_WAVES
#define QSA_MMA_MIN_WAVES 1      // waves per SIMD the register budget is sized for
#endif

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

// Splits eight fp32 values into fp16 hi (round toward zero) and lo = x - hi.
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

// LDS layout of a tile's V codes: cell rows of D bytes at a pitch of D + 16
// (one pad chunk per row).  The transpose read of one 16-lane group touches
// 8 consecutive cells at the same 16-byte column chunk; with the odd pitch
// (in 16-byte units) those 8 chunks, and the next group's 8, fall on
// distinct banks, and every column chunk is an immediate offset from one
// per-lane base address.
template <int D>
struct VTile {
    static constexpr int kChunks = D / 16;                          // per row
    static constexpr int kSlots = kChunks + 1;                      // per row, with pad
    static constexpr int kCopies = (kMmaCells * kSlots + 63) / 64;  // 1 KB copies
    static constexpr int kBytes = kCopies * 1024;
};

// Copies the tile's V codes (padded rows) and V scales ([pair][64 lanes]
// words; lanes 32..63 repeat cells 0..31) into LDS.  `j` is this lane's cell
// id (lane & 31 names the tile cell).  Copy i fills LDS slots 64*i..64*i+63
// (16 bytes each, slot = lane); a pad slot, or a slot past the last row,
// receives a harmless valid chunk.
template <int D>
__device__ __forceinline__ void dma_v_tile_mma(const char* Vb, long long vq_cs, const char* Vsb,
                                               long long vsc_cs, int j, int8_t* v_s,
                                               uint32_t* vsc_s)
{
    using L = VTile<D>;
    constexpr int NPR = D / 64;  // 32-bit scale words per head row
    // Re-derived per tile (empty asm): the per-copy cells and chunks are
    // recomputed here instead of being held in registers across the loop.
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int i = 0; i < L::kCopies; ++i) {
        const int slot = 64 * i + lane;
        int cell = slot / L::kSlots;
        int chunk = slot - cell * L::kSlots;
        if (cell >= kMmaCells)
            cell = 0;
        if (chunk >= L::kChunks)
            chunk = 0;
        const int jj = __shfl(j, cell, 64);
        const char* src = Vb + (long long)jj * vq_cs + chunk * 16;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(v_s + i * 1024), 16, 0,
                                         0);
    }
    const char* ssrc = Vsb + (long long)j * vsc_cs;
#pragma unroll
    for (int pr = 0; pr < NPR; ++pr)
        __builtin_amdgcn_global_load_lds((const void*)(ssrc + 4 * pr), (lds_void_t*)(vsc_s + pr * 64),
                                         4, 0, 0);
}

template <int G, int D, bool QF16>
__global__ __launch_bounds__(64 * kMmaWaves, QSA_MMA_MIN_WAVES) void k_attend_mma(
    const void* __restrict__ q, const int8_t* __restrict__ Kq, const uint8_t* __restrict__ Ksc,
    const int8_t* __restrict__ Vq, const uint8_t* __restrict__ Vsc, long long kq_cs,
    long long ksc_cs, long long vq_cs, long long vsc_cs, long long kq_bs, long long ksc_bs,
    long long vq_bs, long long vsc_bs, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ n_sel, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ po, int T, int Hq, int P, int cap, int N, int BT, float scale)
{
    static_assert(G <= 16, "one 16-row head block per KV head");
    constexpr int NB = D / 32;   // scale blocks per head row
    constexpr int NT = D / 16;   // 16-element slices of the head dimension
    constexpr int NPR = NB / 2;  // 32-bit scale words (block pairs) per head row
    constexpr int TC = kMmaCells;
    constexpr int PP = 36;       // weight table pitch (floats): 32 cells, alpha, pad
    __shared__ __align__(16) int8_t v_all[kMmaWaves][VTile<D>::kBytes];
    __shared__ __align__(16) uint32_t vsc_all[kMmaWaves][NPR * 64];
    __shared__ __align__(16) float p_all[kMmaWaves][16 * PP];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long item = (long long)blockIdx.x * kMmaWaves + wave;
    if (item >= (long long)BT * P)
        return;
    const int bt = (int)(item / P), c = (int)(item % P), g = blockIdx.y;
    int8_t* v_s = v_all[wave];
    uint32_t* vsc_s = vsc_all[wave];
    float* p_s = p_all[wave];
    const int b = bt / T;
    const int lane = threadIdx.x & 63;
    const int hq = lane & 15, q4 = lane >> 4;
    const size_t prow = (size_t)bt * Hq + (size_t)g * G;  // row of head g*G

    const int ns = min(n_sel[bt], cap);
    const int S = (ns + P - 1) / P;
    const int beg = c * S;
    const int end = min(beg + S, ns);

    if (beg >= end) {
        if (lane < G) {
            pm[(prow + lane) * P + c] = -INFINITY;
            pl[(prow + lane) * P + c] = 0.f;
        }
        for (int i = lane; i < G * D / 4; i += 64) {
            const int h = i / (D / 4), e = i % (D / 4);
            *(float4*)(po + ((prow + h) * P + c) * D + 4 * e) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        return;
    }

    // ---- query operand: head hq, elements 32*blk + 8*q4 .. +7 ------------
    half8_t qh[NB], ql[NB];
    {
        const bool hv = hq < G;
        const size_t qoff = (prow + (hv ? hq : 0)) * D + 8 * q4;
        if constexpr (QF16) {
            const half8_t* qr = (const half8_t*)((const _Float16*)q + qoff);
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                const half8_t v = qr[4 * blk];
                qh[blk] = hv ? v : half8_t{};
                ql[blk] = half8_t{};
            }
        } else {
            const float4* qr = (const float4*)((const float*)q + qoff);
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                const float4 a = qr[8 * blk], bq = qr[8 * blk + 1];
                const float x[8] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const _Float16 h = (_Float16)x[e];
                    const _Float16 l = (_Float16)(x[e] - (float)h);
                    qh[blk][e] = hv ? h : (_Float16)0.f;
                    ql[blk][e] = hv ? l : (_Float16)0.f;
                }
            }
        }
    }

    const char* Kb = (const char*)Kq + (long long)b * kq_bs + (long long)g * D;
    const char* Ksb = (const char*)Ksc + (long long)b * ksc_bs + (long long)g * NB * 2;
    const char* Vb = (const char*)Vq + (long long)b * vq_bs + (long long)g * D;
    const char* Vsb = (const char*)Vsc + (long long)b * vsc_bs + (long long)g * NB * 2;
    const int32_t* idr = ids + (size_t)bt * cap;

    // K codes and scales of a tile: lane holds cell 16*half + hq, bytes
    // 32*blk + 8*q4 .. +7 of its row, and the cell's NB scales.
    uint2 kc[2][NB];
    uint32_t ksw[2][NPR];
    auto load_k = [&](int jt) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int jc = __shfl(jt, 16 * hf + hq, 64);
            const char* kr = Kb + (long long)jc * kq_cs + 8 * q4;
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
                kc[hf][blk] = *(const uint2*)(kr + 32 * blk);
            const uint32_t* sr = (const uint32_t*)(Ksb + (long long)jc * ksc_cs);
            if constexpr (NPR == 4) {
                const uint4 w = *(const uint4*)sr;
                ksw[hf][0] = w.x;
                ksw[hf][1] = w.y;
                ksw[hf][2] = w.z;
                ksw[hf][3] = w.w;
            } else {
#pragma unroll
                for (int w = 0; w < NPR; ++w)
                    ksw[hf][w] = sr[w];
            }
        }
    };

    float m_run[4], l_run[4];  // heads 4*q4 + r
    float4_t o[NT];            // O^T: head hq, elements 16*nt + 4*q4 + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m_run[r] = -INFINITY;
        l_run[r] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
        o[t] = float4_t{0.f, 0.f, 0.f, 0.f};

    // Lane & 31 names the tile cell for gathers; ids outside [0, N) are
    // undefined input, clamping keeps every gather inside the cache; tail
    // cells repeat the tile's first cell (their weights are zero).
    const int cl = lane & 31;
    int t0 = beg;
    int nt = min(TC, end - t0);
    int j = min((unsigned)idr[t0 + (cl < nt ? cl : 0)], (unsigned)(N - 1));
    load_k(j);

    // Transpose-read base of this lane: row of tile cell 8*q4 + hq/2, 8-byte
    // half hq&1 (16-lane group q4 reads cells 8*q4 .. 8*q4+7).
    const int8_t* v_rd = v_s + (8 * q4 + (hq >> 1)) * (VTile<D>::kSlots * 16) + 8 * (hq & 1);

#pragma unroll 1
    for (;;) {
        const int t1 = t0 + TC;
        const bool more = t1 < end;
        const int nt1 = more ? min(TC, end - t1) : 0;
        int jn = 0;
        // The K registers were loaded during the previous PV phase; settle
        // them first so the V copy below overlaps the whole QK phase.
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
                asm volatile("" : "+v"(kc[hf][blk].x), "+v"(kc[hf][blk].y));
#pragma unroll
            for (int w = 0; w < NPR; ++w)
                asm volatile("" : "+v"(ksw[hf][w]));
        }
        dma_v_tile_mma<D>(Vb, vq_cs, Vsb, vsc_cs, j, v_s, vsc_s);
        if (more)
            jn = idr[t1 + (cl < nt1 ? cl : 0)];

        // ---- QK on the matrix cores (both 16-cell halves per block) -----
        float4_t s[2] = {float4_t{0.f, 0.f, 0.f, 0.f}, float4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const half8_t k0 = codes_to_half8(kc[0][blk].x, kc[0][blk].y);
            const half8_t k1 = codes_to_half8(kc[1][blk].x, kc[1][blk].y);
            float4_t p0 = mfma16(qh[blk], k0, float4_t{0.f, 0.f, 0.f, 0.f});
            float4_t p1 = mfma16(qh[blk], k1, float4_t{0.f, 0.f, 0.f, 0.f});
            if constexpr (!QF16) {
                p0 = mfma16(ql[blk], k0, p0);
                p1 = mfma16(ql[blk], k1, p1);
            }
            const float ks0 = half_of(ksw[0][blk >> 1], blk & 1);
            const float ks1 = half_of(ksw[1][blk >> 1], blk & 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s[0][r] = fmaf(ks0, p0[r], s[0][r]);
                s[1][r] = fmaf(ks1, p1[r], s[1][r]);
            }
            // At most two blocks in flight: bounds the live partials and
            // converted operands (the scheduler would otherwise hoist all).
            if (blk & 1)
                __builtin_amdgcn_sched_barrier(0);
        }

        // ---- softmax over the tile, folded into the running pair ---------
        {
            const bool v0 = hq < nt, v1 = 16 + hq < nt;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x0 = v0 ? s[0][r] * scale : -INFINITY;
                const float x1 = v1 ? s[1][r] * scale : -INFINITY;
                const float mn = fmaxf(m_run[r], row16_max(fmaxf(x0, x1)));
                const float alpha = __builtin_amdgcn_exp2f((m_run[r] - mn) * kLog2e);
                const float p0 = __builtin_amdgcn_exp2f((x0 - mn) * kLog2e);
                const float p1 = __builtin_amdgcn_exp2f((x1 - mn) * kLog2e);
                l_run[r] = fmaf(l_run[r], alpha, row16_sum(p0 + p1));
                m_run[r] = mn;
                float* prow_s = p_s + (4 * q4 + r) * PP;
                prow_s[hq] = p0 * kWScale;
                prow_s[16 + hq] = p1 * kWScale;
                if (hq == 0)
                    prow_s[32] = alpha;
            }
        }

        // ---- V copy complete; next tile's K in flight during PV ----------
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("" : "+v"(jn));
        int j1 = j;
        if (more) {
            j1 = min((unsigned)jn, (unsigned)(N - 1));
            load_k(j1);
        }
        wave_lds_sync();  // weight table written; V tile landed in LDS

        // ---- PV on the matrix cores: O^T[d][h] += V^T[d][cell] W[cell][h] --
        {
            const float* pr_s = p_s + hq * PP;
            const float4 pa = *(const float4*)(pr_s + 8 * q4);
            const float4 pb = *(const float4*)(pr_s + 8 * q4 + 4);
            const float alpha = pr_s[32];
            if (__ballot(alpha != 1.f)) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    o[t] *= alpha;
            }
            const float pw[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
            for (int pr = 0; pr < NPR; ++pr) {
                const uint4 sa = *(const uint4*)(vsc_s + pr * 64 + 8 * q4);
                const uint4 sb = *(const uint4*)(vsc_s + pr * 64 + 8 * q4 + 4);
                const uint32_t sw[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
                int2v_t raw[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    raw[u] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (lds_int2v_t*)(v_rd + 16 * (4 * pr + u)));
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        x[e] = pw[e] * half_of(sw[e], hb);
                    half8_t whi, wlo;
                    split8(x, whi, wlo);
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int t = 4 * pr + 2 * hb + u;  // slice of scale block 2*pr + hb
                        const int2v_t rw = raw[2 * hb + u];
                        const half8_t va = codes_to_half8((uint32_t)rw.x, (uint32_t)rw.y);
                        o[t] = mfma16(va, whi, o[t]);
                        o[t] = mfma16(va, wlo, o[t]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wave_lds_sync();  // LDS reads done before the next tile's copies
        if (!more)
            break;
        t0 = t1;
        nt = nt1;
        j = j1;
    }

    // ---- partials: m, l per head; o scaled back by 2^-8 --------------------
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * q4 + r;
        if (hq == 0 && h < G) {
            pm[(prow + h) * P + c] = m_run[r];
            pl[(prow + h) * P + c] = l_run[r];
        }
    }
    if (hq < G) {
        float* dst = po + ((prow + hq) * P + c) * D + 4 * q4;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float4_t v = o[t] * (1.f / kWScale);
            *(float4*)(dst + 16 * t) = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

template <int G, int D>
static void launch_mma_gd(const AttnLaunch& a, hipStream_t s)
{
    const long long items = (long long)a.B * a.T * a.P;
    dim3 grid((unsigned)((items + kMmaWaves - 1) / kMmaWaves), (unsigned)a.Hkv);
#define QSA_MMA_ARGS                                                                         \
    a.q, a.Kq, (const uint8_t*)a.Ksc, a.Vq, (const uint8_t*)a.Vsc, a.kq_cs, a.ksc_cs, a.vq_cs, \
        a.vsc_cs, a.kq_bs, a.ksc_bs, a.vq_bs, a.vsc_bs, a.ids, a.n_sel, a.pm, a.pl, a.po, a.T, \
        a.Hq, a.P, a.cap, a.N, a.B * a.T, a.scale
    if (a.q_f16)
        k_attend_mma<G, D, true><<<grid, 64 * kMmaWaves, 0, s>>>(QSA_MMA_ARGS);
    else
        k_attend_mma<G, D, false><<<grid, 64 * kMmaWaves, 0, s>>>(QSA_MMA_ARGS);
#undef QSA_MMA_ARGS
}

template <int D>
static bool launch_mma_d(const AttnLaunch& a, int G, hipStream_t s)
{
    switch (G) {
    case 1: launch_mma_gd<1, D>(a, s); return true;
    case 2: launch_mma_gd<2, D>(a, s); return true;
    case 4: launch_mma_gd<4, D>(a, s); return true;
    case 8: launch_mma_gd<8, D>(a, s); return true;
    case 12: launch_mma_gd<12, D>(a, s); return true;
    case 16: launch_mma_gd<16, D>(a, s); return true;
    default: return false;
    }
}

bool launch_attend_mma(const AttnLaunch& a, hipStream_t s)
{
    const int G = a.Hq / a.Hkv;
    return (a.D == 64) ? launch_mma_d<64>(a, G, s) : launch_mma_d<256>(a, G, s);
}

}  // namespace qsa
