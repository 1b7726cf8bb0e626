// qsa_attend_mma.h -- the matrix-core attention partials as a device
// function of one (virtual) workgroup, so that the standalone kernel and the
// single-launch decode window run the same code (gfx950,
// v_mfma_f32_16x16x32_f16).
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
//   - a softmax weight times a V scale is split the same way (hi rounded
//     toward zero; lo is the exact product minus hi, formed in one mixed
//     fp32/fp16 FMA and rounded toward zero), the weight carried at 2^4
//     times its value so the lo half stays clear of the fp16 subnormal
//     range.
// Two exact power-of-two shifts keep every half finite and normal whatever
// the magnitudes: an item's fp32 query is split as q * 2^-eq with its
// largest |q| in [2^14, 2^15) (the logits are scaled back by 2^eq), and a
// tile's weight x scale operands carry 2^ev with the tile's largest V scale
// in [2^6, 2^7) (the accumulated output is rescaled when ev changes from
// tile to tile, and scaled back at the end).  fp16 products are exact in
// fp32, so the remaining error is fp32 accumulation order plus the 2^-22
// split residue.
//
// Mapping (one wave per (token, chunk) item, four items of one KV head per
// workgroup; a tile is 32 consecutive kept cells):
//   QK  C[h][cell] = sum_d q[h][d] K[cell][d] per 32-element scale block;
//       A = q (row h = lane%16, elements 8*(lane/16)..+7 of the block),
//       B = K codes (column = cell lane%16 of a 16-cell half, the same 8
//       elements: one 8-byte gather per lane), so each lane's accumulator
//       covers one cell and four heads and the block's K scale is that
//       lane's own scalar.
//   softmax  per head over the tile's cells: two halves in-lane, then DPP
//       rotations across the 16 lanes of a row.  The weights go to LDS as a
//       head x cell table (the operand layouts of QK and PV differ).
//   PV  O^T[d][h] = sum_cell V[cell][d] (w[h][cell] vsc[cell][d/32]); A = V
//       codes read from LDS with the transpose read ds_read_b64_tr_b8 (each
//       16-lane group gets an 8-cell x 16-element block, one column per
//       lane), B = weight x V scale for 8 cells of head lane%16.  A lane's
//       accumulator then holds head lane%16 only, so rescaling is a per-lane
//       scalar.
// Running max: m is the exact running max of the logits; the weights use a
// reference max that is moved up only when m exceeds it by more than
// kLazyMax (< ln 16), so the accumulated output is rarely rescaled.  The
// partial is brought to m once at the end (factor exp(ref - m), exactly 1
// when they are equal).
//
// Memory: the tile's V codes reach LDS by global_load_lds (no register
// round trip) laid out as [16-byte chunk][cell], so every lane copies chunks
// of its own cell and the transpose reads of a wave cover whole 256-byte
// bank rows; V scales land as a [scale pair][cell] table.  K codes of the
// next tile are gathered into registers while the current tile's PV runs.
// When the four waves of a workgroup are four chunks of one token (P a
// multiple of 4), the split query is built once into LDS and shared.
#pragma once

#include <math.h>

#include "qsa_device.h"
#include "qsa_merge.h"
#include "qsa_mma.h"

namespace qsa {


constexpr int kMmaWaves = 4;      // (token, chunk) items per workgroup

// SHQ: the four waves of the workgroup are chunks of one token and share the
// split query through LDS (requires P % 4 == 0).  With the query in LDS, or
// fp16 queries (no lo half) in registers, the kernel fits 256 registers and
// runs two waves per SIMD; fp32 queries in registers need one wave per SIMD.
//
// MERGE: the workgroup's four items are all the chunks of whole tokens (P in
// {1, 2, 4}), so instead of writing partials the workgroup merges them
// itself (with the optional output gate) and writes the output: each wave
// leaves m and l in its weight table and its o, scaled exactly as the
// partial would be, in LDS (the V tiles' space, a few heads per round), and
// the merge runs the sequence of the merge kernel on those values, so the
// output equals qsa_attend followed by qsa_merge(_gated) bit for bit.
// Every wave, also one with an empty chunk or past the last item, takes
// part in the workgroup barriers of that epilogue.
//
// MCH (with SHQ, without MERGE): one workgroup per (token, KV head) of a
// split with P a multiple of 4; wave w computes chunks w, w + 4, ..., one
// after another, writing each chunk's partial when it ends, and gathers the
// next chunk's first tile while the current chunk's last tile runs, so a
// wave's gathers never drain between chunks.  Each partial is computed with
// the same operations as in the one-chunk-per-wave mapping (bit-equal).
// With `out` set, the workgroup then merges its token's partials (read back
// from memory it wrote itself, after a workgroup barrier) with the merge
// kernel's sequence and writes the gated output.
template <int G, int D, bool QF16, bool SHQ, bool MERGE = false, bool MCH = false>
__device__ __forceinline__ void attend_mma_block(
    int wg, const void* __restrict__ q, const int8_t* __restrict__ Kq,
    const uint8_t* __restrict__ Ksc, const int8_t* __restrict__ Vq,
    const uint8_t* __restrict__ Vsc, long long kq_cs, long long ksc_cs, long long vq_cs,
    long long vsc_cs, long long kq_bs, long long ksc_bs, long long vq_bs, long long vsc_bs,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ n_sel, float* __restrict__ pm,
    float* __restrict__ pl, float* __restrict__ po, int T, int Hq, int Hkv, int P, int cap, int N,
    int BT, float scale, void* __restrict__ out = nullptr, const void* __restrict__ gate = nullptr,
    int out_f16 = 0)
{
    static_assert(G <= 16, "one 16-row head block per KV head");
    static_assert(!MCH || (SHQ && !MERGE), "several chunks per wave: shared query, partials");
    constexpr int NB = D / 32;                // scale blocks per head row
    constexpr int NT = D / 16;                // 16-element slices (= 16-byte chunks)
    constexpr int NPR = NB / 2;               // 32-bit scale words per head row
    constexpr int TC = kMmaCells;
    constexpr int VCOPIES = NT / 2;           // V copies per tile (two chunks each)
    constexpr int SROWS = NPR < 2 ? 2 : NPR;  // scale-pair rows in LDS
    constexpr int PP = 36;                    // weight table pitch (floats)
    constexpr int QH = QF16 ? 1 : 2;          // query halves kept
    __shared__ __align__(16) int8_t v_all[kMmaWaves][TC * D];
    __shared__ __align__(16) uint32_t vsc_all[kMmaWaves][SROWS * TC];
    __shared__ __align__(16) float p_all[kMmaWaves][16 * PP];
    __shared__ __align__(16) half8_t q_all[SHQ ? QH * NB * 64 : 1];
    __shared__ float s_qmax[kMmaWaves];
    // MERGE with a gate: the gate rows of the workgroup's tokens (G heads of
    // D elements each, in the query dtype), copied at the start.
    constexpr int GTOK = SHQ ? 1 : kMmaWaves;   // tokens per workgroup, at most
    constexpr int GES = QF16 ? 2 : 4;           // gate element bytes
    constexpr int GBYTES = GTOK * G * D * GES;
    __shared__ __align__(16) uint8_t gate_s[MERGE ? (GBYTES + 1023) / 1024 * 1024 : 16];

    // Workgroup w serves KV head g = (w / 8) % Hkv of item group
    // (w / (8 Hkv)) * 8 + w % 8: the groups' KV heads are 8 workgroup ids
    // apart, so (workgroups being spread round-robin over the 8 XCDs) they
    // run on one XCD at about the same time and share its L2 for the cache
    // lines both heads touch (scales, ids).  The grid is padded to a
    // multiple of 8 Hkv.
    const int g = (wg >> 3) % Hkv;
    // (With MCH a group is one token.)
    const long long group = (long long)(wg / (8 * Hkv)) * 8 + (wg & 7);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long item = MCH ? group * P + wave : group * kMmaWaves + wave;
    const int lane = threadIdx.x & 63;
    const int hq = lane & 15, q4 = lane >> 4;
    if ((MCH ? group * P : group * kMmaWaves) >= (long long)BT * P)
        return;  // grid padding (whole workgroup)

    if constexpr (MERGE) {
        // Gate rows of this workgroup's tokens into LDS, 16 bytes a lane,
        // by direct copies that complete during the first tile (every wave
        // waits for them before the epilogue reads them).
        if (gate) {
            constexpr int UPT = G * D * GES / 16;  // 16-byte units per token
            const long long bt0 = group * kMmaWaves / P;
            const int ntok = (int)min((long long)(kMmaWaves / P), (long long)BT - bt0);
            const int units = ntok * UPT;
            for (int u0 = wave * 64; u0 < units; u0 += 64 * kMmaWaves) {
                const int u = u0 + lane;
                if (u < units) {
                    const int tl = u / UPT, w = u % UPT;
                    const char* src = (const char*)gate +
                                      (((bt0 + tl) * Hq + (long long)g * G) * D) * GES + 16 * w;
                    __builtin_amdgcn_global_load_lds((const void*)src,
                                                     (lds_void_t*)(gate_s + 16 * u0), 16, 0, 0);
                }
            }
        }
    }

    const bool live = item < (long long)BT * P;
    if constexpr (!MERGE && !SHQ) {
        if (!live)
            return;
    }
    const int bt = live ? (int)(item / P) : 0;
    int c = live ? (int)(item % P) : 0;
    int8_t* v_s = v_all[wave];
    uint32_t* vsc_s = vsc_all[wave];
    float* p_s = p_all[wave];
    const int b = bt / T;
    const size_t prow = (size_t)bt * Hq + (size_t)g * G;  // row of head g*G

    const int ns = live ? min(n_sel[bt], cap) : 0;
    const int S = (ns + P - 1) / P;
    int beg = c * S;
    int end = min(beg + S, ns);

    // Partial of an empty chunk cc: (-inf, 0, 0).
    auto write_empty = [&](int cc) {
        if (lane < G) {
            pm[(prow + lane) * P + cc] = -INFINITY;
            pl[(prow + lane) * P + cc] = 0.f;
        }
        for (int i = lane; i < G * D / 4; i += 64) {
            const int h = i / (D / 4), e = i % (D / 4);
            *(float4*)(po + ((prow + h) * P + cc) * D + 4 * e) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };

    const char* Kb = (const char*)Kq + (long long)b * kq_bs + (long long)g * D + 8 * q4;
    const char* Ksb = (const char*)Ksc + (long long)b * ksc_bs + (long long)g * NB * 2;
    const char* Vb = (const char*)Vq + (long long)b * vq_bs + (long long)g * D + 16 * (lane >> 5);
    const char* Vsb = (const char*)Vsc + (long long)b * vsc_bs + (long long)g * NB * 2;
    const int32_t* idr = ids + (size_t)bt * cap;

    // Tile cell ids: jv for the V copy (cell lane & 31), ja / jb for the K
    // gathers (cells hq and 16 + hq).  Ids outside [0, N) are undefined
    // input; clamping keeps every gather inside the cache.  Tail cells
    // repeat the tile's first cell (their weights are zero).
    const int cl = lane & 31;
    auto tile_ids = [&](int t0, int nt, int& jv, int& ja, int& jb) {
        jv = idr[t0 + (cl < nt ? cl : 0)];
        ja = idr[t0 + (hq < nt ? hq : 0)];
        jb = idr[t0 + (16 + hq < nt ? 16 + hq : 0)];
    };
    auto clampN = [&](int j) { return (int)min((unsigned)j, (unsigned)(N - 1)); };

    uint2 kc[2][NB];
    uint32_t ksw[2][NPR];
    auto load_k = [&](int ja, int jb) {
        const char* kr[2] = {Kb + (long long)ja * kq_cs, Kb + (long long)jb * kq_cs};
        const char* sr[2] = {Ksb + (long long)ja * ksc_cs, Ksb + (long long)jb * ksc_cs};
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
                kc[hf][blk] = *(const uint2*)(kr[hf] + 32 * blk);
            if constexpr (NPR == 4) {
                const uint4 w = *(const uint4*)sr[hf];
                ksw[hf][0] = w.x;
                ksw[hf][1] = w.y;
                ksw[hf][2] = w.z;
                ksw[hf][3] = w.w;
            } else {
#pragma unroll
                for (int w = 0; w < NPR; ++w)
                    ksw[hf][w] = ((const uint32_t*)sr[hf])[w];
            }
        }
    };

    // The first tile's ids and K gathers go out now, so that their latency
    // overlaps the query build below.
    int t0 = beg;
    int nt = min(TC, end - t0);
    int jv = 0, ja = 0, jb = 0;
    if (beg < end) {
        tile_ids(t0, nt, jv, ja, jb);
        jv = clampN(jv);
        load_k(clampN(ja), clampN(jb));
    }

    int eq = 0;  // fp32 queries are split as q * 2^-eq (see the header)
    if constexpr (SHQ) {
        // Every wave of the block has the same token (P % 4 == 0 and the grid
        // covers whole blocks of items); each builds some query blocks.
        const int bt0 = (int)(MCH ? group : (group * kMmaWaves) / P);
        const size_t prow0 = (size_t)bt0 * Hq + (size_t)g * G;
        if constexpr (!QF16) {
            float amax = 0.f;
            for (int blk = wave; blk < NB; blk += kMmaWaves)
                amax = fmaxf(amax, q_block_absmax<G, D>(q, prow0, hq, q4, blk));
            amax = wave_max16x4(amax);
            if (lane == 0)
                s_qmax[wave] = amax;
            __syncthreads();
            amax = fmaxf(fmaxf(s_qmax[0], s_qmax[1]), fmaxf(s_qmax[2], s_qmax[3]));
            eq = pow2_shift(amax, kQShiftLo);
        }
        for (int blk = wave; blk < NB; blk += kMmaWaves) {
            half8_t hi, lo;
            load_q_block<G, D, QF16>(q, prow0, hq, q4, blk, eq, hi, lo);
            q_all[(QH * blk) * 64 + lane] = hi;
            if constexpr (!QF16)
                q_all[(QH * blk + 1) * 64 + lane] = lo;
        }
        __syncthreads();
    }
    if constexpr (!MERGE && SHQ) {
        if (!live)
            return;
    }
    if (!MERGE && !MCH && beg >= end) {
        write_empty(c);
        return;
    }

    float m_run[4], m_ref[4], l_run[4];  // heads 4*q4 + r
    float4_t o[NT];                      // O^T: head hq, elements 16*t + 4*q4 + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m_run[r] = -INFINITY;
        m_ref[r] = -INFINITY;
        l_run[r] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
        o[t] = float4_t{0.f, 0.f, 0.f, 0.f};
    int ev = 0;  // the accumulated output carries 2^ev (see the header)

    // Partial of chunk cc: m, and l, o brought from the reference max to m.
    auto write_partial = [&](int cc) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = 4 * q4 + r;
            const float f = __builtin_amdgcn_exp2f((m_ref[r] - m_run[r]) * kLog2e);
            if (hq == 0) {
                p_s[h * PP + 33] = f;
                if (h < G) {
                    pm[(prow + h) * P + cc] = m_run[r];
                    pl[(prow + h) * P + cc] = l_run[r] * f;
                }
            }
        }
        wave_lds_sync();
        if (hq < G) {
            const float f = __builtin_amdgcn_ldexpf(p_s[hq * PP + 33] * (1.f / kWScale), -ev);
            float* dst = po + ((prow + hq) * P + cc) * D + 4 * q4;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float4_t v = o[t] * f;
                *(float4*)(dst + 16 * t) = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    };

    if (beg < end) {  // always true here without MERGE or MCH
    half8_t qh[SHQ ? 1 : NB], ql[SHQ ? 1 : NB];
    if constexpr (!SHQ) {
        if constexpr (!QF16) {
            float amax = 0.f;
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
                amax = fmaxf(amax, q_block_absmax<G, D>(q, prow, hq, q4, blk));
            eq = pow2_shift(wave_max16x4(amax), kQShiftLo);
        }
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
            load_q_block<G, D, QF16>(q, prow, hq, q4, blk, eq, qh[blk], ql[blk]);
    }
    const float scale_q = __builtin_amdgcn_ldexpf(scale, eq);  // logit scale of the split query
    // Transpose-read base of this lane: cell 8*q4 + hq/2 of the [chunk][cell]
    // table, 8-byte half hq&1; slice t adds 512*t.
    const int8_t* v_rd = v_s + 16 * (8 * q4 + (hq >> 1)) + 8 * (hq & 1);

#pragma unroll 1
    for (;;) {
        // Next tile: the next one of this chunk or (MCH) the first one of the
        // wave's next chunk, if that chunk has cells.
        int t1 = t0 + TC, end1 = end;
        bool more = t1 < end;
        if constexpr (MCH) {
            const int cn = c + kMmaWaves;
            if (!more && cn < P && cn * S < ns) {
                more = true;
                t1 = cn * S;
                end1 = min(t1 + S, ns);
            }
        }
        const int nt1 = more ? min(TC, end1 - t1) : 0;
        int jvn = 0, jan = 0, jbn = 0;
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
        // ---- V codes and scales of the tile into LDS ---------------------
        // Copy i: lane L takes chunk 2i + L/32 of cell L%32, landing at
        // 16 * (32 * chunk + cell); scale copy i: pair 2i + L/32 at word
        // 32 * pair + cell.
        {
            const char* vr = Vb + (long long)jv * vq_cs;
#pragma unroll
            for (int i = 0; i < VCOPIES; ++i)
                __builtin_amdgcn_global_load_lds((const void*)(vr + 32 * i),
                                                 (lds_void_t*)(v_s + i * 1024), 16, 0, 0);
            const char* sr = Vsb + (long long)jv * vsc_cs;
#pragma unroll
            for (int i = 0; i < SROWS / 2; ++i) {
                const int pr = min(2 * i + (lane >> 5), NPR - 1);
                __builtin_amdgcn_global_load_lds((const void*)(sr + 4 * pr),
                                                 (lds_void_t*)(vsc_s + i * 64), 4, 0, 0);
            }
        }
        if (more)
            tile_ids(t1, nt1, jvn, jan, jbn);

        // ---- QK on the matrix cores (both 16-cell halves per block) -----
        float4_t s[2] = {float4_t{0.f, 0.f, 0.f, 0.f}, float4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            half8_t qa, qb;
            if constexpr (SHQ) {
                qa = q_all[(QH * blk) * 64 + lane];
                if constexpr (!QF16)
                    qb = q_all[(QH * blk + 1) * 64 + lane];
            } else {
                qa = qh[blk];
                qb = ql[blk];
            }
            const half8_t k0 = codes_to_half8(kc[0][blk].x, kc[0][blk].y);
            const half8_t k1 = codes_to_half8(kc[1][blk].x, kc[1][blk].y);
            float4_t p0 = mfma16(qa, k0, float4_t{0.f, 0.f, 0.f, 0.f});
            float4_t p1 = mfma16(qa, k1, float4_t{0.f, 0.f, 0.f, 0.f});
            if constexpr (!QF16) {
                p0 = mfma16(qb, k0, p0);
                p1 = mfma16(qb, k1, p1);
            }
            const float ks0 = half_of(ksw[0][blk >> 1], blk & 1);
            const float ks1 = half_of(ksw[1][blk >> 1], blk & 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s[0][r] = fmaf(ks0, p0[r], s[0][r]);
                s[1][r] = fmaf(ks1, p1[r], s[1][r]);
            }
        }

        // ---- softmax over the tile ---------------------------------------
        {
            const bool v0 = hq < nt, v1 = 16 + hq < nt;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x0 = v0 ? s[0][r] * scale_q : -INFINITY;
                const float x1 = v1 ? s[1][r] * scale_q : -INFINITY;
                m_run[r] = fmaxf(m_run[r], row16_max(fmaxf(x0, x1)));
                // Move the reference max only when the running max exceeds
                // it by more than kLazyMax (always on the first tile).
                const bool move = m_run[r] > m_ref[r] + kLazyMax;
                const float alpha =
                    move ? __builtin_amdgcn_exp2f((m_ref[r] - m_run[r]) * kLog2e) : 1.f;
                m_ref[r] = move ? m_run[r] : m_ref[r];
                const float w0 = __builtin_amdgcn_exp2f((x0 - m_ref[r]) * kLog2e);
                const float w1 = __builtin_amdgcn_exp2f((x1 - m_ref[r]) * kLog2e);
                l_run[r] = fmaf(l_run[r], alpha, row16_sum(w0 + w1));
                float* prow_s = p_s + (4 * q4 + r) * PP;
                prow_s[hq] = w0 * kWScale;
                prow_s[16 + hq] = w1 * kWScale;
                if (hq == 0)
                    prow_s[32] = alpha;
            }
        }

        // ---- V copy complete; next tile's K in flight during PV ----------
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("" : "+v"(jvn), "+v"(jan), "+v"(jbn));
        if (more) {
            jvn = clampN(jvn);
            load_k(clampN(jan), clampN(jbn));
        }
        wave_lds_sync();  // weight table written; V tile landed in LDS

        // ---- PV on the matrix cores: O^T[d][h] += V^T[d][cell] W[cell][h] --
        {
            // Shift of this tile from its largest V scale (tail cells repeat
            // the first cell, so they do not change the max).
            uint32_t smax = 0;
#pragma unroll
            for (int i = 0; i < SROWS * TC / 64; ++i) {
                const uint32_t w = vsc_s[64 * i + lane];
                smax = max(smax, max(w & 0x7fffu, (w >> 16) & 0x7fffu));
            }
            const float vmax = wave_max16x4(half_bits_to_float((uint16_t)smax));
            const int ev_t = vmax > 0.f ? -pow2_shift(vmax, kVShiftLo) : ev;
            const int dev = (t0 == beg) ? 0 : ev_t - ev;
            ev = ev_t;
            const float* pr_s = p_s + hq * PP;
            const float4 pa = *(const float4*)(pr_s + 8 * q4);
            const float4 pb = *(const float4*)(pr_s + 8 * q4 + 4);
            const float alpha = __builtin_amdgcn_ldexpf(pr_s[32], dev);
            if (t0 != beg && __ballot(alpha != 1.f)) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    o[t] *= alpha;
            }
            float pw[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pw[e] = __builtin_amdgcn_ldexpf(pw[e], ev);
#pragma unroll
            for (int pr = 0; pr < NPR; ++pr) {
                const uint4 sa = *(const uint4*)(vsc_s + pr * TC + 8 * q4);
                const uint4 sb = *(const uint4*)(vsc_s + pr * TC + 8 * q4 + 4);
                const uint32_t sw[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
                int2v_t raw[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    raw[u] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (lds_int2v_t*)(v_rd + 512 * (4 * pr + u)));
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    half8_t whi, wlo;
                    if (hb)
                        split8_prod<1>(pw, sw, whi, wlo);
                    else
                        split8_prod<0>(pw, sw, whi, wlo);
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int t = 4 * pr + 2 * hb + u;  // slice of scale block 2*pr + hb
                        const int2v_t rw = raw[2 * hb + u];
                        const half8_t va = codes_to_half8((uint32_t)rw.x, (uint32_t)rw.y);
                        o[t] = mfma16(va, whi, o[t]);
                        o[t] = mfma16(va, wlo, o[t]);
                    }
                }
            }
        }
        wave_lds_sync();  // LDS reads done before the next tile's copies
        if constexpr (MCH) {
            if (t0 + TC >= end) {  // the chunk is done: its partial, then a fresh state
                write_partial(c);
                if (more) {
                    c += kMmaWaves;
                    beg = t1;
                    end = end1;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        m_run[r] = -INFINITY;
                        m_ref[r] = -INFINITY;
                        l_run[r] = 0.f;
                    }
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        o[t] = float4_t{0.f, 0.f, 0.f, 0.f};
                    ev = 0;
                }
            }
        }
        if (!more)
            break;
        t0 = t1;
        nt = nt1;
        jv = jvn;
    }

    }  // beg < end

    if constexpr (MCH) {
        // The wave's chunks after its last one with cells are empty (chunks
        // with cells form a prefix), as are all of them if the first is.
        for (int cc = (beg < end) ? c + kMmaWaves : c; cc < P; cc += kMmaWaves)
            write_empty(cc);
        if (out) {
            // Merge the token's P partials of this KV head's G query heads.
            __syncthreads();  // the partial stores of every wave are visible
            for (int i = threadIdx.x; i < G * (D / 4); i += 64 * kMmaWaves) {
                const int h = i / (D / 4), d4 = i % (D / 4);
                const size_t row = prow + h;
                float res[4];
                merge_elems<4>(pm + row * P, pl + row * P, 1, po + row * P * D + 4 * d4, D, P,
                               res);
                const long long off = (long long)row * D + 4 * d4;
                if (out_f16)
                    gate_store<4, true>(res, gate, QF16 ? 1 : 0, off, out, off);
                else
                    gate_store<4, false>(res, gate, QF16 ? 1 : 0, off, out, off);
            }
        }
    } else if constexpr (!MERGE) {
        write_partial(c);
    } else {
        // ---- fused merge: the same partial values, merged in LDS ------------
        // m and l of head h at slots 34 and 35 of row h of the wave's weight
        // table; o (scaled as the partial) stays in registers until staged.
        if (beg < end) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = 4 * q4 + r;
                const float f = __builtin_amdgcn_exp2f((m_ref[r] - m_run[r]) * kLog2e);
                if (hq == 0) {
                    p_s[h * PP + 33] = f;
                    p_s[h * PP + 34] = m_run[r];
                    p_s[h * PP + 35] = l_run[r] * f;
                }
            }
            wave_lds_sync();
            const float f = __builtin_amdgcn_ldexpf(p_s[hq * PP + 33] * (1.f / kWScale), -ev);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                o[t] = o[t] * f;
        } else {  // empty chunk or no item: m = -inf, l = 0, o = 0
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (hq == 0) {
                    p_s[(4 * q4 + r) * PP + 34] = -INFINITY;
                    p_s[(4 * q4 + r) * PP + 35] = 0.f;
                }
            }
        }
        // Stage: [wave][head of the round][D + 4] floats over the V tiles
        // (the pad spreads a wave's 16 head rows over the LDS banks).
        constexpr int SP = D + 4;
        constexpr int HR = (int)(sizeof(v_all) / (kMmaWaves * SP * sizeof(float)));
        static_assert(HR >= 1, "stage holds at least one head per round");
        float* stage = (float*)&v_all[0][0];
        const int ntok = kMmaWaves / P;                    // tokens of this workgroup
        const long long bt0 = group * kMmaWaves / P;       // its first token
        // Every wave is out of its tile loop (the V tiles are free) and its
        // gate copies have landed.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
#pragma unroll 1
        for (int h0 = 0; h0 < G; h0 += HR) {
            const int hr = min(HR, G - h0);
            if (hq >= h0 && hq < h0 + hr) {
                float* dst = stage + (wave * HR + (hq - h0)) * SP + 4 * q4;
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    *(float4_t*)(dst + 16 * t) = o[t];
            }
            __syncthreads();
            const int n4 = ntok * hr * (D / 4);
            for (int i = threadIdx.x; i < n4; i += 64 * kMmaWaves) {
                const int d4 = i % (D / 4);
                const int hl = (i / (D / 4)) % hr;
                const int tl = i / ((D / 4) * hr);
                const long long tok = bt0 + tl;
                if (tok >= BT)
                    continue;
                const int h = h0 + hl;
                const int w0 = tl * P;  // wave of chunk 0 of this token
                float res[4];
                merge_elems<4>(&p_all[w0][h * PP + 34], &p_all[w0][h * PP + 35], 16 * PP,
                               stage + (w0 * HR + hl) * SP + 4 * d4, (long long)HR * SP, P, res);
                const long long off = (tok * Hq + (long long)g * G + h) * D + 4 * d4;
                const void* gs = gate ? (const void*)gate_s : nullptr;
                const long long goff = ((long long)tl * G + h) * D + 4 * d4;
                if (out_f16)
                    gate_store<4, true>(res, gs, QF16 ? 1 : 0, goff, out, off);
                else
                    gate_store<4, false>(res, gs, QF16 ? 1 : 0, goff, out, off);
            }
            __syncthreads();  // stage read before the next round overwrites it
        }
    }
}

}  // namespace qsa
