// qsa_select.h -- device code of the index stage shared by its kernels and
// the single-launch decode window: the one-token key scan, workgroup scans
// and the 256-thread exact select ("opus r15 track A: prompt_chunk wave
// zipping, fused alpha|beta GEMM, QSA PSO pre-warm, 24 GB chunk 2048", "what
// changed" item 1: qsa_score_mm / qsa_topk).
#pragma once

#include "qsa_device.h"

namespace qsa {

constexpr int kSelThreads = 256;   // threads of the select workgroups
constexpr int kBins = 2048;        // radix histogram bins (11-bit digits)

// Sum over the LPR lanes that share a key row (LPR = 16 or 8 consecutive
// lanes).  16 lanes: DPP row rotations (every lane ends with the total);
// 8 lanes: butterfly shuffles.  Partial sums of grid-valued products are
// exact, so the order does not change the result.
template <int LPR>
__device__ __forceinline__ float row_sum(float v)
{
    if constexpr (LPR == 16) {
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));
    } else {
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1)
            v += __shfl_xor(v, o, LPR);
    }
    return v;
}

// One key row (DI fp16 = DI*2 bytes) is read by LPR = DI/8 consecutive lanes,
// 16 bytes each, so every load instruction of a wave covers 64/LPR whole,
// consecutive rows: fully coalesced.  Each lane keeps the 8 index-query
// values of its slice for all T tokens in registers.  Workgroup (bx, b)
// covers rows bx * 64 * 8 * 256 / DI .. of problem b; the first lane of each
// row calls emit(t, row, score) for every visible row and token.
constexpr int kScanSteps = 8;   // row steps in flight per thread (U)

// The key loads of workgroup bx of idx_scan_rows (rows past nvis_max repeat
// the last visible row).
template <int DI>
__device__ __forceinline__ void idx_scan_load(int bx, int b, const uint4* __restrict__ K_idx,
                                              int N, int nvis_max, uint4 (&kv)[kScanSteps])
{
    constexpr int LPR = DI / 8, RPI = 256 / LPR;
    const int sub = threadIdx.x % LPR;
    const int r0 = bx * (RPI * kScanSteps) + threadIdx.x / LPR;
#pragma unroll
    for (int u = 0; u < kScanSteps; ++u) {
        const int j = min(r0 + u * RPI, nvis_max - 1);
        kv[u] = K_idx[((size_t)b * N + j) * (DI / 8) + sub];
    }
}

// The index-query slice of this lane for tokens 0..T-1 (TT at most).
template <int DI, int TT>
__device__ __forceinline__ void idx_scan_query(int b, const uint4* __restrict__ q_idx, int T,
                                               uint4 (&qv)[TT])
{
    const int sub = threadIdx.x % (DI / 8);
#pragma unroll
    for (int t = 0; t < TT; ++t)
        qv[t] = (t < T) ? q_idx[((size_t)b * T + t) * (DI / 8) + sub] : make_uint4(0, 0, 0, 0);
}

// Scores of the rows loaded by idx_scan_load: emit(t, row, score) from the
// first lane of each visible row.
template <int DI, int TT, class Emit>
__device__ __forceinline__ void idx_scan_compute(int bx, const uint4 (&qv)[TT],
                                                 const uint4 (&kv)[kScanSteps], int T,
                                                 int nvis_max, Emit emit)
{
    constexpr int LPR = DI / 8, RPI = 256 / LPR;
    const int sub = threadIdx.x % LPR;
    const int r0 = bx * (RPI * kScanSteps) + threadIdx.x / LPR;
#pragma unroll
    for (int u = 0; u < kScanSteps; ++u) {
        const int j = r0 + u * RPI;
        const uint32_t kw[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if (t < T) {
                const uint32_t qw[4] = {qv[t].x, qv[t].y, qv[t].z, qv[t].w};
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc = __builtin_amdgcn_fdot2(as_half2(qw[e]), as_half2(kw[e]), acc, false);
                acc = row_sum<LPR>(acc);
                if (sub == 0 && j < nvis_max)
                    emit(t, j, acc);
            }
        }
    }
}

template <int DI, int TT, class Emit>
__device__ __forceinline__ void idx_scan_rows(int bx, int b, const uint4* __restrict__ q_idx,
                                              const uint4* __restrict__ K_idx, int T, int N,
                                              int nvis_max, Emit emit)
{
    uint4 qv[TT];
    idx_scan_query<DI, TT>(b, q_idx, T, qv);
    uint4 kv[kScanSteps];
    idx_scan_load<DI>(bx, b, K_idx, N, nvis_max, kv);
    idx_scan_compute<DI, TT>(bx, qv, kv, T, nvis_max, emit);
}

// Rows a workgroup of idx_scan_rows covers.
template <int DI>
constexpr int idx_scan_rows_per_block()
{
    return (256 / (DI / 8)) * kScanSteps;
}

template <int DI, int TT>
__device__ __forceinline__ void idx_scan_block(int bx, int b, const uint4* __restrict__ q_idx,
                                               const uint4* __restrict__ K_idx,
                                               uint32_t* __restrict__ keys, int T, int N,
                                               int nvis_max)
{
    idx_scan_rows<DI, TT>(bx, b, q_idx, K_idx, T, N, nvis_max, [&](int t, int j, float sc) {
        keys[((size_t)b * T + t) * N + j] = score_key(sc);
    });
}

__host__ __device__ __forceinline__ bool token_selects(int nvis, int k, int dense_max)
{
    return nvis > dense_max && nvis > k;
}

// Exclusive prefix sum over the 256 threads; `total` gets the block sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t& total,
                                                    uint32_t* s_wave)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o)
            x += y;
    }
    if (lane == 63)
        s_wave[w] = x;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kSelThreads / 64; ++i) {
        const uint32_t s = s_wave[i];
        base += (i < w) ? s : 0u;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return base + x - v;
}

// ---- 256-thread k-th largest (sample bounds, candidate lists) ----------

// Bitwise OR and AND over the workgroup (kSelThreads threads).
__device__ __forceinline__ void wg_or_and(uint32_t& o, uint32_t& a, uint32_t* s_red)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        o |= (uint32_t)__shfl_xor((int)o, m, 64);
        a &= (uint32_t)__shfl_xor((int)a, m, 64);
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_red[w] = o;
        s_red[4 + w] = a;
    }
    __syncthreads();
    o = s_red[0] | s_red[1] | s_red[2] | s_red[3];
    a = s_red[4] & s_red[5] & s_red[6] & s_red[7];
    __syncthreads();
}

// Minimum over the workgroup (kSelThreads threads); every thread gets it.
__device__ __forceinline__ float wg_min_f(float v, uint32_t* s_red)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v = fminf(v, __shfl_xor(v, m, 64));
    if ((threadIdx.x & 63) == 0)
        s_red[threadIdx.x >> 6] = __float_as_uint(v);
    __syncthreads();
    v = fminf(fminf(__uint_as_float(s_red[0]), __uint_as_float(s_red[1])),
              fminf(__uint_as_float(s_red[2]), __uint_as_float(s_red[3])));
    __syncthreads();
    return v;
}

// Bin of a descending walk over nb bins holding the r-th element, and the
// number of elements in higher bins (every thread gets both).
__device__ __forceinline__ void wg_find_bin(const uint32_t* hist, int nb, uint32_t r, uint32_t& bin,
                                            uint32_t& above, uint32_t* s_wave, uint32_t* s_pick)
{
    // Thread t owns bins [nb - per (t + 1), nb - per t), read as vectors when
    // per >= 4 (contiguous per thread: no bank conflicts), walked downwards.
    const int per = (nb + kSelThreads - 1) / kSelThreads;
    const int lo = nb - per * ((int)threadIdx.x + 1);
    uint32_t c[8];
    if (per == 8) {
        const uint4 x = *(const uint4*)(hist + lo), y = *(const uint4*)(hist + lo + 4);
        c[0] = x.x; c[1] = x.y; c[2] = x.z; c[3] = x.w;
        c[4] = y.x; c[5] = y.y; c[6] = y.z; c[7] = y.w;
    } else if (per == 4) {
        const uint4 x = *(const uint4*)(hist + lo);
        c[0] = x.x; c[1] = x.y; c[2] = x.z; c[3] = x.w;
    } else {
        for (int i = 0; i < per; ++i)
            c[i] = (lo + i >= 0) ? hist[lo + i] : 0u;
    }
    uint32_t sum = 0;
    for (int i = 0; i < per; ++i)
        sum += c[i];
    uint32_t total;
    const uint32_t ex = block_excl_scan(sum, total, s_wave);
    if (ex < r && r <= ex + sum) {
        uint32_t acc = ex;
        for (int i = per - 1; i >= 0; --i) {
            if (acc < r && r <= acc + c[i]) {
                s_pick[0] = (uint32_t)(lo + i);
                s_pick[1] = acc;
            }
            acc += c[i];
        }
    }
    __syncthreads();
    bin = s_pick[0];
    above = s_pick[1];
    __syncthreads();
}

// The r-th largest (1-based, r at most their number) of the nonzero keys the
// workgroup holds; `each(f)` calls f(key) for every key of this thread (0 =
// no key, never counted).  On return r is the number of keys equal to the
// result that rank within the r largest.  Radix digits of up to 11 bits,
// starting below the bits that all keys share, so clustered keys (all above
// a bound) spread over the bins.
template <class Each>
__device__ uint32_t wg_kth_largest(Each each, uint32_t& r, uint32_t* hist, uint32_t* s_red,
                                   uint32_t* s_wave, uint32_t* s_pick)
{
    uint32_t o = 0u, a = 0xffffffffu;
    each([&](uint32_t v) {
        if (v) {
            o |= v;
            a &= v;
        }
    });
    wg_or_and(o, a, s_red);
    const uint32_t diff = o ^ a;
    if (diff == 0u)
        return a;   // one distinct key
    int rem = 32 - __clz(diff);
    uint32_t pmask = rem == 32 ? 0u : ~((1u << rem) - 1u);
    uint32_t prefix = a & pmask;
#pragma unroll 1
    while (rem > 0) {
        const int nbits = min(11, rem);
        const int shift = rem - nbits;
        const int nb = 1 << nbits;
        for (int i = threadIdx.x; i < nb; i += kSelThreads)
            hist[i] = 0u;
        __syncthreads();
        each([&](uint32_t v) {
            if (v && (v & pmask) == prefix)
                atomicAdd(&hist[(v >> shift) & (uint32_t)(nb - 1)], 1u);
        });
        __syncthreads();
        uint32_t bin, above;
        wg_find_bin(hist, nb, r, bin, above, s_wave, s_pick);
        r -= above;
        prefix |= bin << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        rem = shift;
    }
    return prefix;
}

// Exact top-k of one row of keys in memory (`nvis` keys, 0 = absent) by one
// workgroup of kSelThreads threads: radix select over the row, then each
// thread takes a contiguous run of cells (counts, prefix sums, ordered
// writes), so the ids come out ascending and ties at the k-th key go to the
// lowest cells.  Writes k ids, -1 up to cap, and the count.
__device__ __forceinline__ void select_row_stream(const uint32_t* __restrict__ kr, int nvis, int k,
                                                  int cap, int32_t* __restrict__ out,
                                                  int32_t* __restrict__ n_out, uint32_t* hist,
                                                  uint32_t* s_red, uint32_t* s_wave,
                                                  uint32_t* s_pick)
{
    const int tid = threadIdx.x;
    uint32_t req = (uint32_t)k;
    const uint32_t tau = wg_kth_largest(
        [&](auto f) {
            for (int i = tid; i < nvis; i += kSelThreads)
                f(kr[i]);
        },
        req, hist, s_red, s_wave, s_pick);
    const int run = (nvis + kSelThreads - 1) / kSelThreads;
    const int c0 = min(tid * run, nvis), c1 = min(c0 + run, nvis);
    uint32_t gt = 0, eq = 0;
    for (int c = c0; c < c1; ++c) {
        const uint32_t u = kr[c];
        gt += u > tau ? 1u : 0u;
        eq += u == tau ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t eq_before = block_excl_scan(eq, total, s_wave);
    const uint32_t take_eq = eq_before >= req ? 0u : min(eq, req - eq_before);
    uint32_t pos = block_excl_scan(gt + take_eq, total, s_wave);
    uint32_t taken = 0;
    for (int c = c0; c < c1; ++c) {
        const uint32_t u = kr[c];
        const bool is_eq = u == tau;
        if (u > tau || (is_eq && taken < take_eq))
            out[pos++] = c;
        taken += is_eq ? 1u : 0u;
    }
    for (int i = k + tid; i < cap; i += kSelThreads)
        out[i] = -1;
    if (tid == 0)
        *n_out = k;
}

// The same selection for rows of at most kSelThreads * KPT keys, held in
// registers: thread t reads the keys of cells t*KPT .. t*KPT+KPT-1 once
// (0 past nvis), so the radix passes cost no memory traffic.  Same result as
// select_row_stream.
template <int KPT>
__device__ __forceinline__ void select_row_regs(const uint32_t* __restrict__ kr, int nvis, int k,
                                                int cap, int32_t* __restrict__ out,
                                                int32_t* __restrict__ n_out, uint32_t* hist,
                                                uint32_t* s_red, uint32_t* s_wave,
                                                uint32_t* s_pick)
{
    const int tid = threadIdx.x;
    const int c0 = tid * KPT;
    uint32_t key[KPT];
    if (c0 + KPT <= nvis && ((uintptr_t)kr & 15) == 0) {
#pragma unroll
        for (int j = 0; j < KPT; j += 4) {
            const uint4 v = *(const uint4*)(kr + c0 + j);
            key[j] = v.x;
            key[j + 1] = v.y;
            key[j + 2] = v.z;
            key[j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            key[j] = (c0 + j < nvis) ? kr[c0 + j] : 0u;
    }
    uint32_t req = (uint32_t)k;
    const uint32_t tau = wg_kth_largest(
        [&](auto f) {
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                f(key[j]);
        },
        req, hist, s_red, s_wave, s_pick);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        gt += key[j] > tau ? 1u : 0u;
        eq += key[j] == tau ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t eq_before = block_excl_scan(eq, total, s_wave);
    const uint32_t take_eq = eq_before >= req ? 0u : min(eq, req - eq_before);
    uint32_t pos = block_excl_scan(gt + take_eq, total, s_wave);
    uint32_t taken = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool is_eq = key[j] == tau;
        if (key[j] > tau || (is_eq && taken < take_eq))
            out[pos++] = c0 + j;
        taken += is_eq ? 1u : 0u;
    }
    for (int i = k + tid; i < cap; i += kSelThreads)
        out[i] = -1;
    if (tid == 0)
        *n_out = k;
}

// Every visible cell kept (kSelThreads threads): ids 0..nvis-1, then -1.
__device__ __forceinline__ void dense_row_wg(int nvis, int cap, int32_t* __restrict__ out,
                                             int32_t* __restrict__ n_out)
{
    if (threadIdx.x == 0)
        *n_out = nvis;
    for (int i = threadIdx.x; i < cap; i += kSelThreads)
        out[i] = (i < nvis) ? i : -1;
}

}  // namespace qsa
