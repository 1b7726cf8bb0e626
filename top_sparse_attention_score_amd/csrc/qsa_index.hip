// qsa_index.hip -- index scores and exact top-k selection (gfx950).
//
// Method: the indexer scores every visible cached cell against the token
// (qsa_score_mm) and keeps the top-k (qsa_topk); both run only once a token
// sees more than 2051 cells ("opus r15 track A: prompt_chunk wave zipping,
// fused alpha|beta GEMM, QSA PSO pre-warm, 24 GB chunk 2048", "what changed"
// item 1), and the kept ids fill a 2051-word row per token ("Round 5 Track C
// Report: Direct FP16 qcurh in qsa_prep + PromptGemm Dead Buffer Removal &
// Layer-Local Aliasing", section 1, Target 2).
//
// Kernels
//   k_idx_scan   one token (T = 1): streams every visible cell's fp16 key
//                row once, 16 lanes per row (coalesced), scores it with
//                v_dot2 (fp16 x fp16 products, fp32 accumulation) and sums
//                the row across its lanes with DPP.
//   k_idx_mscan  2 <= T <= 16 (draft): the same stream, scored on MFMA
//                (v_mfma_f32_16x16x32_f16, tokens padded to 16 rows), no
//                cross-lane reduction.
//   k_scan_select one token with a row of at most 16384 cells (decode):
//                scan and select fused in one workgroup per token.
//   k_idx_gemm   prompt chunk (T > 16): [T x d_idx] x [d_idx x N] on MFMA
//                (v_mfma_f32_16x16x32_f16), 64 tokens x 256 cells per wave.
//   k_sel_row    exact top-k of rows up to 65536 cells, one workgroup per
//                token, keys in registers.
//   k_sel_*      exact top-k over the score keys of longer rows, tiled over
//                the whole chip (histogram, filter + pivot, ordered write).
#include <algorithm>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

// ---------------------------------------------------------------- scan ---

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
// values of its slice for all T tokens in registers.
template <int DI, int TT>
__global__ __launch_bounds__(256) void k_idx_scan(const uint4* __restrict__ q_idx,
                                                  const uint4* __restrict__ K_idx,
                                                  uint32_t* __restrict__ keys, int T, int N,
                                                  int nvis_max)
{
    constexpr int LPR = DI / 8;           // lanes per row
    constexpr int RPI = 256 / LPR;        // rows per block-wide step
    constexpr int U = 8;                  // steps in flight per thread
    const int b = blockIdx.y;
    const int sub = threadIdx.x % LPR;
    const int r0 = blockIdx.x * (RPI * U) + threadIdx.x / LPR;

    uint4 qv[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t)
        qv[t] = (t < T) ? q_idx[((size_t)b * T + t) * (DI / 8) + sub] : make_uint4(0, 0, 0, 0);

    uint4 kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = min(r0 + u * RPI, nvis_max - 1);
        kv[u] = K_idx[((size_t)b * N + j) * (DI / 8) + sub];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
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
                    keys[((size_t)b * T + t) * N + j] = score_key(acc);
            }
        }
    }
}

// A few tokens (2 <= T <= 16) against every visible cell on the matrix
// cores: a wave takes 16 consecutive cells per group; C[token][cell] =
// sum_d q[token][d] K[cell][d] with v_mfma_f32_16x16x32_f16 (A = the T
// index queries padded to 16 rows, B = the 16 cells' keys).  The reduction
// index is permuted (the same way in both operands): at step s lane group g
// supplies elements 64*(s/2) + 16*g + 8*(s%2) .. +7, so over a step pair a
// lane reads 32 contiguous bytes and the four groups a whole 128-byte line
// of its cell.  Every lane then holds four tokens' scores of one cell, with
// no cross-lane reduction; on the seeded grid inputs fp32 accumulation is
// exact in any order.
constexpr int kMscanGroups = 2;  // 16-cell groups in flight per wave (measured: 2 beats 4 and 8)
template <int DI>
__global__ __launch_bounds__(256) void k_idx_mscan(const _Float16* __restrict__ q_idx,
                                                   const _Float16* __restrict__ K_idx,
                                                   uint32_t* __restrict__ keys, int T, int N,
                                                   int nvis_max)
{
    typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
    constexpr int KS = DI / 32;   // MFMA steps per key row
    constexpr int U = kMscanGroups;  // 16-cell groups per wave
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, q4 = lane >> 4;

    // A operand: token col (zero rows beyond T), elements 32s + 8*q4 .. +7.
    h8_t qa[KS];
#pragma unroll
    for (int st = 0; st < KS; ++st) {
        if (col < T)
            qa[st] = *(const h8_t*)(q_idx + ((size_t)b * T + col) * DI + 64 * (st >> 1) +
                                    16 * q4 + 8 * (st & 1));
        else
            qa[st] = h8_t{};
    }
    const int c0 = (blockIdx.x * 4 + wave) * (16 * U);
    h8_t kb[U][KS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = min(c0 + 16 * u + col, nvis_max - 1);
        const _Float16* kr = K_idx + ((size_t)b * N + j) * DI + 16 * q4;
#pragma unroll
        for (int st = 0; st < KS; ++st)
            kb[u][st] = *(const h8_t*)(kr + 64 * (st >> 1) + 8 * (st & 1));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < KS; ++st)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[st], kb[u][st], acc, 0, 0, 0);
        // lane holds tokens 4*q4 + r of cell c0 + 16u + col
        const int j = c0 + 16 * u + col;
        if (j < nvis_max) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * q4 + r;
                if (t < T)
                    keys[((size_t)b * T + t) * N + j] = score_key(acc[r]);
            }
        }
    }
}

// ---------------------------------------------------------------- gemm ---

// A wave keeps the index queries of 64 tokens in registers (A operands of
// v_mfma_f32_16x16x32_f16, four 16-token row blocks) and walks 8 blocks of
// 32 consecutive cells, so every key row is read once per 64 tokens and
// every query once per 256 cells.  The reduction index is permuted as in
// k_idx_mscan (lane group g supplies elements 64*(s/2) + 16*g + 8*(s%2) ..
// +7 at step s, in both operands), so a lane reads 32 contiguous bytes per
// step pair.  Result of a 16x16 block: lane l, element e holds token row
// 4*(l/16)+e and cell column l%16.  Scores are exact on the seeded grid in
// any accumulation order.
constexpr int kGemmTok = 64;    // tokens per wave
constexpr int kGemmBlocks = 8;  // 32-cell blocks per wave
template <int DI>
__global__ __launch_bounds__(256) void k_idx_gemm(const _Float16* __restrict__ q_idx,
                                                  const _Float16* __restrict__ K_idx,
                                                  uint32_t* __restrict__ keys, int T, int N,
                                                  int nvis_max)
{
    typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
    constexpr int KS = DI / 32;  // MFMA steps per row
    const int b = blockIdx.z;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;
    const int tok0 = blockIdx.y * kGemmTok;
    const int cell_base = (blockIdx.x * 4 + w) * (32 * kGemmBlocks);
    if (cell_base >= nvis_max)
        return;

    auto kofs = [&](int st) { return 64 * (st >> 1) + 16 * grp + 8 * (st & 1); };
    h8_t qa[4][KS];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = min(tok0 + 16 * i + r, T - 1);
        const _Float16* src = q_idx + ((size_t)b * T + tok) * DI;
#pragma unroll
        for (int st = 0; st < KS; ++st)
            qa[i][st] = *(const h8_t*)(src + kofs(st));
    }
#pragma unroll 1
    for (int cb = 0; cb < kGemmBlocks; ++cb) {
        const int c0 = cell_base + 32 * cb;
        if (c0 >= nvis_max)
            break;
        h8_t kb[2][KS];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int cell = min(c0 + 16 * jj + r, nvis_max - 1);
            const _Float16* src = K_idx + ((size_t)b * N + cell) * DI;
#pragma unroll
            for (int st = 0; st < KS; ++st)
                kb[jj][st] = *(const h8_t*)(src + kofs(st));
        }
        float4_t acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                acc[i][jj] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < KS; ++st)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[i][st], kb[jj][st],
                                                                        acc[i][jj], 0, 0, 0);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int cell = c0 + 16 * jj + r;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tok = tok0 + 16 * i + 4 * grp + e;
                    if (tok < T && cell < nvis_max)
                        keys[((size_t)b * T + tok) * N + cell] = score_key(acc[i][jj][e]);
                }
            }
    }
}

// -------------------------------------------------------------- select ---
//
// Exact top-k over the fp32 score keys of one token, spread over the whole
// chip.  Keys are order-preserving uint32 images of the scores; the kept set
// is every cell that is not below the pivot, the k-th cell in the total order
// (key descending, cell index ascending), so ties at the threshold go to the
// lowest indices.  A token is cut into tiles of kTile cells:
//   k_sel_hist    per tile: LDS histogram of the top 11 key bits, merged into
//                 the token's 2048-bin histogram with global atomics;
//   k_sel_filter  per tile: from that histogram the bin holding the k-th key;
//                 counts the tile's cells above that bin (all kept) and
//                 appends the cells inside it to the token's candidate list;
//   k_sel_pivot   per token: resolves the pivot with two more radix digits
//                 on the key, then on the cell index among equal keys, and
//                 turns the per-tile kept counts into output offsets;
//   k_sel_write   per tile: ordered compaction of the kept cells to their
//                 offsets, so ids come out in ascending cell order.
// Tokens that see at most max(dense_max, k) cells keep all of them.  If the
// threshold bin holds more than kCap candidates (massive exact ties), the
// pivot kernel streams the token's keys instead.  Kernel boundaries order the
// steps; no workgroup waits on another.

constexpr int kSelThreads = 256;
constexpr int kTile = 4096;                         // cells per select tile
constexpr int kPerLane = kTile / kSelThreads;       // 16 keys per thread
constexpr int kBins = 2048;
constexpr int kCap = 4096;                          // candidates per token
constexpr int kMaxTiles = 1024;                     // n_cells <= 2^22

struct SelWs {
    uint32_t* keys;      // [BT][N]
    uint32_t* hist;      // [BT][kBins]
    uint32_t* tile_def;  // [BT][NT] cells above the threshold bin, per tile
    uint32_t* tile_off;  // [BT][NT] output offset of each tile
    uint32_t* cand_n;    // [BT] candidates appended
    uint32_t* done;      // [BT] finished filter tiles
    uint32_t* cand;      // [BT][kCap][2] (key, cell)
    uint32_t* pivot;     // [BT][2] (key, cell index) of the k-th kept cell
};

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

// Given a histogram of nb bins (LDS), finds the bin b holding the r-th
// largest element (1-based) and the count of elements in higher bins.
// Every thread gets the result.
__device__ __forceinline__ void find_bin_desc(const uint32_t* hist, int nb, uint32_t r,
                                              uint32_t& bin, uint32_t& above,
                                              uint32_t* s_wave, uint32_t* s_pick)
{
    const int per = nb / kSelThreads;  // bins per thread (8 or 4)
    const int hi = nb - 1 - threadIdx.x * per;  // thread's bins: hi, hi-1, ...
    uint32_t sum = 0;
    for (int i = 0; i < per; ++i)
        sum += hist[hi - i];
    uint32_t total;
    const uint32_t ex = block_excl_scan(sum, total, s_wave);
    if (ex < r && r <= ex + sum) {
        uint32_t acc = ex;
        for (int i = 0; i < per; ++i) {
            const uint32_t c = hist[hi - i];
            if (acc < r && r <= acc + c) {
                s_pick[0] = (uint32_t)(hi - i);
                s_pick[1] = acc;
            }
            acc += c;
        }
    }
    __syncthreads();
    bin = s_pick[0];
    above = s_pick[1];
    __syncthreads();
}

// Radix select: among the values produced by get(i, v) for i < n (get returns
// false to skip), whose bits under pmask equal prefix, finds the r-th largest.
// Digits (11, 11, 10 bits) from digit `first` on.  On return prefix is the
// value and r the number of elements equal to it still to take.
template <class Get>
__device__ void radix_kth_largest(int n, Get get, int first, uint32_t& prefix,
                                  uint32_t& pmask, uint32_t& r, uint32_t* hist,
                                  uint32_t* s_wave, uint32_t* s_pick)
{
    for (int d = first; d < 3; ++d) {
        const int shift = (d == 0) ? 21 : (d == 1) ? 10 : 0;
        const int nb = (d == 2) ? 1024 : 2048;
        for (int i = threadIdx.x; i < nb; i += kSelThreads)
            hist[i] = 0u;
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += kSelThreads) {
            uint32_t v;
            if (get(i, v) && (v & pmask) == prefix)
                atomicAdd(&hist[(v >> shift) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        uint32_t bin, above;
        find_bin_desc(hist, nb, r, bin, above, s_wave, s_pick);
        r -= above;
        prefix |= bin << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
    }
}

__global__ __launch_bounds__(kSelThreads) void k_sel_clear(SelWs w, int BT)
{
    const size_t n = (size_t)BT * kBins;
    for (size_t i = (size_t)blockIdx.x * kSelThreads + threadIdx.x; i < n;
         i += (size_t)gridDim.x * kSelThreads)
        w.hist[i] = 0u;
    for (size_t i = (size_t)blockIdx.x * kSelThreads + threadIdx.x; i < (size_t)BT;
         i += (size_t)gridDim.x * kSelThreads) {
        w.cand_n[i] = 0u;
        w.done[i] = 0u;
    }
}

__global__ __launch_bounds__(kSelThreads) void k_sel_hist(SelWs w, int T, int N, int pos0,
                                                          int k, int dense_max)
{
    __shared__ uint32_t hist[kBins];
    const int bt = blockIdx.y;
    const int nvis = pos0 + (bt % T) + 1;
    const int j0 = blockIdx.x * kTile;
    if (!token_selects(nvis, k, dense_max) || j0 >= nvis)
        return;
    for (int i = threadIdx.x; i < kBins; i += kSelThreads)
        hist[i] = 0u;
    __syncthreads();
    const uint32_t* kr = w.keys + (size_t)bt * N;
    const int j1 = min(j0 + kTile, nvis);
    uint32_t u[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int j = j0 + i * kSelThreads + (int)threadIdx.x;
        u[i] = (j < j1) ? kr[j] : 0u;
    }
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
        if (j0 + i * kSelThreads + (int)threadIdx.x < j1)
            atomicAdd(&hist[u[i] >> 21], 1u);
    __syncthreads();
    uint32_t* gh = w.hist + (size_t)bt * kBins;
    for (int i = threadIdx.x; i < kBins; i += kSelThreads) {
        const uint32_t c = hist[i];
        if (c)
            atomicAdd(&gh[i], c);
    }
}

__global__ __launch_bounds__(kSelThreads) void k_sel_filter(SelWs w, int T, int N, int NT,
                                                            int pos0, int k, int dense_max)
{
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t s_wave[kSelThreads / 64];
    __shared__ uint32_t s_pick[2];

    const int bt = blockIdx.y;
    const int nvis = pos0 + (bt % T) + 1;
    const int tile = blockIdx.x;
    const int j0 = tile * kTile;
    if (!token_selects(nvis, k, dense_max) || j0 >= nvis)
        return;
    const uint32_t* kr = w.keys + (size_t)bt * N;

    // Bin of the k-th largest key, and how many keys lie above that bin.
    const uint32_t* gh = w.hist + (size_t)bt * kBins;
    for (int i = threadIdx.x; i < kBins; i += kSelThreads)
        hist[i] = gh[i];
    __syncthreads();
    uint32_t b1, above1;
    find_bin_desc(hist, kBins, (uint32_t)k, b1, above1, s_wave, s_pick);

    // This tile: count keys above the bin, append keys inside it.  Each wave
    // owns a contiguous quarter of the tile, loads it 64 keys per step with
    // all loads in flight at once, counts with ballots; one atomic per
    // workgroup reserves candidate slots, then the candidates are written.
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int j1 = min(j0 + kTile, nvis);
    const int wb = j0 + wv * (kTile / 4);
    uint32_t u[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int j = wb + i * 64 + lane;
        u[i] = (j < j1) ? kr[j] : 0u;
    }
    uint32_t n_def = 0, n_cand = 0;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const bool ok = wb + i * 64 + lane < j1;
        const uint32_t bin = u[i] >> 21;
        n_def += (uint32_t)__popcll(__ballot(ok && bin > b1));
        n_cand += (uint32_t)__popcll(__ballot(ok && bin == b1));
    }
    __shared__ uint32_t s_nc[kSelThreads / 64], s_nd[kSelThreads / 64], s_base;
    if (lane == 0) {
        s_nc[wv] = n_cand;
        s_nd[wv] = n_def;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t tc = 0, td = 0;
        for (int i = 0; i < kSelThreads / 64; ++i) {
            tc += s_nc[i];
            td += s_nd[i];
        }
        s_base = tc ? atomicAdd(&w.cand_n[bt], tc) : 0u;
        w.tile_def[(size_t)bt * NT + tile] = td;
    }
    __syncthreads();
    uint32_t* cand = w.cand + (size_t)bt * kCap * 2;
    uint32_t slot = s_base;
    for (int i = 0; i < wv; ++i)
        slot += s_nc[i];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int j = wb + i * 64 + lane;
        const bool is_c = j < j1 && (u[i] >> 21) == b1;
        const unsigned long long m = __ballot(is_c);
        const uint32_t pos = slot + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (is_c && pos < (uint32_t)kCap) {
            cand[2 * pos] = u[i];
            cand[2 * pos + 1] = (uint32_t)j;
        }
        slot += (uint32_t)__popcll(m);
    }

}

// One workgroup per selecting token: from the per-tile counts and the
// candidate list, the exact pivot (key, cell) of the k-th kept cell, and the
// output offset of every tile.
__global__ __launch_bounds__(kSelThreads) void k_sel_pivot(SelWs w, int32_t* __restrict__ n_sel,
                                                           int T, int N, int NT, int pos0,
                                                           int k, int dense_max)
{
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t s_wave[kSelThreads / 64];
    __shared__ uint32_t s_pick[2];
    __shared__ uint32_t c_key[kCap];
    __shared__ uint32_t c_idx[kCap];
    __shared__ uint32_t s_tile[kMaxTiles];

    const int bt = blockIdx.x;
    const int nvis = pos0 + (bt % T) + 1;
    if (!token_selects(nvis, k, dense_max))
        return;
    const int nt_eff = (nvis + kTile - 1) / kTile;
    const uint32_t* kr = w.keys + (size_t)bt * N;
    const uint32_t* cand = w.cand + (size_t)bt * kCap * 2;

    // Threshold bin again (same histogram, same answer as the filter).
    const uint32_t* gh = w.hist + (size_t)bt * kBins;
    for (int i = threadIdx.x; i < kBins; i += kSelThreads)
        hist[i] = gh[i];
    __syncthreads();
    uint32_t b1, above1;
    find_bin_desc(hist, kBins, (uint32_t)k, b1, above1, s_wave, s_pick);

    // Tile counts of every tile of this token (written by the filter).
    __shared__ uint32_t s_def[kMaxTiles];
    for (int i = threadIdx.x; i < nt_eff; i += kSelThreads)
        s_def[i] = w.tile_def[(size_t)bt * NT + i];
    uint32_t part = 0;
    for (int i = threadIdx.x; i < nt_eff; i += kSelThreads)
        part += w.tile_def[(size_t)bt * NT + i];
    uint32_t above;
    block_excl_scan(part, above, s_wave);
    // above: keys in bins higher than the threshold bin, over all tiles.
    const uint32_t need = (uint32_t)k - above;   // kept keys inside the bin, >= 1
    const uint32_t nc = w.cand_n[bt];

    uint32_t prefix = b1 << 21, pmask = 0xffe00000u, r = need;
    uint32_t tau, cut;
    for (int i = threadIdx.x; i < nt_eff; i += kSelThreads)
        s_tile[i] = 0u;
    if (nc <= (uint32_t)kCap) {
#pragma unroll
        for (int q = 0; q < kCap / kSelThreads; ++q) {
            const int i = q * kSelThreads + (int)threadIdx.x;
            if (i < (int)nc) {
                const uint2 e = ((const uint2*)cand)[i];
                c_key[i] = e.x;
                c_idx[i] = e.y;
            }
        }
        __syncthreads();
        radix_kth_largest((int)nc, [&](int i, uint32_t& v) { v = c_key[i]; return true; }, 1,
                          prefix, pmask, r, hist, s_wave, s_pick);
        tau = prefix;
        uint32_t ip = 0u, im = 0u;   // r-th smallest index among keys == tau
        radix_kth_largest((int)nc,
                          [&](int i, uint32_t& v) {
                              v = ~c_idx[i];
                              return c_key[i] == tau;
                          },
                          0, ip, im, r, hist, s_wave, s_pick);
        cut = ~ip;
        for (int i = threadIdx.x; i < (int)nc; i += kSelThreads) {
            const uint32_t u = c_key[i], j = c_idx[i];
            if (u > tau || (u == tau && j <= cut))
                atomicAdd(&s_tile[j / kTile], 1u);
        }
    } else {
        // Too many keys share the threshold bin: stream the token's keys.
        __syncthreads();
        radix_kth_largest(nvis, [&](int i, uint32_t& v) { v = kr[i]; return true; }, 1, prefix,
                          pmask, r, hist, s_wave, s_pick);
        tau = prefix;
        uint32_t ip = 0u, im = 0u;
        radix_kth_largest(nvis,
                          [&](int i, uint32_t& v) {
                              v = ~(uint32_t)i;
                              return kr[i] == tau;
                          },
                          0, ip, im, r, hist, s_wave, s_pick);
        cut = ~ip;
        for (int i = threadIdx.x; i < nvis; i += kSelThreads) {
            const uint32_t u = kr[i];
            if ((u >> 21) == b1 && (u > tau || (u == tau && (uint32_t)i <= cut)))
                atomicAdd(&s_tile[i / kTile], 1u);
        }
    }
    __syncthreads();
    // Output offset of each tile: exclusive prefix of its kept count
    // (kMaxTiles / kSelThreads = 4 consecutive tiles per thread).
    uint32_t* to = w.tile_off + (size_t)bt * NT;
    constexpr int TPT = kMaxTiles / kSelThreads;
    uint32_t tsum = 0;
    for (int i = 0; i < TPT; ++i) {
        const int t = threadIdx.x * TPT + i;
        tsum += (t < nt_eff) ? s_def[t] + s_tile[t] : 0u;
    }
    uint32_t ttot;
    uint32_t off = block_excl_scan(tsum, ttot, s_wave);
    for (int i = 0; i < TPT; ++i) {
        const int t = threadIdx.x * TPT + i;
        if (t < nt_eff) {
            to[t] = off;
            off += s_def[t] + s_tile[t];
        }
    }
    if (threadIdx.x == 0) {
        w.pivot[2 * bt] = tau;
        w.pivot[2 * bt + 1] = cut;
        n_sel[bt] = k;
    }
}

__global__ __launch_bounds__(kSelThreads) void k_sel_write(SelWs w, int32_t* __restrict__ ids,
                                                           int32_t* __restrict__ n_sel, int T,
                                                           int N, int NT, int pos0, int k,
                                                           int dense_max, int cap)
{
    const int bt = blockIdx.y;
    const int nvis = pos0 + (bt % T) + 1;
    const int tile = blockIdx.x;
    const int j0 = tile * kTile;
    int32_t* row = ids + (size_t)bt * cap;

    if (!token_selects(nvis, k, dense_max)) {
        // Keep every visible cell: ids 0..nvis-1, then -1.
        if (tile == 0 && threadIdx.x == 0)
            n_sel[bt] = nvis;
        const int e0 = j0, e1 = min(j0 + kTile, cap);
        for (int i = e0 + threadIdx.x; i < e1; i += kSelThreads)
            row[i] = (i < nvis) ? i : -1;
        return;
    }
    if (tile == 0)
        for (int i = k + threadIdx.x; i < cap; i += kSelThreads)
            row[i] = -1;
    if (j0 >= nvis)
        return;
    const uint32_t tau = w.pivot[2 * bt], cut = w.pivot[2 * bt + 1];
    const uint32_t base = w.tile_off[(size_t)bt * NT + tile];
    const uint32_t* kr = w.keys + (size_t)bt * N;
    // Each wave owns a contiguous quarter of the tile (so output order is
    // wave order, then lane order): count its kept cells with ballots, then
    // write them at their offsets.
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int j1 = min(j0 + kTile, nvis);
    const int wb = j0 + wv * (kTile / 4);
    uint32_t u[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int j = wb + i * 64 + lane;
        u[i] = (j < j1) ? kr[j] : 0u;
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const uint32_t j = (uint32_t)(wb + i * 64 + lane);
        const bool keep = (int)j < j1 && (u[i] > tau || (u[i] == tau && j <= cut));
        cnt += (uint32_t)__popcll(__ballot(keep));
    }
    __shared__ uint32_t s_cnt[kSelThreads / 64];
    if (lane == 0)
        s_cnt[wv] = cnt;
    __syncthreads();
    uint32_t wpos = base;
    for (int i = 0; i < wv; ++i)
        wpos += s_cnt[i];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const uint32_t j = (uint32_t)(wb + i * 64 + lane);
        const bool keep = (int)j < j1 && (u[i] > tau || (u[i] == tau && j <= cut));
        const unsigned long long m = __ballot(keep);
        const uint32_t pos = wpos + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (keep && pos < (uint32_t)k)
            row[pos] = (int32_t)j;
        wpos += (uint32_t)__popcll(m);
    }
}

// ------------------------------------------------- single-block select ---
//
// Rows of at most kRowThreads * KPT cells are selected by one workgroup per
// token: thread t holds the keys of cells t*KPT .. t*KPT+KPT-1 in registers,
// a radix select over them (digits of 11, 11 and 10 bits, LDS histograms)
// finds the k-th largest key v and how many keys equal to v are kept (the
// lowest cells first), and two block-wide prefix sums give every thread the
// output position of its kept cells, so the ids come out in ascending order.
// Cells past the token's position hold key 0, below every score key.

constexpr int kRowThreads = 1024;

// Exclusive prefix sum over the kRowThreads threads; `total` gets the sum.
__device__ __forceinline__ uint32_t row_excl_scan(uint32_t v, uint32_t& total,
                                                  uint32_t* s_wave)
{
    constexpr int NW = kRowThreads / 64;
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
    for (int i = 0; i < NW; ++i) {
        const uint32_t sv = s_wave[i];
        base += (i < w) ? sv : 0u;
        tot += sv;
    }
    __syncthreads();
    total = tot;
    return base + x - v;
}

// Selects the k largest of the row's keys, which thread t holds for cells
// c0 = t*KPT .. c0+KPT-1 (0 for cells past the token's position), and writes
// the kept cells in ascending order, -1 padding and the count.
template <int KPT>
__device__ __forceinline__ void select_row(const uint32_t (&key)[KPT], int c0, int k, int cap,
                                           int32_t* __restrict__ out, int32_t* __restrict__ n_out,
                                           uint32_t* hist, uint32_t* s_wave, uint32_t* s_pick)
{
    const int tid = threadIdx.x;
    // Radix select of the k-th largest key.
    uint32_t prefix = 0, pmask = 0, r = (uint32_t)k;
#pragma unroll 1
    for (int d = 0; d < 3; ++d) {
        const int shift = (d == 0) ? 21 : (d == 1) ? 10 : 0;
        const int nb = (d == 2) ? 1024 : 2048;
        for (int i = tid; i < nb; i += kRowThreads)
            hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if ((key[j] & pmask) == prefix)
                atomicAdd(&hist[(key[j] >> shift) & (uint32_t)(nb - 1)], 1u);
        __syncthreads();
        // Bin holding the r-th largest: thread t sums bins nb-1-2t and
        // nb-2-2t (nb / kRowThreads = 2 or 1 bins per thread).
        const int per = nb / kRowThreads;
        const int hi = nb - 1 - tid * per;
        uint32_t cnt_i[2] = {0u, 0u};
        for (int i = 0; i < per; ++i)
            cnt_i[i] = hist[hi - i];
        const uint32_t sum = cnt_i[0] + cnt_i[1];
        uint32_t total;
        const uint32_t ex = row_excl_scan(sum, total, s_wave);
        if (ex < r && r <= ex + sum) {
            uint32_t acc = ex;
            for (int i = 0; i < per; ++i) {
                const uint32_t cnt = cnt_i[i];
                if (acc < r && r <= acc + cnt) {
                    s_pick[0] = (uint32_t)(hi - i);
                    s_pick[1] = acc;
                }
                acc += cnt;
            }
        }
        __syncthreads();
        r -= s_pick[1];
        prefix |= s_pick[0] << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        __syncthreads();
    }

    // prefix is the k-th largest key; r keys equal to it are kept, lowest
    // cells first.
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        gt += key[j] > prefix ? 1u : 0u;
        eq += key[j] == prefix ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t eq_before = row_excl_scan(eq, total, s_wave);
    const uint32_t take_eq = eq_before >= r ? 0u : min(eq, r - eq_before);
    const uint32_t pos = row_excl_scan(gt + take_eq, total, s_wave);
    uint32_t o = pos, taken = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool is_eq = key[j] == prefix;
        const bool keep = key[j] > prefix || (is_eq && taken < take_eq);
        taken += is_eq ? 1u : 0u;
        if (keep)
            out[o++] = c0 + j;
    }
    for (int i = k + tid; i < cap; i += kRowThreads)
        out[i] = -1;
    if (tid == 0)
        *n_out = k;
}

// Dense row: ids 0..nvis-1, then -1.
__device__ __forceinline__ void dense_row(int nvis, int cap, int32_t* __restrict__ out,
                                          int32_t* __restrict__ n_out)
{
    if (threadIdx.x == 0)
        *n_out = nvis;
    for (int i = threadIdx.x; i < cap; i += kRowThreads)
        out[i] = (i < nvis) ? i : -1;
}

template <int KPT>
__global__ __launch_bounds__(kRowThreads) void k_sel_row(const uint32_t* __restrict__ keys,
                                                         int32_t* __restrict__ ids,
                                                         int32_t* __restrict__ n_sel, int T, int N,
                                                         int pos0, int k, int dense_max, int cap)
{
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t s_wave[kRowThreads / 64];
    __shared__ uint32_t s_pick[2];
    const int row = blockIdx.x;
    const int nvis = pos0 + (row % T) + 1;
    int32_t* out = ids + (size_t)row * cap;
    if (!token_selects(nvis, k, dense_max)) {
        dense_row(nvis, cap, out, n_sel + row);
        return;
    }
    const int c0 = threadIdx.x * KPT;
    const uint32_t* kr = keys + (size_t)row * N + c0;
    uint32_t key[KPT];
    if ((N & 3) == 0 && c0 + KPT <= nvis) {
#pragma unroll
        for (int j = 0; j < KPT; j += 4) {
            const uint4 v = *(const uint4*)(kr + j);
            key[j] = v.x;
            key[j + 1] = v.y;
            key[j + 2] = v.z;
            key[j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            key[j] = (c0 + j < nvis) ? kr[j] : 0u;
    }
    select_row<KPT>(key, c0, k, cap, out, n_sel + row, hist, s_wave, s_pick);
}

// One token (T == 1) per workgroup, scan and select fused: the 1024
// threads score the visible key rows (16 lanes per 256-byte row as in
// k_idx_scan, eight rows in flight per lane) into an LDS key table, then
// select from it.  Used while the row's keys fit in LDS.
template <int DI, int KPT>
__global__ __launch_bounds__(kRowThreads) void k_scan_select(const uint4* __restrict__ q_idx,
                                                             const uint4* __restrict__ K_idx,
                                                             int32_t* __restrict__ ids,
                                                             int32_t* __restrict__ n_sel, int N,
                                                             int pos0, int k, int dense_max, int cap)
{
    constexpr int LPR = DI / 8;                // lanes per key row
    constexpr int RPS = kRowThreads / LPR;     // rows per block-wide step
    constexpr int U = 16;                      // steps in flight per thread
    __shared__ uint32_t keys_s[kRowThreads * KPT];
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t s_wave[kRowThreads / 64];
    __shared__ uint32_t s_pick[2];
    const int b = blockIdx.x;
    const int nvis = pos0 + 1;
    int32_t* out = ids + (size_t)b * cap;
    if (!token_selects(nvis, k, dense_max)) {
        dense_row(nvis, cap, out, n_sel + b);
        return;
    }
    const int tid = threadIdx.x;
    const int sub = tid % LPR;
    const uint4 qv = q_idx[(size_t)b * (DI / 8) + sub];
    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
    const uint4* Kb = K_idx + (size_t)b * N * (DI / 8) + sub;
    for (int r0 = tid / LPR; r0 < nvis; r0 += RPS * U) {
        uint4 kv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = min(r0 + u * RPS, nvis - 1);
            kv[u] = Kb[(size_t)j * (DI / 8)];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = r0 + u * RPS;
            const uint32_t kw[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc = __builtin_amdgcn_fdot2(as_half2(qw[e]), as_half2(kw[e]), acc, false);
            acc = row_sum<LPR>(acc);
            if (sub == 0 && j < nvis)
                keys_s[j] = score_key(acc);
        }
    }
    __syncthreads();
    const int c0 = tid * KPT;
    uint32_t key[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        key[j] = (c0 + j < nvis) ? keys_s[c0 + j] : 0u;
    select_row<KPT>(key, c0, k, cap, out, n_sel + b, hist, s_wave, s_pick);
}

// Keys per thread of the single-block select for rows of N cells (0 if a row
// is too long for it).
static int row_select_kpt(int N)
{
    for (int kpt = 4; kpt <= 64; kpt *= 2)
        if ((long long)kRowThreads * kpt >= N)
            return kpt;
    return 0;
}

// ------------------------------------------------------------- launch ---

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static SelWs carve(void* ws, int B, int T, int N, size_t* total)
{
    const size_t BT = (size_t)B * T;
    const int NT = (N + kTile - 1) / kTile;
    char* p = (char*)ws;
    size_t off = 0;
    SelWs w;
    auto take = [&](size_t bytes) {
        char* q = p ? p + off : nullptr;
        off += align256(bytes);
        return q;
    };
    w.keys = (uint32_t*)take(BT * N * 4);
    w.hist = (uint32_t*)take(BT * kBins * 4);
    w.tile_def = (uint32_t*)take(BT * NT * 4);
    w.tile_off = (uint32_t*)take(BT * NT * 4);
    w.cand_n = (uint32_t*)take(BT * 4);
    w.done = (uint32_t*)take(BT * 4);
    w.cand = (uint32_t*)take(BT * kCap * 8);
    w.pivot = (uint32_t*)take(BT * 8);
    if (total)
        *total = off;
    return w;
}

size_t index_workspace_bytes(int B, int T, int N)
{
    size_t total = 0;
    carve(nullptr, B, T, N, &total);
    return total;
}

int index_max_cells() { return kMaxTiles * kTile; }

template <int DI>
static void launch_scan(const IndexLaunch& a, uint32_t* keys, int nvis_max, hipStream_t s)
{
    constexpr int rows_per_block = (256 / (DI / 8)) * 8;
    dim3 grid((nvis_max + rows_per_block - 1) / rows_per_block, a.B);
    k_idx_scan<DI, 1><<<grid, 256, 0, s>>>((const uint4*)a.q_idx, (const uint4*)a.K_idx, keys,
                                           a.T, a.N, nvis_max);
}

template <int DI>
static void launch_gemm(const IndexLaunch& a, uint32_t* keys, int nvis_max, hipStream_t s)
{
    constexpr int cells_per_block = 4 * 32 * kGemmBlocks;
    dim3 grid((nvis_max + cells_per_block - 1) / cells_per_block,
              (a.T + kGemmTok - 1) / kGemmTok, a.B);
    k_idx_gemm<DI><<<grid, 256, 0, s>>>((const _Float16*)a.q_idx, (const _Float16*)a.K_idx,
                                         keys, a.T, a.N, nvis_max);
}

hipError_t launch_index_topk(const IndexLaunch& a, hipStream_t s)
{
    SelWs w = carve(a.ws, a.B, a.T, a.N, nullptr);
    const int BT = a.B * a.T;
    const int NT = (a.N + kTile - 1) / kTile;
    // Scores are needed only when some token keeps fewer cells than it sees.
    const int nvis_max = a.pos0 + a.T;  // cells visible to the last token
    const bool any_select = token_selects(nvis_max, a.k, a.dense_max);
    // The fused kernel runs one workgroup per token; with fewer tokens than
    // about half the CUs the chip-wide scan is faster.
    if (any_select && a.T == 1 && a.N <= kRowThreads * 16 && a.B >= 128) {
        const uint4* q = (const uint4*)a.q_idx;
        const uint4* K = (const uint4*)a.K_idx;
#define QSA_FUSED(DI, KPT)                                                               \
    k_scan_select<DI, KPT><<<a.B, kRowThreads, 0, s>>>(q, K, a.ids, a.n_sel, a.N, a.pos0, a.k, \
                                                       a.dense_max, a.cap)
        const int kpt = row_select_kpt(a.N);
        if (a.DI == 64) {
            if (kpt <= 4) QSA_FUSED(64, 4); else if (kpt <= 8) QSA_FUSED(64, 8); else QSA_FUSED(64, 16);
        } else {
            if (kpt <= 4) QSA_FUSED(128, 4); else if (kpt <= 8) QSA_FUSED(128, 8); else QSA_FUSED(128, 16);
        }
#undef QSA_FUSED
        return hipGetLastError();
    }
    if (any_select) {
        if (a.T == 1) {
            if (a.DI == 64)
                launch_scan<64>(a, w.keys, nvis_max, s);
            else
                launch_scan<128>(a, w.keys, nvis_max, s);
        } else if (a.T <= 16) {
            const dim3 grid((nvis_max + 64 * kMscanGroups - 1) / (64 * kMscanGroups), a.B);
            if (a.DI == 64)
                k_idx_mscan<64><<<grid, 256, 0, s>>>((const _Float16*)a.q_idx,
                                                     (const _Float16*)a.K_idx, w.keys, a.T, a.N,
                                                     nvis_max);
            else
                k_idx_mscan<128><<<grid, 256, 0, s>>>((const _Float16*)a.q_idx,
                                                      (const _Float16*)a.K_idx, w.keys, a.T, a.N,
                                                      nvis_max);
        } else {
            if (a.DI == 64)
                launch_gemm<64>(a, w.keys, nvis_max, s);
            else
                launch_gemm<128>(a, w.keys, nvis_max, s);
        }
        const int kpt = row_select_kpt(a.N);
        if (kpt) {
#define QSA_ROW_ARGS w.keys, a.ids, a.n_sel, a.T, a.N, a.pos0, a.k, a.dense_max, a.cap
            switch (kpt) {
            case 4: k_sel_row<4><<<BT, kRowThreads, 0, s>>>(QSA_ROW_ARGS); break;
            case 8: k_sel_row<8><<<BT, kRowThreads, 0, s>>>(QSA_ROW_ARGS); break;
            case 16: k_sel_row<16><<<BT, kRowThreads, 0, s>>>(QSA_ROW_ARGS); break;
            case 32: k_sel_row<32><<<BT, kRowThreads, 0, s>>>(QSA_ROW_ARGS); break;
            default: k_sel_row<64><<<BT, kRowThreads, 0, s>>>(QSA_ROW_ARGS); break;
            }
#undef QSA_ROW_ARGS
            return hipGetLastError();
        }
        const int clear_blocks = (int)std::min<size_t>(((size_t)BT * kBins + 1023) / 1024, 4096);
        k_sel_clear<<<clear_blocks, kSelThreads, 0, s>>>(w, BT);
        const dim3 grid(NT, BT);
        k_sel_hist<<<grid, kSelThreads, 0, s>>>(w, a.T, a.N, a.pos0, a.k, a.dense_max);
        k_sel_filter<<<grid, kSelThreads, 0, s>>>(w, a.T, a.N, NT, a.pos0, a.k, a.dense_max);
        k_sel_pivot<<<BT, kSelThreads, 0, s>>>(w, a.n_sel, a.T, a.N, NT, a.pos0, a.k,
                                                 a.dense_max);
    }
    const int NTw = std::max(NT, (a.cap + kTile - 1) / kTile);
    k_sel_write<<<dim3(NTw, BT), kSelThreads, 0, s>>>(w, a.ids, a.n_sel, a.T, a.N, NT, a.pos0,
                                                       a.k, a.dense_max, a.cap);
    return hipGetLastError();
}

}  // namespace qsa
