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
//   k_idx_mscan  2 <= T <= 16 outside the fused path's range (rows under
//                16384 or over 65536 cells): the same stream, scored on MFMA
//                (v_mfma_f32_16x16x32_f16, tokens padded to 16 rows), no
//                cross-lane reduction.
//   k_scan_select one token with a row of at most 16384 cells (decode):
//                scan and select fused in one workgroup per token.
//   k_idx_sample, k_sel_thresh, k_idx_collect, k_sel_cand
//                two or more tokens (a draft batch, a prompt chunk) against
//                rows of 16384 to 65536 cells: the score GEMM on MFMA keeps only the
//                cells at or above a sampled bound, then an exact select
//                among them; the score matrix is never written (see the
//                section "many tokens: fused select").
//   k_scan_collect  one token against rows of 65537 to 262144 cells (long
//                context): the k_idx_scan stream keeping only the cells at or
//                above a sampled bound (k_idx_sample, k_sel_thresh), then
//                k_sel_cand's exact select among them.
//   k_idx_gemm   other many-token calls: [T x d_idx] x [d_idx x N] on MFMA
//                (v_mfma_f32_16x16x32_f16), 64 tokens x 256 cells per wave,
//                all score keys written for the select below.
//   k_sel_row    exact top-k of rows up to 65536 cells, one workgroup per
//                token, keys in registers.
//   k_sel_*      exact top-k over the score keys of longer rows, tiled over
//                the whole chip (histogram, filter + pivot, ordered write).
#include <algorithm>

#include "qsa_append.h"
#include "qsa_device.h"
#include "qsa_launch.h"
#include "qsa_select.h"

namespace qsa {

// ---------------------------------------------------------------- scan ---

template <int DI, int TT>
__global__ __launch_bounds__(256) void k_idx_scan(const uint4* __restrict__ q_idx,
                                                  const uint4* __restrict__ K_idx,
                                                  uint32_t* __restrict__ keys, int T, int N,
                                                  int nvis_max)
{
    idx_scan_block<DI, TT>(blockIdx.x, blockIdx.y, q_idx, K_idx, keys, T, N, nvis_max);
}

// The new index key of a one-token append, as the scan kernels that fold
// the append in handle it: lane `sub` of a key-row group holds 16 bytes of
// the key (the new fp32 row rounded to fp16, nearest even, as qsa_kv_append
// writes it); the group scores it with the scan's own dot2 sequence and
// row reduction, so the score equals the one the scan computes from the
// written key.
template <int DI>
__device__ __forceinline__ uint4 new_key_slice(const AppendLaunch& ap, int b, int sub)
{
    const float4* src = (const float4*)(ap.kidx_new + (size_t)b * DI) + 2 * sub;
    const float4 x0 = src[0], x1 = src[1];
    return make_uint4(pack_half2_rne(x0.x, x0.y), pack_half2_rne(x0.z, x0.w),
                      pack_half2_rne(x1.x, x1.y), pack_half2_rne(x1.z, x1.w));
}

template <int DI>
__device__ __forceinline__ float new_key_score(const uint32_t (&qw)[4], uint4 nkey)
{
    const uint32_t kw[4] = {nkey.x, nkey.y, nkey.z, nkey.w};
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_fdot2(as_half2(qw[e]), as_half2(kw[e]), acc, false);
    return row_sum<DI / 8>(acc);
}

// Slice `sub` of the new key into its cache row (cell pos0 of problem b).
template <int DI>
__device__ __forceinline__ void write_new_key(const AppendLaunch& ap, int b, int sub, uint4 nkey)
{
    *((uint4*)(ap.K_idx + ((size_t)b * ap.N + ap.pos0) * DI) + sub) = nkey;
}

// k_idx_scan for one token with the step's append folded in (qsa_step with
// fewer problems than the fused scan/select takes).  The workgroup whose
// rows end with the new cell (the last visible row, pos0) also writes the
// problem's new token: the new fp32 K/V rows are loaded at the start and
// written as codes and scales after the scan by the quantisation lanes of
// qsa_kv_append; the scan skips the new cell's row (its old contents) and
// wave 0 scores the new fp16 key with the scan's own dot2 sequence and row
// reduction -- the score the scan would compute from the written key --
// and writes the key.  Needs Hkv * D / 2 <= 256 quantisation lanes.
template <int DI>
__global__ __launch_bounds__(256) void k_idx_scan_append(const uint4* __restrict__ q_idx,
                                                         const uint4* __restrict__ K_idx,
                                                         uint32_t* __restrict__ keys, int N,
                                                         int nvis, AppendLaunch ap)
{
    constexpr int LPR = DI / 8;   // lanes per key row
    const int bx = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, sub = tid % LPR;
    const int jnew = nvis - 1;
    const bool owner = jnew / idx_scan_rows_per_block<DI>() == bx;
    const bool newkey = owner && ap.kidx_new != nullptr;
    const long long nq = (long long)ap.Hkv * (ap.D / 32) * 16;
    const bool qlane = owner && tid < nq;
    const long long wq = (long long)b * nq + tid;
    float4 nv = make_float4(0.f, 0.f, 0.f, 0.f);
    uint4 nkey = make_uint4(0u, 0u, 0u, 0u);
    if (qlane)
        nv = append_quant_load(ap, wq);
    if (newkey && tid < LPR)
        nkey = new_key_slice<DI>(ap, b, sub);
    idx_scan_rows<DI, 1>(bx, b, q_idx, K_idx, 1, N, nvis, [&](int, int j, float sc) {
        if (!(newkey && j == jnew))
            keys[(size_t)b * N + j] = score_key(sc);
    });
    if (newkey && tid < 64) {   // wave 0: lanes 0 .. LPR-1 hold the key
        const uint4 qv = q_idx[(size_t)b * (DI / 8) + sub];
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
        const float acc = new_key_score<DI>(qw, nkey);
        if (tid == 0)
            keys[(size_t)b * N + jnew] = score_key(acc);
        if (tid < LPR)
            write_new_key<DI>(ap, b, sub, nkey);
    }
    if (qlane)
        append_quant_store(ap, wq, nv, true);  // whole 8-lane groups (nq % 16 == 0)
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

constexpr int kTile = 4096;                         // cells per select tile
constexpr int kPerLane = kTile / kSelThreads;       // 16 keys per thread
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
    // fused many-token path
    uint32_t* thr;       // [BT] candidate bound (key)
    uint32_t* gcount;    // [BT] candidates appended
    uint32_t* samp;      // [BT][kSampleCells] sample keys
    uint2* fcand;        // [BT][kCandCap] (fp32 score bits, cell)
};

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
    __shared__ uint32_t s_pick[3];

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
    __shared__ uint32_t s_pick[3];
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

// The k-th largest of the keys the kRowThreads threads hold (KPT each; 0 for
// an absent key, below every real key): returns it, and in r the number of
// keys equal to it that rank within the k largest.  Radix digits of 11, 11
// and 10 bits with LDS histograms.
// `each(f)` calls f(key) for every key this thread holds.
// PRE0: hist already holds the first digit's counts of the real keys (built
// while the keys were produced; absent keys, all in bin 0 below every real
// key there, do not change which bin holds the k-th key or its rank in it).
// When the bin holding the k-th key must be kept whole (its count equals
// the keys still needed), the selection is every key at or above the bin's
// lowest key: the result is then (bin prefix) - 1 with r = 0, which keeps
// exactly those keys, and the remaining digits are skipped.
template <bool PRE0 = false, class Each>
__device__ __forceinline__ uint32_t row_kth_largest_each(Each each, uint32_t k, uint32_t& r,
                                                         uint32_t* hist, uint32_t* s_wave,
                                                         uint32_t* s_pick)
{
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0;
    r = k;
#pragma unroll 1
    for (int d = 0; d < 3; ++d) {
        const int shift = (d == 0) ? 21 : (d == 1) ? 10 : 0;
        const int nb = (d == 2) ? 1024 : 2048;
        if (!(PRE0 && d == 0)) {
            for (int i = tid; i < nb; i += kRowThreads)
                hist[i] = 0u;
            __syncthreads();
            each([&](uint32_t v) {
                if ((v & pmask) == prefix)
                    atomicAdd(&hist[(v >> shift) & (uint32_t)(nb - 1)], 1u);
            });
            __syncthreads();
        }
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
                    s_pick[2] = cnt;
                }
                acc += cnt;
            }
        }
        __syncthreads();
        r -= s_pick[1];
        prefix |= s_pick[0] << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        const bool whole = s_pick[2] == r && prefix != 0u && d < 2;
        __syncthreads();
        if (whole) {
            r = 0;
            return prefix - 1u;
        }
    }
    return prefix;
}

template <int KPT, bool PRE0 = false>
__device__ __forceinline__ uint32_t row_kth_largest(const uint32_t (&key)[KPT], uint32_t k,
                                                    uint32_t& r, uint32_t* hist, uint32_t* s_wave,
                                                    uint32_t* s_pick)
{
    return row_kth_largest_each<PRE0>(
        [&](auto f) {
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                f(key[j]);
        },
        k, r, hist, s_wave, s_pick);
}

// Selects the k largest of the row's keys, which thread t holds for cells
// c0 = t*KPT .. c0+KPT-1 (0 for cells past the token's position), and writes
// the kept cells in ascending order, -1 padding and the count.
template <int KPT, bool PRE0 = false>
__device__ __forceinline__ void select_row(const uint32_t (&key)[KPT], int c0, int k, int cap,
                                           int32_t* __restrict__ out, int32_t* __restrict__ n_out,
                                           uint32_t* hist, uint32_t* s_wave, uint32_t* s_pick)
{
    const int tid = threadIdx.x;
    uint32_t r;
    const uint32_t prefix =
        row_kth_largest<KPT, PRE0>(key, (uint32_t)k, r, hist, s_wave, s_pick);

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
    __shared__ uint32_t s_pick[3];
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
// APPEND: the workgroup also writes its problem's new token (T == 1) into
// the cache, off the scan's critical path: the new rows are loaded at the
// start; the scan skips the new cell's key row (its old contents); after
// the scan one row group scores the new fp16 key with the scan's own
// arithmetic (same dot2 sequence and row reduction, so the same fp32 score
// the scan would compute from the written key) and writes the key, and the
// quantisation lanes of qsa_kv_append for this problem write the codes and
// scales.  Needs Hkv * D / 2 <= kRowThreads quantisation lanes.
template <int DI, int KPT, bool APPEND>
__global__ __launch_bounds__(kRowThreads) void k_scan_select(const uint4* __restrict__ q_idx,
                                                             const uint4* __restrict__ K_idx,
                                                             int32_t* __restrict__ ids,
                                                             int32_t* __restrict__ n_sel, int N,
                                                             int pos0, int k, int dense_max, int cap,
                                                             AppendLaunch ap)
{
    constexpr int LPR = DI / 8;                // lanes per key row
    constexpr int RPS = kRowThreads / LPR;     // rows per block-wide step
    constexpr int U = 16;                      // steps in flight per thread
    __shared__ uint32_t keys_s[kRowThreads * KPT];
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t s_wave[kRowThreads / 64];
    __shared__ uint32_t s_pick[3];
    const int b = blockIdx.x;
    const int nvis = pos0 + 1;
    int32_t* out = ids + (size_t)b * cap;
    if (!token_selects(nvis, k, dense_max)) {
        if constexpr (APPEND) {
            append_problem(ap, b, kRowThreads);
        }
        dense_row(nvis, cap, out, n_sel + b);
        return;
    }
    const int tid = threadIdx.x;
    const int sub = tid % LPR;
    // APPEND: this lane's new K/V elements and (wave 0) its part of the new
    // index key, loaded now and used after the scan.
    const long long nq = APPEND ? (long long)ap.Hkv * (ap.D / 32) * 16 : 0;
    const bool qlane = tid < nq;
    const long long wq = (long long)b * nq + tid;
    const bool newkey = APPEND && ap.kidx_new != nullptr;
    float4 nv = make_float4(0.f, 0.f, 0.f, 0.f);
    uint4 nkey = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (APPEND) {
        if (qlane)
            nv = append_quant_load(ap, wq);
        if (newkey && tid < 64)
            nkey = new_key_slice<DI>(ap, b, sub);
    }
    const int jnew = newkey ? nvis - 1 : -1;  // the new cell: scored after the scan
    // The select's first-digit histogram is counted as the keys are made.
    for (int i = tid; i < 2048; i += kRowThreads)
        hist[i] = 0u;
    __syncthreads();
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
            if (sub == 0 && j < nvis && j != jnew) {
                const uint32_t kk = score_key(acc);
                keys_s[j] = kk;
                atomicAdd(&hist[kk >> 21], 1u);
            }
        }
    }
    if constexpr (APPEND) {
        if (newkey && tid < 64) {
            // wave 0: the new cell's score as the loop computes it
            const float acc = new_key_score<DI>(qw, nkey);
            if (tid == 0) {
                const uint32_t kk = score_key(acc);
                keys_s[jnew] = kk;
                atomicAdd(&hist[kk >> 21], 1u);
            }
            if (tid < LPR)
                write_new_key<DI>(ap, b, sub, nkey);
        }
        if (qlane)
            append_quant_store(ap, wq, nv, true);  // whole 8-lane groups (nq % 16 == 0)
    }
    __syncthreads();
    const int c0 = tid * KPT;
    uint32_t key[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        key[j] = (c0 + j < nvis) ? keys_s[c0 + j] : 0u;
    select_row<KPT, true>(key, c0, k, cap, out, n_sel + b, hist, s_wave, s_pick);
}

// ------------------------------------------ many tokens: fused select ---
//
// For two or more tokens against rows of kFusedMinCells to kFusedMaxCells
// cells the score matrix is never written.  Four kernels:
//   k_idx_sample   scores a fixed sample of kSampleCells cells of the row
//                  (evenly spread, each at a hashed offset inside its stride)
//                  for every token and writes their keys (0 where the token
//                  cannot see the cell);
//   k_sel_thresh   per token, a lower bound for the k-th largest key: the
//                  r-th largest sample key, r = mu + 4 sqrt(mu) + 4 with mu =
//                  k * (visible samples) / (visible cells) the expected number
//                  of samples among the k largest; resets the token's
//                  candidate count;
//   k_idx_collect  the whole score GEMM on the matrix cores, keeping only the
//                  (score, cell) pairs at or above the bound: per-token lists
//                  in LDS, flushed to the token's candidate list with one
//                  atomic per (workgroup, token);
//   k_sel_cand     per token, the exact top-k among the candidates (radix
//                  select on the key, then on the cell index among equal
//                  keys, so ties go to the lower index) and the kept ids in
//                  ascending order through an LDS bitmap of the row.
// Exactness: the candidates are every visible cell whose key is at or above
// the bound.  When there are at least k of them the row's k-th largest key is
// at or above the bound, so every cell that can be kept is a candidate and
// the selection among the candidates is the selection of the row.  A token
// with fewer than k candidates (bound too high) or more than kCandCap (list
// overflow, e.g. massive exact ties) scores its whole row again, with the
// same matrix instructions and operand layout and so the same fp32 scores,
// into its key row of the workspace and runs the register select of
// k_sel_row on it.

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));

constexpr int kSampleCells = 2048;    // sampled cells per row
constexpr int kCandCap = 8192;        // candidates kept per token
constexpr int kCollectList = 64;      // LDS candidate slots per (workgroup, token)
constexpr int kFusedMaxCells = 65536; // longest row of the fused path (bitmap, registers)
constexpr int kFusedMinCells = 16384; // shorter rows write their keys instead
constexpr int kFusedMinTokens = 2;    // fewer tokens per problem take the one-token paths
// One-token rows between the register select's limit and this length take
// the sampled-bound path with k_scan_collect (bitmap of the row in LDS).
constexpr int kLongFusedMaxCells = 262144;

// Reduction-index permutation of the matrix-core score kernels: at step st,
// lane group g (lanes 16g .. 16g+15) supplies row elements
// 64*(st/2) + 16*g + 8*(st%2) .. +7, in both operands, so over a step pair a
// lane reads 32 contiguous bytes of its row.
__device__ __forceinline__ int kperm(int st, int grp)
{
    return 64 * (st >> 1) + 16 * grp + 8 * (st & 1);
}

// Scores of 16 cells against 16 tokens on the matrix cores
// (v_mfma_f32_16x16x32_f16): A = the cells' keys (lane l supplies row l%16),
// B = the tokens' index queries (lane l supplies column l%16).  Lane l gets
// cells 4*(l/16) + e, e = 0..3, of token column l%16.  Each element is the
// same dot product in the same order whatever else shares the instruction.
template <int KS>
__device__ __forceinline__ float4_t score_block(const h8_t (&kc)[KS], const h8_t (&qt)[KS])
{
    float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KS; ++st)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kc[st], qt[st], acc, 0, 0, 0);
    return acc;
}

// Cell of sample s of a row whose sampled span is `span` cells (< span).
__device__ __forceinline__ int sample_cell(int s, int span)
{
    const int stride = max(1, span / kSampleCells);
    return s * stride + (int)((((uint32_t)s * 0x9E3779B1u) >> 16) % (uint32_t)stride);
}

// The smallest score whose key is `key` (inverse of score_key): a score s
// satisfies score_key(s) >= key exactly when s >= key_to_score(key).  Key 0
// (take every cell) gives -inf; key 0xffffffff (take none) gives NaN, which
// no comparison passes.
__device__ __forceinline__ float key_to_score(uint32_t key)
{
    if (key == 0u)
        return -INFINITY;
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Grid (kSampleCells / 256, ceil(T / 64), B); a wave scores 64 tokens
// against 64 samples, 16 samples per step.
template <int DI>
__global__ __launch_bounds__(256) void k_idx_sample(const _Float16* __restrict__ q_idx,
                                                    const _Float16* __restrict__ K_idx,
                                                    uint32_t* __restrict__ samp, int T, int N,
                                                    int pos0, int span)
{
    constexpr int KS = DI / 32;
    const int b = blockIdx.z;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;
    const int tok0 = blockIdx.y * 64;
    const int s_base = (blockIdx.x * 4 + w) * 64;
    h8_t qt[4][KS];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = min(tok0 + 16 * i + r, T - 1);
        const _Float16* src = q_idx + ((size_t)b * T + tok) * DI;
#pragma unroll
        for (int st = 0; st < KS; ++st)
            qt[i][st] = *(const h8_t*)(src + kperm(st, grp));
    }
    h8_t kc4[4][KS];   // all four groups' keys in flight together
#pragma unroll
    for (int g16 = 0; g16 < 4; ++g16) {
        const int cell = sample_cell(s_base + 16 * g16 + r, span);
        const _Float16* src = K_idx + ((size_t)b * N + cell) * DI;
#pragma unroll
        for (int st = 0; st < KS; ++st)
            kc4[g16][st] = *(const h8_t*)(src + kperm(st, grp));
    }
#pragma unroll
    for (int g16 = 0; g16 < 4; ++g16) {
        const int s0 = s_base + 16 * g16;
        const h8_t (&kc)[KS] = kc4[g16];
        int ce[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            ce[e] = sample_cell(s0 + 4 * grp + e, span);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4_t acc = score_block<KS>(kc, qt[i]);
            const int tok = tok0 + 16 * i + r;
            if (tok < T) {
                const int nvis = pos0 + tok + 1;
                uint4 v;
                v.x = ce[0] < nvis ? score_key(acc[0]) : 0u;
                v.y = ce[1] < nvis ? score_key(acc[1]) : 0u;
                v.z = ce[2] < nvis ? score_key(acc[2]) : 0u;
                v.w = ce[3] < nvis ? score_key(acc[3]) : 0u;
                *(uint4*)(samp + ((size_t)b * T + tok) * kSampleCells + s0 + 4 * grp) = v;
            }
        }
    }
}

// Number of keys of the wave at or above t: K keys per lane, 0 = absent.
template <int K>
__device__ __forceinline__ uint32_t wave_count_ge(const uint32_t (&v)[K], uint32_t t)
{
    uint32_t n = 0;
#pragma unroll
    for (int m = 0; m < K; ++m)
        n += (uint32_t)__popcll(__ballot(v[m] >= t));
    return n;
}

// The r-th largest key of the wave (r >= 1, at most the number of nonzero
// keys), given that it lies in [lo, hi] (lo >= 1): the largest t with at
// least r keys >= t, built bit by bit below the bits that lo and hi share,
// each trial value kept when the wave-wide count still reaches r.
template <int K>
__device__ __forceinline__ uint32_t wave_kth_in(const uint32_t (&v)[K], uint32_t r, uint32_t lo,
                                                uint32_t hi)
{
    const uint32_t diff = lo ^ hi;
    if (diff == 0u)
        return lo;
    const int nb = 32 - __clz(diff);
    uint32_t t = lo & ~((nb == 32 ? 0u : (1u << nb)) - 1u);
#pragma unroll 1
    for (int bit = nb - 1; bit >= 0; --bit) {
        const uint32_t c = t | (1u << bit);
        if (wave_count_ge(v, c) >= r)
            t = c;
    }
    return t;
}

// One wave per token: the candidate bound from the token's sample keys, 32
// per lane in registers.  The r-th largest key x is found in three stages:
//   1. each lane's two largest keys; the r-th largest of these 128 values,
//      L, is at most x (they are a subset of the keys);
//   2. the keys >= L (all keys >= x among them: about r plus a few dozen
//      for evenly spread samples) are compacted into LDS;
//   3. the exact r-th largest of those, at most four per lane, bit by bit.
// When L is 0 (r above the number of nonzero top-two values) or more than
// 256 keys reach it, stage 3 runs on all 32 keys per lane instead.  Absent
// samples (key 0) never count, since every trial value is nonzero.
__global__ __launch_bounds__(64) void k_sel_thresh(const uint32_t* __restrict__ samp,
                                                   uint32_t* __restrict__ thr,
                                                   uint32_t* __restrict__ gcount, int T, int pos0,
                                                   int k, int dense_max)
{
    constexpr int M = kSampleCells / 64;
    constexpr int C = 4;   // compacted keys per lane
    __shared__ uint32_t s_k[64 * C];
    const int bt = blockIdx.x, lane = threadIdx.x;
    const int nvis = pos0 + bt % T + 1;
    if (!token_selects(nvis, k, dense_max)) {
        if (lane == 0) {
            thr[bt] = 0xffffffffu;   // above every score key: no candidates
            gcount[bt] = 0u;
        }
        return;
    }
    const uint4* row = (const uint4*)(samp + (size_t)bt * kSampleCells);
    uint32_t v[M];
#pragma unroll
    for (int m = 0; m < M / 4; ++m) {
        const uint4 x = row[m * 64 + lane];
        v[4 * m] = x.x;
        v[4 * m + 1] = x.y;
        v[4 * m + 2] = x.z;
        v[4 * m + 3] = x.w;
    }
    uint32_t total = 0;
#pragma unroll
    for (int m = 0; m < M; ++m)
        total += (uint32_t)__popcll(__ballot(v[m] != 0u));
    const float mu = (float)k * (float)total / (float)nvis;
    const uint32_t r = (uint32_t)ceilf(mu + 4.f * sqrtf(mu) + 4.f);
    uint32_t bound = 0u;   // 0: every visible cell is a candidate
    if (r < total) {
        uint32_t top[2] = {0u, 0u};   // this lane's two largest keys
#pragma unroll
        for (int m = 0; m < M; ++m) {
            top[1] = max(top[1], min(top[0], v[m]));
            top[0] = max(top[0], v[m]);
        }
        uint32_t hi = top[0];   // the wave's largest key
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
        const uint32_t L = wave_count_ge(top, 1u) >= r ? wave_kth_in(top, r, 1u, hi) : 0u;
        uint32_t n = 0;   // keys >= L, compacted in order of (register, lane)
        if (L != 0u) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const bool in = v[m] >= L;
                const unsigned long long bal = __ballot(in);
                const uint32_t pos = n + __builtin_amdgcn_mbcnt_hi(
                                             (uint32_t)(bal >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                if (in && pos < (uint32_t)(64 * C))
                    s_k[pos] = v[m];
                n += (uint32_t)__popcll(bal);
            }
        }
        if (L != 0u && n <= (uint32_t)(64 * C)) {
            __syncthreads();
            uint32_t c[C];
#pragma unroll
            for (int j = 0; j < C; ++j)
                c[j] = (uint32_t)(j * 64 + lane) < n ? s_k[j * 64 + lane] : 0u;
            bound = wave_kth_in(c, r, L, hi);
        } else {
            bound = wave_kth_in(v, r, 1u, hi);
        }
    }
    if (lane == 0) {
        thr[bt] = bound;
        gcount[bt] = 0u;
    }
}

// Grid: 8 x (cell ranges of 1024 per XCD) x ceil(T / 64) x B workgroups,
// arranged so that the workgroups of one cell range run on one XCD one
// after another (dispatch goes round-robin over the 8 XCDs): the range's
// keys stay in that XCD's L2 for all its token blocks.  The four waves share
// 16 NCB tokens (NCB 16-token column blocks: 4, or 1 when a problem has at
// most 16 tokens), whose query operands sit in LDS; a wave walks 256 cells,
// 32 per step, with the next step's keys in flight, and keeps the (score,
// cell) pairs at or above each token's bound.
template <int DI, int NCB>
__global__ __launch_bounds__(256, 3) void k_idx_collect(const _Float16* __restrict__ q_idx,
                                                     const _Float16* __restrict__ K_idx,
                                                     const uint32_t* __restrict__ thr,
                                                     uint32_t* __restrict__ gcount,
                                                     uint2* __restrict__ cand, int T, int N,
                                                     int pos0, int n_cr, int n_tb, int B)
{
    constexpr int KS = DI / 32;
    // Row pitch kCollectList + 1 entries, so the lists of the 16 tokens that
    // one instruction appends to start on different LDS banks.
    __shared__ uint2 lst[16 * NCB][kCollectList + 1];
    __shared__ uint32_t cnt[16 * NCB];
    // Query operands: slot (i, st) holds, for lane (r, g), token 16 i + r,
    // elements kperm(st, g): one 16-byte slot per lane, lanes contiguous.
    __shared__ h8_t qs[NCB][KS][64];
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int tb = local % n_tb;
    const int crb = (local / n_tb) * 8 + xcd;     // (problem, cell range) index
    if (crb >= n_cr * B)
        return;
    const int b = crb / n_cr, cr = crb % n_cr;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, grp = lane >> 4;
    const int tok0 = tb * 16 * NCB;
    const int cell_base = cr * 1024 + w * 256;
    const int nvis_hi = pos0 + min(tok0 + 16 * NCB, T);   // cells seen by the block's last token
    const int nvis_lo = pos0 + tok0 + 1;             // cells seen by its first token
    if (threadIdx.x < 16 * NCB)
        cnt[threadIdx.x] = 0u;
    if (w < NCB) {   // wave w fills column block w of the query operands
        const int tok = min(tok0 + 16 * w + r, T - 1);
        const _Float16* src = q_idx + ((size_t)b * T + tok) * DI;
#pragma unroll
        for (int st = 0; st < KS; ++st)
            qs[w][st][lane] = *(const h8_t*)(src + kperm(st, grp));
    }
    float thf[NCB];   // score bound of the lane's token in each column block
    int nv[NCB];
#pragma unroll
    for (int i = 0; i < NCB; ++i) {
        const int tok = tok0 + 16 * i + r;
        thf[i] = key_to_score(tok < T ? thr[(size_t)b * T + tok] : 0xffffffffu);
        nv[i] = pos0 + tok + 1;
    }
    const int n_steps = max(0, min(8, (nvis_hi - cell_base + 31) / 32));
    auto load_step = [&](int cb, h8_t (&kc)[2][KS]) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int cell = min(cell_base + 32 * cb + 16 * jj + r, nvis_hi - 1);
            const _Float16* src = K_idx + ((size_t)b * N + cell) * DI;
#pragma unroll
            for (int st = 0; st < KS; ++st)
                kc[jj][st] = *(const h8_t*)(src + kperm(st, grp));
        }
    };

    // One step: the eight products (independent accumulators, so the matrix
    // instructions pipeline), then the keys of step cb + 1 into the same
    // registers, then the candidates while those are in flight.
    auto step = [&](int cb, h8_t (&kc)[2][KS]) {
        // The query operands are read from LDS at every step rather than
        // held in 16 KS registers across the loop (three waves per SIMD).
        __asm__ volatile("" ::: "memory");
        float4_t acc[NCB][2];
#pragma unroll
        for (int i = 0; i < NCB; ++i) {
            h8_t qv[KS];
#pragma unroll
            for (int st = 0; st < KS; ++st)
                qv[st] = qs[i][st][lane];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                acc[i][jj] = score_block<KS>(kc[jj], qv);
        }
        if (cb + 1 < n_steps)
            load_step(cb + 1, kc);
        const int c0 = cell_base + 32 * cb;
        // Candidate masks, bit 4*jj + e: cell c0 + 16 jj + 4 grp + e of the
        // lane's token in column block i (non-short-circuit tests, no
        // branches; visibility only where part of the step lies past a token).
        uint32_t mk[NCB];
        if (c0 + 32 <= nvis_lo) {
#pragma unroll
            for (int i = 0; i < NCB; ++i) {
                mk[i] = 0u;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        mk[i] |= (acc[i][jj][e] >= thf[i]) ? 1u << (4 * jj + e) : 0u;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NCB; ++i) {
                mk[i] = 0u;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        mk[i] |= ((acc[i][jj][e] >= thf[i]) & (c0 + 16 * jj + 4 * grp + e < nv[i]))
                                     ? 1u << (4 * jj + e) : 0u;
            }
        }
        // Appends the candidates of column block i (accumulators a0, a1 by
        // value, so nothing is indexed at run time).
        auto append = [&](int i, float4_t a0, float4_t a1, uint32_t mm) {
            const int tl = 16 * i + r;
            const uint32_t n = (uint32_t)__popc(mm);
            uint32_t slot = atomicAdd(&cnt[tl], n);
            // Each set bit in turn (a few per lane at most): the element is
            // picked from the accumulators by its bit position.
            while (mm) {
                const uint32_t bp = (uint32_t)__builtin_ctz(mm);
                mm &= mm - 1u;
                const float4_t a4 = (bp & 4u) ? a1 : a0;
                const float x0 = (bp & 2u) ? a4[2] : a4[0];
                const float x1 = (bp & 2u) ? a4[3] : a4[1];
                const uint2 ent = make_uint2(
                    __float_as_uint((bp & 1u) ? x1 : x0),
                    (uint32_t)(c0 + 16 * (int)(bp >> 2) + 4 * grp + (int)(bp & 3u)));
                if (slot < (uint32_t)kCollectList) {
                    lst[tl][slot] = ent;
                } else {   // the token's LDS list is full: straight to its list
                    const size_t bt = (size_t)b * T + tok0 + tl;
                    const uint32_t p = atomicAdd(&gcount[bt], 1u);
                    if (p < (uint32_t)kCandCap)
                        cand[bt * kCandCap + p] = ent;
                }
                ++slot;
            }
        };
#pragma unroll
        for (int i = 0; i < NCB; ++i)
            append(i, acc[i][0], acc[i][1], mk[i]);
    };

    h8_t kc[2][KS];
    if (n_steps > 0)
        load_step(0, kc);
    __syncthreads();   // query operands and list counts ready
#pragma unroll 1
    for (int cb = 0; cb < n_steps; ++cb)
        step(cb, kc);
    __syncthreads();
    // Flush: wave w appends the lists of tokens 16w .. 16w+15, reserving all
    // sixteen slot ranges at once (lane j for token 16w + j).
    if (w >= NCB)
        return;
    const int tl_l = 16 * w + (lane & 15);
    const int tok_l = tok0 + tl_l;
    const uint32_t n_l = (tok_l < T) ? min(cnt[tl_l], (uint32_t)kCollectList) : 0u;
    uint32_t base_l = 0;
    if (lane < 16 && n_l)
        base_l = atomicAdd(&gcount[(size_t)b * T + tok_l], n_l);
    for (int j = 0; j < 16; ++j) {
        const uint32_t n = (uint32_t)__shfl((int)n_l, j, 64);
        if (n == 0)
            continue;
        const uint32_t base = (uint32_t)__shfl((int)base_l, j, 64);
        const int tl = 16 * w + j;
        uint2* dst = cand + ((size_t)b * T + tok0 + tl) * kCandCap;
        for (uint32_t idx = lane; idx < n; idx += 64)
            if (base + idx < (uint32_t)kCandCap)
                dst[base + idx] = lst[tl][idx];
    }
}

// One token (T = 1) against a long row: the chip-wide scan of k_idx_scan,
// keeping only the (score, cell) pairs at or above the problem's bound
// instead of writing every key.  A workgroup scans kScanCollectSpan row
// blocks and stages its candidates in LDS, so the problem's list takes one
// atomic per workgroup (same-address device atomics are slow); a full LDS
// list spills straight to the problem's list until that overflows.  Grid
// (ceil(row blocks / kScanCollectSpan), B).
constexpr int kScanCollectSpan = 4;
constexpr int kScanCollectList = 512;

template <int DI>
__global__ __launch_bounds__(256) void k_scan_collect(const uint4* __restrict__ q_idx,
                                                      const uint4* __restrict__ K_idx,
                                                      const uint32_t* __restrict__ thr,
                                                      uint32_t* __restrict__ gcount,
                                                      uint2* __restrict__ cand, int N, int nvis)
{
    constexpr int RB = idx_scan_rows_per_block<DI>();
    __shared__ uint2 lst[kScanCollectList];
    __shared__ uint32_t s_cnt, s_base;
    const int b = blockIdx.y;
    const float bound = key_to_score(thr[b]);   // score_key(s) >= thr  <=>  s >= bound
    uint32_t* gc = gcount + b;
    uint2* list = cand + (size_t)b * kCandCap;
    if (threadIdx.x == 0)
        s_cnt = 0u;
    __syncthreads();
    bool full = false;   // this lane saw the problem's list overflow
    const int nrb = (nvis + RB - 1) / RB;
    const int bx0 = blockIdx.x * kScanCollectSpan;
    const int nb = min(kScanCollectSpan, nrb - bx0);
    uint4 qv[1];
    idx_scan_query<DI, 1>(b, q_idx, 1, qv);
    auto emit = [&](int, int j, float sc) {
        if (sc >= bound) {
            const uint2 e = make_uint2(__float_as_uint(sc), (uint32_t)j);
            const uint32_t slot = atomicAdd(&s_cnt, 1u);
            if (slot < (uint32_t)kScanCollectList) {
                lst[slot] = e;
            } else if (!full) {
                const uint32_t p = atomicAdd(gc, 1u);
                if (p < (uint32_t)kCandCap)
                    list[p] = e;
                else
                    full = true;
            }
        }
    };
    // Row blocks in turn, the next block's keys in flight while the current
    // one is scored (two register buffers, alternating).
    uint4 ka[kScanSteps], kb[kScanSteps];
    idx_scan_load<DI>(bx0, b, K_idx, N, nvis, ka);
#pragma unroll 1
    for (int i = 0; i < nb; i += 2) {
        if (i + 1 < nb)
            idx_scan_load<DI>(bx0 + i + 1, b, K_idx, N, nvis, kb);
        idx_scan_compute<DI, 1>(bx0 + i, qv, ka, 1, nvis, emit);
        if (i + 1 >= nb)
            break;
        if (i + 2 < nb)
            idx_scan_load<DI>(bx0 + i + 2, b, K_idx, N, nvis, ka);
        idx_scan_compute<DI, 1>(bx0 + i + 1, qv, kb, 1, nvis, emit);
    }
    __syncthreads();
    const uint32_t n = min(s_cnt, (uint32_t)kScanCollectList);
    if (threadIdx.x == 0)
        s_base = n ? atomicAdd(gc, n) : 0u;
    __syncthreads();
    const uint32_t base = s_base;
    for (uint32_t i = threadIdx.x; i < n; i += 256)
        if (base + i < (uint32_t)kCandCap)
            list[base + i] = lst[i];
}

// One workgroup per token: the exact top-k among its candidates, or the
// whole-row fallback (see above).
template <int DI, int MAXC, bool SCAN1>
__global__ __launch_bounds__(kSelThreads) void k_sel_cand(const _Float16* __restrict__ q_idx,
                                                          const _Float16* __restrict__ K_idx,
                                                          const uint32_t* __restrict__ gcount,
                                                          const uint2* __restrict__ cand,
                                                          uint32_t* __restrict__ keys,
                                                          int32_t* __restrict__ ids,
                                                          int32_t* __restrict__ n_sel, int T,
                                                          int N, int pos0, int k, int dense_max,
                                                          int cap)
{
    constexpr int CPT = kCandCap / kSelThreads;    // candidates per thread
    constexpr int WPT = MAXC / 32 / kSelThreads;   // bitmap words per thread
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t s_wave[kSelThreads / 64];
    __shared__ uint32_t s_pick[3];
    __shared__ uint32_t s_red[8];
    __shared__ uint32_t bm[MAXC / 32];
    const int bt = blockIdx.x, tid = threadIdx.x;
    const int nvis = pos0 + bt % T + 1;
    int32_t* out = ids + (size_t)bt * cap;
    if (!token_selects(nvis, k, dense_max)) {
        dense_row_wg(nvis, cap, out, n_sel + bt);
        return;
    }
    const uint32_t nc = gcount[bt];
    if (nc >= (uint32_t)k && nc <= (uint32_t)kCandCap) {
        const uint2* cr = cand + (size_t)bt * kCandCap;
        float sc[CPT];      // scores (-inf: empty slot)
        uint32_t cc[CPT];   // cells
        float smax = -INFINITY, smin = INFINITY;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const uint32_t i = (uint32_t)(j * kSelThreads + tid);
            const uint2 e = i < nc ? cr[i] : make_uint2(__float_as_uint(-INFINITY), 0u);
            sc[j] = __uint_as_float(e.x);
            cc[j] = e.y;
            if (i < nc) {
                smax = fmaxf(smax, sc[j]);
                smin = fminf(smin, sc[j]);
            }
        }
        // Linear bins over [smin, smax]: bin(s) = floor((s - smin) * nb / (smax - smin)),
        // evaluated in fp32; every step is monotone, so bin order follows score order
        // and equal scores share a bin.
        smax = -wg_min_f(-smax, s_red);
        smin = wg_min_f(smin, s_red);
        float inv = (smax > smin) ? (float)kBins / (smax - smin) : 0.f;
        if (!(inv < INFINITY))
            inv = 0.f;   // range too narrow to scale: one bin, radix path below
        auto bin_of = [&](float x) { return min(kBins - 1, (int)((x - smin) * inv)); };
        for (int i = tid; i < kBins; i += kSelThreads)
            hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            if ((uint32_t)(j * kSelThreads + tid) < nc)
                atomicAdd(&hist[bin_of(sc[j])], 1u);
        __syncthreads();
        uint32_t tb, above;   // bin of the k-th largest, count in higher bins
        wg_find_bin(hist, kBins, (uint32_t)k, tb, above, s_wave, s_pick);
        const uint32_t need = (uint32_t)k - above;   // kept from bin tb
        // The members of bin tb, then each one's rank among them by (score desc,
        // cell asc); the `need` best are kept.
        if (tid == 0)
            s_red[0] = 0u;
        __syncthreads();
        uint2* mem = (uint2*)bm;   // reused: at most kSelThreads members
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            if ((uint32_t)(j * kSelThreads + tid) < nc && bin_of(sc[j]) == (int)tb) {
                const uint32_t slot = atomicAdd(&s_red[0], 1u);
                if (slot < (uint32_t)kSelThreads)
                    mem[slot] = make_uint2(__float_as_uint(sc[j]), cc[j]);
            }
        __syncthreads();
        const uint32_t m = s_red[0];
        uint32_t keep_cell = 0xffffffffu;   // this thread's kept member of bin tb
        if (m <= (uint32_t)kSelThreads) {
            if (tid < (int)m) {
                const float x = __uint_as_float(mem[tid].x);
                const uint32_t c = mem[tid].y;
                uint32_t rank = 0;
                for (uint32_t i = 0; i < m; ++i) {
                    const float y = __uint_as_float(mem[i].x);
                    rank += (y > x || (y == x && mem[i].y < c)) ? 1u : 0u;
                }
                if (rank < need)
                    keep_cell = c;
            }
        }
        __syncthreads();
        const int nw = (nvis + 31) >> 5;
        for (int i = tid; i < nw; i += kSelThreads)
            bm[i] = 0u;
        __syncthreads();
        if (m <= (uint32_t)kSelThreads) {
#pragma unroll
            for (int j = 0; j < CPT; ++j)
                if ((uint32_t)(j * kSelThreads + tid) < nc && bin_of(sc[j]) > (int)tb)
                    atomicOr(&bm[cc[j] >> 5], 1u << (cc[j] & 31));
            if (keep_cell != 0xffffffffu)
                atomicOr(&bm[keep_cell >> 5], 1u << (keep_cell & 31));
        } else {
            // Heavy ties in one bin: exact radix select over all candidates,
            // read again from the list (keys), then on the cell index among
            // the keys equal to the k-th.
            auto key_at = [&](uint32_t i) { return score_key(__uint_as_float(cr[i].x)); };
            uint32_t req = (uint32_t)k;
            const uint32_t tau = wg_kth_largest(
                [&](auto f) {
                    for (uint32_t i = tid; i < nc; i += kSelThreads)
                        f(key_at(i));
                },
                req, hist, s_red, s_wave, s_pick);
            uint32_t nties = 0;
            for (uint32_t i = tid; i < nc; i += kSelThreads)
                nties += key_at(i) == tau ? 1u : 0u;
            uint32_t ties;
            block_excl_scan(nties, ties, s_wave);
            uint32_t cut = 0xffffffffu;
            if (ties > req) {
                uint32_t r2 = req;
                cut = ~wg_kth_largest(
                    [&](auto f) {
                        for (uint32_t i = tid; i < nc; i += kSelThreads)
                            f(key_at(i) == tau ? ~cr[i].y : 0u);
                    },
                    r2, hist, s_red, s_wave, s_pick);
            }
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const uint32_t kj = (uint32_t)(j * kSelThreads + tid) < nc ? score_key(sc[j]) : 0u;
                if (kj > tau || (kj == tau && kj != 0u && cc[j] <= cut))
                    atomicOr(&bm[cc[j] >> 5], 1u << (cc[j] & 31));
            }
        }
        __syncthreads();
        uint32_t wd[WPT];
        uint32_t cntw = 0;
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int wi = WPT * tid + i;
            wd[i] = wi < nw ? bm[wi] : 0u;
            cntw += (uint32_t)__popc(wd[i]);
        }
        uint32_t total;
        uint32_t pos = block_excl_scan(cntw, total, s_wave);
#pragma unroll
        for (int i = 0; i < WPT; ++i)
            for (uint32_t mm = wd[i]; mm && pos < (uint32_t)k; mm &= mm - 1)
                out[pos++] = 32 * (WPT * tid + i) + __builtin_ctz(mm);
        for (int i = k + tid; i < cap; i += kSelThreads)
            out[i] = -1;
        if (tid == 0)
            n_sel[bt] = k;
        return;
    }

    // Fallback: the whole row again (with the arithmetic of the kernel that
    // collected the candidates) into the token's key row, then the exact
    // select over that row.
    uint32_t* kr = keys + (size_t)bt * N;
    if constexpr (SCAN1) {
        constexpr int RB = idx_scan_rows_per_block<DI>();
        for (int bx = 0; bx * RB < nvis; ++bx)
            idx_scan_block<DI, 1>(bx, bt, (const uint4*)q_idx, (const uint4*)K_idx, keys, 1, N,
                                  nvis);
        __threadfence_block();
        __syncthreads();
        select_row_stream(kr, nvis, k, cap, out, n_sel + bt, hist, s_red, s_wave, s_pick);
        return;
    }
    constexpr int KS = DI / 32;
    const int lane = tid & 63, wv = tid >> 6, r = lane & 15, grp = lane >> 4;
    const int b = bt / T;
    h8_t qt[KS];   // the token's query in every column
#pragma unroll
    for (int st = 0; st < KS; ++st)
        qt[st] = *(const h8_t*)(q_idx + (size_t)bt * DI + kperm(st, grp));
    for (int c0 = 16 * wv; c0 < nvis; c0 += 16 * (kSelThreads / 64)) {
        const int cell = min(c0 + r, nvis - 1);
        const _Float16* src = K_idx + ((size_t)b * N + cell) * DI;
        h8_t kc[KS];
#pragma unroll
        for (int st = 0; st < KS; ++st)
            kc[st] = *(const h8_t*)(src + kperm(st, grp));
        const float4_t acc = score_block<KS>(kc, qt);
        if (r == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c0 + 4 * grp + e < nvis)
                    kr[c0 + 4 * grp + e] = score_key(acc[e]);
        }
    }
    __threadfence_block();
    __syncthreads();
    select_row_stream(kr, nvis, k, cap, out, n_sel + bt, hist, s_red, s_wave, s_pick);
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
    // fused many-token path (k_idx_sample .. k_sel_cand)
    const bool fused = (T >= kFusedMinTokens && N <= kFusedMaxCells) ||
                       (T == 1 && N > kRowThreads * 64 && N <= kLongFusedMaxCells);
    w.thr = (uint32_t*)take(fused ? BT * 4 : 0);
    w.gcount = (uint32_t*)take(fused ? BT * 4 : 0);
    w.samp = (uint32_t*)take(fused ? BT * kSampleCells * 4 : 0);
    w.fcand = (uint2*)take(fused ? BT * kCandCap * 8 : 0);
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
static void launch_scan_append(const IndexLaunch& a, uint32_t* keys, int nvis_max,
                               const AppendLaunch& ap, hipStream_t s)
{
    constexpr int rows_per_block = (256 / (DI / 8)) * 8;
    dim3 grid((nvis_max + rows_per_block - 1) / rows_per_block, a.B);
    k_idx_scan_append<DI><<<grid, 256, 0, s>>>((const uint4*)a.q_idx, (const uint4*)a.K_idx,
                                               keys, a.N, nvis_max, ap);
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

hipError_t launch_index_topk(const IndexLaunch& a, hipStream_t s, const AppendLaunch* ap)
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
        const AppendLaunch none{};
        // The scan kernel's workgroups write the new tokens while they fit
        // its quantisation lanes; otherwise the append kernel runs first.
        const bool fold = ap && (long long)ap->Hkv * ap->D / 2 <= kRowThreads;
        if (ap && !fold) {
            const hipError_t e = launch_kv_append(*ap, s);
            if (e != hipSuccess)
                return e;
        }
#define QSA_FUSED(DI, KPT)                                                                      \
    do {                                                                                        \
        if (fold)                                                                               \
            k_scan_select<DI, KPT, true><<<a.B, kRowThreads, 0, s>>>(                           \
                q, K, a.ids, a.n_sel, a.N, a.pos0, a.k, a.dense_max, a.cap, *ap);               \
        else                                                                                    \
            k_scan_select<DI, KPT, false><<<a.B, kRowThreads, 0, s>>>(                          \
                q, K, a.ids, a.n_sel, a.N, a.pos0, a.k, a.dense_max, a.cap, none);              \
    } while (0)
        const int kpt = row_select_kpt(a.N);
        if (a.DI == 64) {
            if (kpt <= 4) QSA_FUSED(64, 4); else if (kpt <= 8) QSA_FUSED(64, 8); else QSA_FUSED(64, 16);
        } else {
            if (kpt <= 4) QSA_FUSED(128, 4); else if (kpt <= 8) QSA_FUSED(128, 8); else QSA_FUSED(128, 16);
        }
#undef QSA_FUSED
        return hipGetLastError();
    }
    // One token through the chip-wide scan: the workgroup holding the new
    // cell's row writes the new token while its quantisation lanes fit.
    const bool long1 = any_select && a.T == 1 && a.N > kRowThreads * 64 &&
                       a.N <= kLongFusedMaxCells && a.k <= kCandCap / 2;
    const bool scan_fold = ap && any_select && a.T == 1 && !long1 && ap->T == 1 &&
                           (long long)ap->Hkv * ap->D / 2 <= 256;
    // Every other path: the append as its own kernel first.
    if (ap && !scan_fold) {
        const hipError_t e = launch_kv_append(*ap, s);
        if (e != hipSuccess)
            return e;
    }
    const bool fused = any_select && a.T >= kFusedMinTokens && a.N <= kFusedMaxCells &&
                       nvis_max >= kFusedMinCells && a.k <= kCandCap / 2;
    if (fused) {
        const dim3 gs(kSampleCells / 256, (a.T + 63) / 64, a.B);
        const int ncb = a.T <= 16 ? 1 : 4;   // 16-token column blocks per workgroup
        const int n_cr = (nvis_max + 1023) / 1024, n_tb = (a.T + 16 * ncb - 1) / (16 * ncb);
        const int gc = ((n_cr * a.B + 7) / 8) * 8 * n_tb;
        const _Float16* q = (const _Float16*)a.q_idx;
        const _Float16* K = (const _Float16*)a.K_idx;
#define QSA_FUSED(DI)                                                                          \
    k_idx_sample<DI><<<gs, 256, 0, s>>>(q, K, w.samp, a.T, a.N, a.pos0, nvis_max);             \
    k_sel_thresh<<<BT, 64, 0, s>>>(w.samp, w.thr, w.gcount, a.T, a.pos0, a.k, a.dense_max);   \
    if (ncb == 1)                                                                              \
        k_idx_collect<DI, 1><<<gc, 256, 0, s>>>(q, K, w.thr, w.gcount, w.fcand, a.T, a.N, a.pos0, \
                                                n_cr, n_tb, a.B);                              \
    else                                                                                       \
        k_idx_collect<DI, 4><<<gc, 256, 0, s>>>(q, K, w.thr, w.gcount, w.fcand, a.T, a.N, a.pos0, \
                                                n_cr, n_tb, a.B);                              \
    k_sel_cand<DI, kFusedMaxCells, false><<<BT, kSelThreads, 0, s>>>(                          \
        q, K, w.gcount, w.fcand, w.keys, a.ids, a.n_sel,                                      \
                                              a.T, a.N, a.pos0, a.k, a.dense_max, a.cap)
        if (a.DI == 64) {
            QSA_FUSED(64);
        } else {
            QSA_FUSED(128);
        }
#undef QSA_FUSED
        return hipGetLastError();
    }
    // One token against a row too long for the register select: sampled
    // bound, then the chip-wide scan keeps only the candidates, then the
    // exact select among them (no key array, no chip-wide select).
    if (long1) {
        const dim3 gs(kSampleCells / 256, 1, a.B);
        const _Float16* q = (const _Float16*)a.q_idx;
        const _Float16* K = (const _Float16*)a.K_idx;
#define QSA_LONG1(DI)                                                                          \
    k_idx_sample<DI><<<gs, 256, 0, s>>>(q, K, w.samp, 1, a.N, a.pos0, nvis_max);               \
    k_sel_thresh<<<a.B, 64, 0, s>>>(w.samp, w.thr, w.gcount, 1, a.pos0, a.k, a.dense_max);    \
    k_scan_collect<DI><<<dim3((nvis_max + idx_scan_rows_per_block<DI>() * kScanCollectSpan -   \
                               1) / (idx_scan_rows_per_block<DI>() * kScanCollectSpan),       \
                              a.B),                                                            \
                         256, 0, s>>>((const uint4*)a.q_idx, (const uint4*)a.K_idx, w.thr,     \
                                      w.gcount, w.fcand, a.N, nvis_max);                       \
    k_sel_cand<DI, kLongFusedMaxCells, true><<<a.B, kSelThreads, 0, s>>>(                      \
        q, K, w.gcount, w.fcand, w.keys, a.ids, a.n_sel, 1, a.N, a.pos0, a.k, a.dense_max, a.cap)
        if (a.DI == 64) {
            QSA_LONG1(64);
        } else {
            QSA_LONG1(128);
        }
#undef QSA_LONG1
        return hipGetLastError();
    }
    if (any_select) {
        if (a.T == 1 && scan_fold) {
            if (a.DI == 64)
                launch_scan_append<64>(a, w.keys, nvis_max, *ap, s);
            else
                launch_scan_append<128>(a, w.keys, nvis_max, *ap, s);
        } else if (a.T == 1) {
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
