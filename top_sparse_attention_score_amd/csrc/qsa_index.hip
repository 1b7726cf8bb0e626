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
//   k_idx_scan   decode (T <= 16): streams every visible cell's fp16 key row
//                once, 16 lanes per row (coalesced), scores it against all T
//                tokens with v_dot2 (fp16 x fp16 products, fp32
//                accumulation) and sums the row across its lanes with DPP.
//   k_idx_gemm   prompt chunk (T > 16): [T x d_idx] x [d_idx x N] on MFMA
//                (v_mfma_f32_16x16x16_f16), 64 tokens x 64 cells per
//                workgroup.
//   k_select_row one 1024-thread workgroup per token: 3-digit radix select
//                (11/11/10 bits) of the k-th largest key in LDS histograms,
//                then an ordered compaction that writes the kept ids in
//                ascending cell order, giving the tie quota at the threshold
//                to the lowest cell indices.
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

// ---------------------------------------------------------------- gemm ---

// Each wave computes 32 tokens x 32 cells as 2 x 2 MFMA 16x16 blocks.  In an
// MFMA step lane group g (lanes 16g..16g+15) supplies k-slots 4g..4g+3; here
// lane group g instead supplies row elements [g*DI/4 + 4s, g*DI/4 + 4s + 4) at
// step s for both operands, so over the DI/16 steps every element of the dot
// product is used exactly once (a permutation of the reduction index).
template <int DI>
__global__ __launch_bounds__(256) void k_idx_gemm(const _Float16* __restrict__ q_idx,
                                                  const _Float16* __restrict__ K_idx,
                                                  uint32_t* __restrict__ keys, int T, int N,
                                                  int nvis_max)
{
    constexpr int KQ = DI / 4;
    constexpr int STEPS = DI / 16;
    const int b = blockIdx.z;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tok0 = blockIdx.y * 64 + (w >> 1) * 32;
    const int cell0 = blockIdx.x * 64 + (w & 1) * 32;
    const int r = lane & 15, grp = lane >> 4;

    half4_t a[2][STEPS], kb[2][STEPS];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tok = min(tok0 + 16 * i + r, T - 1);
        const half4_t* src = (const half4_t*)(q_idx + ((size_t)b * T + tok) * DI + grp * KQ);
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
            a[i][s] = src[s];
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int cell = min(cell0 + 16 * jj + r, nvis_max - 1);
        const half4_t* src = (const half4_t*)(K_idx + ((size_t)b * N + cell) * DI + grp * KQ);
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
            kb[jj][s] = src[s];
    }
    float4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
            acc[i][jj] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x16f16(a[i][s], kb[jj][s],
                                                                   acc[i][jj], 0, 0, 0);
    // Result layout of a 16x16 block: lane l, element e holds row 4*(l/16)+e,
    // column l%16 (rows = tokens, columns = cells).
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tok = tok0 + 16 * i + 4 * grp + e;
                const int cell = cell0 + 16 * jj + r;
                if (tok < T && cell < nvis_max)
                    keys[((size_t)b * T + tok) * N + cell] = score_key(acc[i][jj][e]);
            }
}

// -------------------------------------------------------------- select ---

constexpr int kSelThreads = 1024;

// Exclusive prefix sum over the 1024 threads of the block; `total` receives
// the block sum.  s_wave holds 16 words of LDS.
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

__global__ __launch_bounds__(kSelThreads) void k_select_row(const uint32_t* __restrict__ keys,
                                                            int32_t* __restrict__ ids,
                                                            int32_t* __restrict__ n_sel, int T,
                                                            int N, int pos0, int k,
                                                            int dense_max, int cap)
{
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t s_wave[kSelThreads / 64];
    __shared__ uint32_t s_pick[2];
    if (threadIdx.x == 0) {
        s_pick[0] = 0u;
        s_pick[1] = 0u;
    }

    const int bt = blockIdx.x;
    const int t = bt % T;
    const int nvis = pos0 + t + 1;
    const int tid = threadIdx.x;
    int32_t* row = ids + (size_t)bt * cap;

    if (nvis <= dense_max || nvis <= k) {
        // Dense fallback, or no more visible cells than k: keep them all.
        for (int i = tid; i < cap; i += kSelThreads)
            row[i] = (i < nvis) ? i : -1;
        if (tid == 0)
            n_sel[bt] = nvis;
        return;
    }

    const uint32_t* kr = keys + (size_t)bt * N;
    uint32_t prefix = 0u, pmask = 0u;
    uint32_t need = (uint32_t)k;  // rank (from the top) still to locate

    // Radix select over the 32-bit key: digits of 11, 11 and 10 bits.
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = (pass == 0) ? 21 : (pass == 1) ? 10 : 0;
        const int nb = (pass == 2) ? 1024 : 2048;
        for (int i = tid; i < nb; i += kSelThreads)
            hist[i] = 0u;
        __syncthreads();
        for (int j = tid; j < nvis; j += kSelThreads) {
            const uint32_t u = kr[j];
            if ((u & pmask) == prefix)
                atomicAdd(&hist[(u >> shift) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        // Walk bins from the top: thread tid owns the bins at descending
        // positions 2*tid, 2*tid+1 (2048 bins) or tid (1024 bins).
        uint32_t c_hi, c_lo;
        int b_hi;
        if (nb == 2048) {
            b_hi = nb - 1 - 2 * tid;
            c_hi = hist[b_hi];
            c_lo = hist[b_hi - 1];
        } else {
            b_hi = nb - 1 - tid;
            c_hi = hist[b_hi];
            c_lo = 0u;
        }
        uint32_t total;
        const uint32_t above = block_excl_scan(c_hi + c_lo, total, s_wave);
        if (above < need && need <= above + c_hi) {
            s_pick[0] = (uint32_t)b_hi;
            s_pick[1] = above;
        } else if (nb == 2048 && above + c_hi < need && need <= above + c_hi + c_lo) {
            s_pick[0] = (uint32_t)(b_hi - 1);
            s_pick[1] = above + c_hi;
        }
        __syncthreads();
        const uint32_t bin = s_pick[0];
        need -= s_pick[1];
        prefix |= bin << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        __syncthreads();
    }

    // prefix is now the key of the k-th kept cell; `need` of the cells with
    // exactly that key are kept, lowest indices first.  Ordered compaction.
    const uint32_t tau = prefix;
    uint32_t run_gt = 0u, run_eq = 0u;
#pragma unroll 1
    for (int base = 0; base < nvis; base += kSelThreads) {
        const int j = base + tid;
        const uint32_t u = (j < nvis) ? kr[j] : 0u;
        const uint32_t gt = (u > tau) ? 1u : 0u;
        const uint32_t eq = (u == tau) ? 1u : 0u;
        uint32_t total;
        const uint32_t ex = block_excl_scan(gt | (eq << 16), total, s_wave);
        const uint32_t gt_ex = ex & 0xffffu, eq_ex = ex >> 16;
        const uint32_t eq_before = run_eq + eq_ex;
        if (gt || (eq && eq_before < need)) {
            const uint32_t pos = run_gt + gt_ex + min(eq_before, need);
            if (pos < (uint32_t)k)
                row[pos] = j;
        }
        run_gt += total & 0xffffu;
        run_eq += total >> 16;
        if (run_gt + min(run_eq, need) >= (uint32_t)k)
            break;
    }
    for (int i = k + tid; i < cap; i += kSelThreads)
        row[i] = -1;
    if (tid == 0)
        n_sel[bt] = k;
}

// ------------------------------------------------------------- launch ---

size_t index_workspace_bytes(int B, int T, int N)
{
    return (size_t)B * (size_t)T * (size_t)N * sizeof(uint32_t);
}

template <int DI>
static void launch_scan(const IndexLaunch& a, int nvis_max, hipStream_t s)
{
    constexpr int rows_per_block = (256 / (DI / 8)) * 8;
    dim3 grid((nvis_max + rows_per_block - 1) / rows_per_block, a.B);
    const uint4* q = (const uint4*)a.q_idx;
    const uint4* K = (const uint4*)a.K_idx;
    if (a.T <= 1)
        k_idx_scan<DI, 1><<<grid, 256, 0, s>>>(q, K, a.keys, a.T, a.N, nvis_max);
    else if (a.T <= 2)
        k_idx_scan<DI, 2><<<grid, 256, 0, s>>>(q, K, a.keys, a.T, a.N, nvis_max);
    else if (a.T <= 4)
        k_idx_scan<DI, 4><<<grid, 256, 0, s>>>(q, K, a.keys, a.T, a.N, nvis_max);
    else if (a.T <= 8)
        k_idx_scan<DI, 8><<<grid, 256, 0, s>>>(q, K, a.keys, a.T, a.N, nvis_max);
    else
        k_idx_scan<DI, 16><<<grid, 256, 0, s>>>(q, K, a.keys, a.T, a.N, nvis_max);
}

template <int DI>
static void launch_gemm(const IndexLaunch& a, int nvis_max, hipStream_t s)
{
    dim3 grid((nvis_max + 63) / 64, (a.T + 63) / 64, a.B);
    k_idx_gemm<DI><<<grid, 256, 0, s>>>((const _Float16*)a.q_idx, (const _Float16*)a.K_idx,
                                         a.keys, a.T, a.N, nvis_max);
}

hipError_t launch_index_topk(const IndexLaunch& a, hipStream_t s)
{
    // Scores are needed only when some token keeps fewer cells than it sees.
    const int nvis_max = a.pos0 + a.T;  // cells visible to the last token
    const bool any_select = nvis_max > a.dense_max && nvis_max > a.k;
    if (any_select) {
        if (a.T <= 16) {
            if (a.DI == 64)
                launch_scan<64>(a, nvis_max, s);
            else
                launch_scan<128>(a, nvis_max, s);
        } else {
            if (a.DI == 64)
                launch_gemm<64>(a, nvis_max, s);
            else
                launch_gemm<128>(a, nvis_max, s);
        }
    }
    k_select_row<<<dim3((unsigned)(a.B * a.T)), kSelThreads, 0, s>>>(
        a.keys, a.ids, a.n_sel, a.T, a.N, a.pos0, a.k, a.dense_max, a.cap);
    return hipGetLastError();
}

}  // namespace qsa
