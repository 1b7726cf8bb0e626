// qsa_window.hip -- the whole decode window in one launch: KV append ->
// index scan -> top-k select -> attention partials -> gated merge.
//
// The audit pages time the QSA step of a decode token as one window of five
// dependent dispatches ("opus r20 track A: MTP map mlock + qsa_attn /
// qsa_merge decode tweaks", section 4 "timings").  For a few problems the
// launch gaps between them cost more than the work, so here one cooperative
// launch runs the five phases with grid-wide barriers between them.  Every
// phase runs the same device code as the separate kernels (qsa_append.h,
// qsa_select.h, qsa_attend_mma.h, qsa_merge.h); only the top-k of a row is
// taken by a 256-thread exact select with the row in registers (rows of up
// to 16384 visible cells) instead of the 1024-thread one, which keeps the
// same cells, so the results equal the multi-launch path bit for bit.
//
// Barrier: a counter and a generation word in device memory (zero when the
// code object loads).  A workgroup makes its writes visible (agent-scope
// release), adds itself to the counter; the last one resets the counter and
// advances the generation; the others wait for the generation to move
// (agent-scope acquire).  The counter is back at zero after every barrier,
// so launches follow each other without any set-up.  The cooperative launch
// guarantees that all workgroups are resident, so every wait ends; the wait
// is bounded anyway: a wait that gives up sets the workspace's status word
// (cleared by workgroup 0 at the start of each launch) and the kernel still
// runs to the end, with invalid results and the barrier words of the device
// left inconsistent.  Launches on one GPU must not overlap (they share the
// barrier words).
#include <atomic>

#include "qsa_append.h"
#include "qsa_attend_mma.h"
#include "qsa_launch.h"
#include "qsa_merge.h"
#include "qsa_select.h"

namespace qsa {

// The barrier words, each on a cache line of its own (the waiting
// workgroups poll the generation; the arrivals update the counter).
struct WindowBarrier {
    alignas(256) unsigned int count;
    alignas(256) unsigned int gen;
};
static __device__ WindowBarrier g_win;

// Bound of one barrier wait, in polls (about a second): far beyond any phase
// of a decode window, so it only ends a wait whose grid cannot finish.
constexpr unsigned kSpinLimit = 1u << 20;

// Longest row (visible cells) the window selects: one workgroup holds the
// row's keys in registers (kSelThreads x 64).
constexpr int kWindowMaxVisible = kSelThreads * 64;

struct WindowArgs {
    AppendLaunch ap;
    long long q_lanes, n_quant, n_idx;  // append item counts (as launch_kv_append)
    IndexLaunch ix;
    AttnLaunch at;
    uint32_t* keys;      // [B][N] score keys
    uint32_t* status;    // nonzero after a barrier timeout
    int n_scan_x;        // scan workgroups per problem
    int n_attend;        // attention workgroups
    int n_merge;         // merge workgroups
    int selects;         // some token keeps fewer cells than it sees
};

// Grid-wide barrier (see the header).  Every wave first waits until its own
// memory operations are complete, so the device-scope release that thread 0
// then performs (write-back of this XCD's L2) covers the whole workgroup's
// writes.  Waiting workgroups poll the generation with relaxed loads (read
// from the device-coherent level, no cache invalidation per poll) and make
// one acquire when it moves.  `gen` is this workgroup's view of the
// generation, held by thread 0.
__device__ __forceinline__ void grid_sync(unsigned& gen, uint32_t* status)
{
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned g = gen;
        __threadfence();
        if (atomicAdd(&g_win.count, 1u) == gridDim.x - 1) {
            atomicExch(&g_win.count, 0u);
            __threadfence();
            atomicAdd(&g_win.gen, 1u);
        } else {
            unsigned spins = 0;
            while (__hip_atomic_load(&g_win.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins == kSpinLimit) {
                    atomicOr(status, 1u);
                    break;
                }
            }
        }
        __threadfence();
        gen = g + 1;
    }
    __syncthreads();
}

// Exact top-k of one problem's row (or every cell when it keeps them all).
__device__ __forceinline__ void window_select(const uint32_t* kr, int nvis, int k, int dense_max,
                                              int cap, int32_t* out, int32_t* n_out,
                                              uint32_t* hist, uint32_t* s_red, uint32_t* s_wave,
                                              uint32_t* s_pick)
{
    if (!token_selects(nvis, k, dense_max))
        dense_row_wg(nvis, cap, out, n_out);
    else if (nvis <= kSelThreads * 8)
        select_row_regs<8>(kr, nvis, k, cap, out, n_out, hist, s_red, s_wave, s_pick);
    else if (nvis <= kSelThreads * 16)
        select_row_regs<16>(kr, nvis, k, cap, out, n_out, hist, s_red, s_wave, s_pick);
    else if (nvis <= kSelThreads * 32)
        select_row_regs<32>(kr, nvis, k, cap, out, n_out, hist, s_red, s_wave, s_pick);
    else
        select_row_regs<64>(kr, nvis, k, cap, out, n_out, hist, s_red, s_wave, s_pick);
}

template <int G, int D, int DI, int EPL>
__global__ __launch_bounds__(256, 1) void k_decode_window(WindowArgs w)
{
    unsigned gen = 0;
    if (threadIdx.x == 0) {
        gen = __hip_atomic_load(&g_win.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (blockIdx.x == 0)
            *w.status = 0;
    }
    const int nblk = gridDim.x;

    // 1. append the step's token into its cell
    append_blocks(w.ap, w.q_lanes, w.n_quant, w.n_idx, blockIdx.x, nblk);
    grid_sync(gen, w.status);

    // 2. score every visible cell (one token per problem)
    const IndexLaunch& ix = w.ix;
    const int nvis = ix.pos0 + 1;
    if (w.selects) {
        for (int v = blockIdx.x; v < w.n_scan_x * ix.B; v += nblk)
            idx_scan_block<DI, 1>(v % w.n_scan_x, v / w.n_scan_x, (const uint4*)ix.q_idx,
                                  (const uint4*)ix.K_idx, w.keys, 1, ix.N, nvis);
    }
    grid_sync(gen, w.status);

    // 3. top-k of each problem's row
    {
        __shared__ uint32_t hist[kBins];
        __shared__ uint32_t s_wave[kSelThreads / 64];
        __shared__ uint32_t s_pick[2];
        __shared__ uint32_t s_red[8];
        for (int v = blockIdx.x; v < ix.B; v += nblk) {
            window_select(w.keys + (size_t)v * ix.N, nvis, ix.k, ix.dense_max, ix.cap,
                          ix.ids + (size_t)v * ix.cap, ix.n_sel + v, hist, s_red, s_wave,
                          s_pick);
            __syncthreads();
        }
    }
    grid_sync(gen, w.status);

    // 4. attention partials
    const AttnLaunch& a = w.at;
    for (int v = blockIdx.x; v < w.n_attend; v += nblk) {
        attend_mma_block<G, D, false, true>(
            v, a.q, a.Kq, (const uint8_t*)a.Ksc, a.Vq, (const uint8_t*)a.Vsc, a.kq_cs, a.ksc_cs,
            a.vq_cs, a.vsc_cs, a.kq_bs, a.ksc_bs, a.vq_bs, a.vsc_bs, a.ids, a.n_sel, a.pm, a.pl,
            a.po, a.T, a.Hq, a.Hkv, a.P, a.cap, a.N, a.B * a.T, a.scale);
        __syncthreads();   // LDS of this item group free before the next
    }
    grid_sync(gen, w.status);

    // 5. merge (with the output gate when given)
    const long long rows = (long long)a.B * a.T * a.Hq;
    for (int v = blockIdx.x; v < w.n_merge; v += nblk)
        merge_block<D, EPL, false>(v, a.pm, a.pl, a.po, a.out, a.P, rows, a.gate, 0);
}

// Maximum co-resident workgroups of one instantiation on the current device
// (queried once per device; 0 if the query fails).
template <int G, int D, int DI, int EPL>
static int window_capacity()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 0;
    int cap = cached[dev].load(std::memory_order_relaxed);
    if (cap > 0)
        return cap;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode_window<G, D, DI, EPL>, 256,
                                                     0) != hipSuccess)
        return 0;
    cap = cus * per_cu;
    cached[dev].store(cap, std::memory_order_relaxed);
    return cap;
}

template <int G, int D, int DI, int EPL>
static hipError_t launch_window_t(WindowArgs& w, hipStream_t s)
{
    const int cap = window_capacity<G, D, DI, EPL>();
    if (cap <= 0)
        return hipErrorInvalidConfiguration;
    const int need = std::max(std::max(w.n_scan_x * w.ix.B, w.ix.B),
                              std::max(std::max(w.n_attend, w.n_merge), 1));
    const int grid = std::min(cap, need);
    void* args[] = {&w};
    return hipLaunchCooperativeKernel((const void*)k_decode_window<G, D, DI, EPL>, dim3(grid),
                                      dim3(256), args, 0, s);
}

bool window_supported(int G, int D, int DI, int P, int nvis)
{
    return ((G == 12 && D == 256) || (G == 4 && D == 64)) && (DI == 64 || DI == 128) &&
           P % kMmaWaves == 0 && P <= 64 && nvis <= kWindowMaxVisible;
}

size_t window_workspace_bytes(int B, int N, int Hq, int P, int D)
{
    const size_t rows = (size_t)B * Hq * P;
    return 256 + ((size_t)B * N * 4 + 255) / 256 * 256 + rows * (2 + (size_t)D) * 4;
}

hipError_t launch_window(const AppendLaunch& ap, const IndexLaunch& ix, const AttnLaunch& at0,
                         void* ws, hipStream_t s)
{
    WindowArgs w;
    w.ap = ap;
    w.q_lanes = (long long)ap.B * ap.T * ap.Hkv * (ap.D / 32) * 2 * 8;
    w.n_quant = (w.q_lanes + 255) / 256 * 256;
    w.n_idx = ap.kidx_new ? (long long)ap.B * ap.T * (ap.DI / 4) : 0;
    w.ix = ix;
    w.at = at0;
    char* p = (char*)ws;
    w.status = (uint32_t*)p;
    w.keys = (uint32_t*)(p + 256);
    const size_t rows = (size_t)at0.B * at0.T * at0.Hq * at0.P;
    float* part = (float*)(p + 256 + ((size_t)ix.B * ix.N * 4 + 255) / 256 * 256);
    w.at.pm = part;
    w.at.pl = part + rows;
    w.at.po = part + 2 * rows;
    const int nvis = ix.pos0 + 1;
    w.selects = (nvis > ix.dense_max && nvis > ix.k) ? 1 : 0;
    const int rows_per_block = (256 / (ix.DI / 8)) * 8;
    w.n_scan_x = (nvis + rows_per_block - 1) / rows_per_block;
    const long long groups = ((long long)at0.B * at0.T * at0.P + kMmaWaves - 1) / kMmaWaves;
    w.n_attend = (int)((groups + 7) / 8 * 8LL * at0.Hkv);
    const bool wide = at0.P >= 32;
    const long long lanes = (long long)at0.B * at0.T * at0.Hq * (at0.D / (wide ? 1 : 4));
    w.n_merge = (int)((lanes + 255) / 256);
    const int G = at0.Hq / at0.Hkv;
#define QSA_WIN(GG, DD, DDI)                                                              \
    (wide ? launch_window_t<GG, DD, DDI, 1>(w, s) : launch_window_t<GG, DD, DDI, 4>(w, s))
    if (G == 12 && at0.D == 256)
        return ix.DI == 64 ? QSA_WIN(12, 256, 64) : QSA_WIN(12, 256, 128);
    if (G == 4 && at0.D == 64)
        return ix.DI == 64 ? QSA_WIN(4, 64, 64) : QSA_WIN(4, 64, 128);
#undef QSA_WIN
    return hipErrorInvalidValue;
}

}  // namespace qsa
