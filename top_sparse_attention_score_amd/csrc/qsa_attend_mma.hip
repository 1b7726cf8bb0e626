// qsa_attend_mma.hip -- split-KV attention partials on the gfx950 matrix
// cores: the kernel over the device function of qsa_attend_mma.h and its
// launchers.
#include "qsa_attend_mma.h"
#include "qsa_launch.h"

namespace qsa {

template <int G, int D, bool QF16, bool SHQ>
__global__ __launch_bounds__(64 * kMmaWaves, (SHQ || QF16) ? 2 : 1) void k_attend_mma(
    const void* __restrict__ q, const int8_t* __restrict__ Kq, const uint8_t* __restrict__ Ksc,
    const int8_t* __restrict__ Vq, const uint8_t* __restrict__ Vsc, long long kq_cs,
    long long ksc_cs, long long vq_cs, long long vsc_cs, long long kq_bs, long long ksc_bs,
    long long vq_bs, long long vsc_bs, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ n_sel, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ po, int T, int Hq, int Hkv, int P, int cap, int N, int BT, float scale)
{
    attend_mma_block<G, D, QF16, SHQ>(blockIdx.x, q, Kq, Ksc, Vq, Vsc, kq_cs, ksc_cs, vq_cs,
                                      vsc_cs, kq_bs, ksc_bs, vq_bs, vsc_bs, ids, n_sel, pm, pl,
                                      po, T, Hq, Hkv, P, cap, N, BT, scale);
}

// Attention with the merge (and output gate) fused: P in {1, 2, 4}, so each
// workgroup's four items are all the chunks of whole tokens.
template <int G, int D, bool QF16, bool SHQ>
__global__ __launch_bounds__(64 * kMmaWaves, (SHQ || QF16) ? 2 : 1) void k_attend_merge_mma(
    const void* __restrict__ q, const int8_t* __restrict__ Kq, const uint8_t* __restrict__ Ksc,
    const int8_t* __restrict__ Vq, const uint8_t* __restrict__ Vsc, long long kq_cs,
    long long ksc_cs, long long vq_cs, long long vsc_cs, long long kq_bs, long long ksc_bs,
    long long vq_bs, long long vsc_bs, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ n_sel, int T, int Hq, int Hkv, int P, int cap, int N, int BT,
    float scale, void* __restrict__ out, const void* __restrict__ gate, int out_f16)
{
    attend_mma_block<G, D, QF16, SHQ, true>(blockIdx.x, q, Kq, Ksc, Vq, Vsc, kq_cs, ksc_cs,
                                            vq_cs, vsc_cs, kq_bs, ksc_bs, vq_bs, vsc_bs, ids,
                                            n_sel, nullptr, nullptr, nullptr, T, Hq, Hkv, P, cap,
                                            N, BT, scale, out, gate, out_f16);
}

// Several chunks per wave: one workgroup per (token, KV head), the four
// waves taking chunks w, w + 4, ... (P a multiple of 4); with out set, the
// workgroup also merges the token's partials and writes the gated output.
template <int G, int D, bool QF16>
__global__ __launch_bounds__(64 * kMmaWaves, 2) void k_attend_mch_mma(
    const void* __restrict__ q, const int8_t* __restrict__ Kq, const uint8_t* __restrict__ Ksc,
    const int8_t* __restrict__ Vq, const uint8_t* __restrict__ Vsc, long long kq_cs,
    long long ksc_cs, long long vq_cs, long long vsc_cs, long long kq_bs, long long ksc_bs,
    long long vq_bs, long long vsc_bs, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ n_sel, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ po, int T, int Hq, int Hkv, int P, int cap, int N, int BT, float scale,
    void* __restrict__ out, const void* __restrict__ gate, int out_f16)
{
    attend_mma_block<G, D, QF16, true, false, true>(
        blockIdx.x, q, Kq, Ksc, Vq, Vsc, kq_cs, ksc_cs, vq_cs, vsc_cs, kq_bs, ksc_bs, vq_bs, vsc_bs,
        ids, n_sel, pm, pl, po, T, Hq, Hkv, P, cap, N, BT, scale, out, gate, out_f16);
}

// Grid of the matrix kernels: whole groups of kMmaWaves items (with several
// chunks per wave: one group per token), 8 Hkv workgroups per 8 groups (see
// attend_mma_block).
static unsigned mma_grid(const AttnLaunch& a, bool mch = false)
{
    const long long items = (long long)a.B * a.T * a.P;
    const long long groups = mch ? (long long)a.B * a.T : (items + kMmaWaves - 1) / kMmaWaves;
    const long long per = 8LL * a.Hkv;  // workgroups per 8 groups
    return (unsigned)((groups + 7) / 8 * per);
}

bool attend_mch(const AttnLaunch& a)
{
    // Enough (token, KV head) workgroups for two per CU on 256 CUs.
    return a.algo != 2 && a.P % kMmaWaves == 0 && a.P > kMmaWaves &&
           (long long)a.B * a.T * a.Hkv >= 512;
}

template <int G, int D, bool QF16>
static void launch_mch_mma_gdq(const AttnLaunch& a, hipStream_t s)
{
    k_attend_mch_mma<G, D, QF16><<<mma_grid(a, true), 64 * kMmaWaves, 0, s>>>(
        a.q, a.Kq, (const uint8_t*)a.Ksc, a.Vq, (const uint8_t*)a.Vsc, a.kq_cs, a.ksc_cs, a.vq_cs,
        a.vsc_cs, a.kq_bs, a.ksc_bs, a.vq_bs, a.vsc_bs, a.ids, a.n_sel, a.pm, a.pl, a.po, a.T,
        a.Hq, a.Hkv, a.P, a.cap, a.N, a.B * a.T, a.scale, a.out, a.gate, a.out_f16 ? 1 : 0);
}

template <int G, int D, bool QF16>
static void launch_merge_mma_gdq(const AttnLaunch& a, hipStream_t s)
{
    const unsigned grid = mma_grid(a);
#define QSA_MMA_ARGS                                                                         \
    a.q, a.Kq, (const uint8_t*)a.Ksc, a.Vq, (const uint8_t*)a.Vsc, a.kq_cs, a.ksc_cs, a.vq_cs, \
        a.vsc_cs, a.kq_bs, a.ksc_bs, a.vq_bs, a.vsc_bs, a.ids, a.n_sel, a.T, a.Hq, a.Hkv, a.P, \
        a.cap, a.N, a.B * a.T, a.scale, a.out, a.gate, a.out_f16 ? 1 : 0
    if (a.P == kMmaWaves)
        k_attend_merge_mma<G, D, QF16, true><<<grid, 64 * kMmaWaves, 0, s>>>(QSA_MMA_ARGS);
    else
        k_attend_merge_mma<G, D, QF16, false><<<grid, 64 * kMmaWaves, 0, s>>>(QSA_MMA_ARGS);
#undef QSA_MMA_ARGS
}

template <int G, int D, bool QF16>
static void launch_mma_gdq(const AttnLaunch& a, hipStream_t s)
{
    if (attend_mch(a)) {
        launch_mch_mma_gdq<G, D, QF16>(a, s);
        return;
    }
    if (a.out) {
        launch_merge_mma_gdq<G, D, QF16>(a, s);
        return;
    }
    const unsigned grid = mma_grid(a);
#define QSA_MMA_ARGS                                                                         \
    a.q, a.Kq, (const uint8_t*)a.Ksc, a.Vq, (const uint8_t*)a.Vsc, a.kq_cs, a.ksc_cs, a.vq_cs, \
        a.vsc_cs, a.kq_bs, a.ksc_bs, a.vq_bs, a.vsc_bs, a.ids, a.n_sel, a.pm, a.pl, a.po, a.T, \
        a.Hq, a.Hkv, a.P, a.cap, a.N, a.B * a.T, a.scale
    if (a.P % kMmaWaves == 0)
        k_attend_mma<G, D, QF16, true><<<grid, 64 * kMmaWaves, 0, s>>>(QSA_MMA_ARGS);
    else
        k_attend_mma<G, D, QF16, false><<<grid, 64 * kMmaWaves, 0, s>>>(QSA_MMA_ARGS);
#undef QSA_MMA_ARGS
}

template <int G, int D>
static void launch_mma_gd(const AttnLaunch& a, hipStream_t s)
{
    if (a.q_f16)
        launch_mma_gdq<G, D, true>(a, s);
    else
        launch_mma_gdq<G, D, false>(a, s);
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
