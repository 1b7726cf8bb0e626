// qsa_launch.h -- host-side launchers of the QSA kernels (internal).
// Arguments are validated by the C-ABI layer before these are called; each
// launcher only enqueues kernels and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qsa {

struct IndexLaunch {
    int B, T, N, DI, k, pos0, dense_max, cap;
    const void* q_idx;
    const void* K_idx;
    int32_t* ids;
    int32_t* n_sel;
    void* ws;  // workspace of index_workspace_bytes(B, T, N) bytes
};

// Bytes of workspace the index path needs (score keys, histograms,
// candidates, per-tile counts).
size_t index_workspace_bytes(int B, int T, int N);
// Largest n_cells the select kernels handle.
int index_max_cells();

struct AttnLaunch;
struct AppendLaunch;

// With `ap` (the same step's append: T == a.T, pos0 == a.pos0, same B and
// N) the new tokens are written into the cache first: inside the scan
// kernel where one workgroup serves one problem, else by the append kernel.
hipError_t launch_index_topk(const IndexLaunch& a, hipStream_t s,
                             const AppendLaunch* ap = nullptr);

struct AttnLaunch {
    int B, T, Hq, Hkv, D, P, cap, N;
    float scale;
    bool q_f16, out_f16;
    int algo;  // qsa_attend_algo
    const void* q;
    const int8_t* Kq;
    const void* Ksc;
    const int8_t* Vq;
    const void* Vsc;
    long long kq_cs, ksc_cs, vq_cs, vsc_cs;  // cell strides, bytes
    long long kq_bs, ksc_bs, vq_bs, vsc_bs;  // batch strides, bytes
    const int32_t* ids;
    const int32_t* n_sel;
    float* pm;
    float* pl;
    float* po;
    void* out;
    const void* gate;  // output gate (q layout and dtype) or null
};

// True if a kernel variant exists for (G, D, q dtype).
bool attend_supported(int G, int D);

struct AppendLaunch {
    int B, T, N, pos0, Hkv, D, DI;
    const float* k_new;
    const float* v_new;
    const float* kidx_new;  // may be null
    int8_t* Kq;
    uint16_t* Ksc;
    int8_t* Vq;
    uint16_t* Vsc;
    uint16_t* K_idx;
    long long kq_cs, ksc_cs, vq_cs, vsc_cs;  // cell strides, bytes
    long long kq_bs, ksc_bs, vq_bs, vsc_bs;  // batch strides, bytes
};

hipError_t launch_kv_append(const AppendLaunch& a, hipStream_t s);

hipError_t launch_attend(const AttnLaunch& a, hipStream_t s);
// Matrix-core attend kernel (qsa_attend_mma.hip); false if no variant fits.
// With a.out set (P in {1, 2, 4}) the kernel also merges the chunks, applies
// a.gate and writes a.out instead of the partials.
// With a.P a multiple of 4 above 4 and at least 512 (token, KV head) pairs,
// the kernel runs several chunks per wave (attend_mch); then a.out, if set,
// also makes it merge the partials it wrote (a.pm/pl/po must be set).
bool launch_attend_mma(const AttnLaunch& a, hipStream_t s);
bool attend_mch(const AttnLaunch& a);
hipError_t launch_merge(const AttnLaunch& a, hipStream_t s);

// Single-launch decode window (qsa_window.hip): append, index, attend and
// gated merge of one token per problem in one cooperative kernel.
bool window_supported(int G, int D, int DI, int P, int nvis);
// Workspace: status word, [B][N] score keys, partials.
size_t window_workspace_bytes(int B, int N, int Hq, int P, int D);
// `ap`, `ix`, `at` describe the same T = 1 problems (the caller checks that);
// the partial pointers of `at` are ignored (the window keeps them in `ws`).
hipError_t launch_window(const AppendLaunch& ap, const IndexLaunch& ix, const AttnLaunch& at,
                         void* ws, hipStream_t s);

}  // namespace qsa
