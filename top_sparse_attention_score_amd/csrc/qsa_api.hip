// qsa_api.hip -- the C ABI declared in include/qsa.h: argument validation,
// defaults, and dispatch to the kernel launchers.  Every check happens on the
// host before anything is enqueued; nothing here allocates or synchronises.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "qsa.h"
#include "qsa_launch.h"

// Workspace of qsa_index_topk_noalloc: a fixed array in device memory, one
// per GPU (each device that loads the library holds its own copy until the
// process ends).  Host code never names it directly: the array's name is a
// host-side stand-in, not a device address, so its address on each device is
// taken once with hipGetSymbolAddress and kept in g_scratch below.
static __device__ __align__(256) unsigned char scratch[QSA_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on device dev (made current for the lookup).
hipError_t scratch_address(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev)
            e = hipSetDevice(dev);
        void* p = nullptr;
        if (e == hipSuccess)
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess)
                e = e2;
        }
        g_scratch[dev] = (e == hipSuccess) ? p : nullptr;
        g_scratch_err[dev] = e;
    });
    *out = g_scratch[dev];
    return g_scratch_err[dev];
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int check_index(const qsa_index_desc* d)
{
    if (!d)
        return QSA_ERR_INVALID_ARG;
    if (d->batch < 1 || d->T < 1 || d->n_cells < 1 || d->k < 1 || d->pos0 < 0 ||
        d->dense_max < 0 || d->ids_cap < 1)
        return QSA_ERR_INVALID_ARG;
    if ((long long)d->pos0 + d->T > d->n_cells)
        return QSA_ERR_INVALID_ARG;
    if (d->k > d->ids_cap || d->dense_max > d->ids_cap)
        return QSA_ERR_INVALID_ARG;
    if (d->d_idx != 64 && d->d_idx != 128)
        return QSA_ERR_UNSUPPORTED;
    if (d->batch > 65535 || (long long)d->batch * d->T > 65535)
        return QSA_ERR_UNSUPPORTED;
    if (d->n_cells > qsa::index_max_cells() || (long long)d->ids_cap > INT_MAX / 2)
        return QSA_ERR_UNSUPPORTED;
    return QSA_OK;
}

// Fills `L` from the descriptor (defaults for zero strides) and validates it.
int check_attn(const qsa_attn_desc* d, qsa::AttnLaunch* L)
{
    if (!d)
        return QSA_ERR_INVALID_ARG;
    if (d->batch < 1 || d->T < 1 || d->Hq < 1 || d->Hkv < 1 || d->D < 32 || d->P < 1 ||
        d->ids_cap < 1 || d->n_cells < 1)
        return QSA_ERR_INVALID_ARG;
    if (d->Hq % d->Hkv != 0 || d->D % 32 != 0 || !isfinite(d->scale))
        return QSA_ERR_INVALID_ARG;
    if ((d->q_dtype != QSA_F32 && d->q_dtype != QSA_F16) ||
        (d->out_dtype != QSA_F32 && d->out_dtype != QSA_F16))
        return QSA_ERR_INVALID_ARG;
    if (d->algo < QSA_ATTEND_AUTO || d->algo > QSA_ATTEND_VECTOR)
        return QSA_ERR_INVALID_ARG;
    if (d->P > 64)
        return QSA_ERR_UNSUPPORTED;
    if (!qsa::attend_supported(d->Hq / d->Hkv, d->D))
        return QSA_ERR_UNSUPPORTED;
    const long long bt = (long long)d->batch * d->T;
    if (bt * d->P > INT_MAX || bt * d->Hq * d->P > INT_MAX || d->Hkv > 65535)
        return QSA_ERR_UNSUPPORTED;

    const long long row = (long long)d->Hkv * d->D;           // int8 codes per cell
    const long long srow = (long long)d->Hkv * (d->D / 32) * 2;  // scale bytes per cell
    L->kq_cs = d->kq_cell_stride ? d->kq_cell_stride : row;
    L->vq_cs = d->vq_cell_stride ? d->vq_cell_stride : row;
    L->ksc_cs = d->ksc_cell_stride ? d->ksc_cell_stride : srow;
    L->vsc_cs = d->vsc_cell_stride ? d->vsc_cell_stride : srow;
    L->kq_bs = d->kq_batch_stride ? d->kq_batch_stride : L->kq_cs * d->n_cells;
    L->vq_bs = d->vq_batch_stride ? d->vq_batch_stride : L->vq_cs * d->n_cells;
    L->ksc_bs = d->ksc_batch_stride ? d->ksc_batch_stride : L->ksc_cs * d->n_cells;
    L->vsc_bs = d->vsc_batch_stride ? d->vsc_batch_stride : L->vsc_cs * d->n_cells;
    if (L->kq_cs < 0 || L->vq_cs < 0 || L->ksc_cs < 0 || L->vsc_cs < 0 || L->kq_bs < 0 ||
        L->vq_bs < 0 || L->ksc_bs < 0 || L->vsc_bs < 0)
        return QSA_ERR_INVALID_ARG;
    const long long srow_g = d->D / 16;  // scale bytes of one head row
    if (L->kq_cs % 16 || L->vq_cs % 16 || L->ksc_cs % srow_g || L->vsc_cs % srow_g)
        return QSA_ERR_INVALID_ARG;
    if (L->kq_bs % 16 || L->vq_bs % 16 || L->ksc_bs % 16 || L->vsc_bs % 16)
        return QSA_ERR_INVALID_ARG;

    L->B = d->batch;
    L->T = d->T;
    L->Hq = d->Hq;
    L->Hkv = d->Hkv;
    L->D = d->D;
    L->P = d->P;
    L->cap = d->ids_cap;
    L->N = d->n_cells;
    L->scale = d->scale != 0.f ? d->scale : 1.f / sqrtf((float)d->D);
    L->q_f16 = d->q_dtype == QSA_F16;
    L->out_f16 = d->out_dtype == QSA_F16;
    L->algo = d->algo;
    L->gate = nullptr;
    return QSA_OK;
}

// Validates an index call's descriptor and pointers and fills `a` (all but
// the workspace).
int fill_index(const qsa_index_desc* desc, const void* q_idx, const void* K_idx, int32_t* ids,
               int32_t* n_sel, qsa::IndexLaunch* a)
{
    const int st = check_index(desc);
    if (st != QSA_OK)
        return st;
    if (!q_idx || !K_idx || !ids || !n_sel)
        return QSA_ERR_INVALID_ARG;
    if (!aligned(q_idx, 16) || !aligned(K_idx, 16) || !aligned(ids, 4) || !aligned(n_sel, 4))
        return QSA_ERR_INVALID_ARG;
    a->B = desc->batch;
    a->T = desc->T;
    a->N = desc->n_cells;
    a->DI = desc->d_idx;
    a->k = desc->k;
    a->pos0 = desc->pos0;
    a->dense_max = desc->dense_max;
    a->cap = desc->ids_cap;
    a->q_idx = q_idx;
    a->K_idx = K_idx;
    a->ids = ids;
    a->n_sel = n_sel;
    a->ws = nullptr;
    return QSA_OK;
}

// Validates an append call's descriptor and pointers and fills `a`.
int fill_append(const qsa_append_desc* d, const float* k_new, const float* v_new,
                const float* kidx_new, int8_t* Kq, void* Ksc, int8_t* Vq, void* Vsc, void* K_idx,
                qsa::AppendLaunch* a)
{
    if (!d)
        return QSA_ERR_INVALID_ARG;
    if (d->batch < 1 || d->T < 1 || d->n_cells < 1 || d->pos0 < 0 || d->Hkv < 1 ||
        d->D < 32 || d->D % 32 || d->reserved != 0)
        return QSA_ERR_INVALID_ARG;
    if ((long long)d->pos0 + d->T > d->n_cells)
        return QSA_ERR_INVALID_ARG;
    if (d->D > 1024)
        return QSA_ERR_UNSUPPORTED;
    if (kidx_new && (d->d_idx < 4 || d->d_idx % 4))
        return QSA_ERR_INVALID_ARG;
    if ((long long)d->batch * d->T * d->Hkv * (d->D / 32) > (1LL << 30))
        return QSA_ERR_UNSUPPORTED;
    if (!k_new || !v_new || !Kq || !Ksc || !Vq || !Vsc || (kidx_new && !K_idx))
        return QSA_ERR_INVALID_ARG;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || (kidx_new && !aligned(kidx_new, 16)) ||
        !aligned(Kq, 16) || !aligned(Vq, 16) || !aligned(Ksc, 2) || !aligned(Vsc, 2) ||
        (kidx_new && !aligned(K_idx, 8)))
        return QSA_ERR_INVALID_ARG;
    const long long row = (long long)d->Hkv * d->D;
    const long long srow = (long long)d->Hkv * (d->D / 32) * 2;
    a->kq_cs = d->kq_cell_stride ? d->kq_cell_stride : row;
    a->vq_cs = d->vq_cell_stride ? d->vq_cell_stride : row;
    a->ksc_cs = d->ksc_cell_stride ? d->ksc_cell_stride : srow;
    a->vsc_cs = d->vsc_cell_stride ? d->vsc_cell_stride : srow;
    a->kq_bs = d->kq_batch_stride ? d->kq_batch_stride : a->kq_cs * d->n_cells;
    a->vq_bs = d->vq_batch_stride ? d->vq_batch_stride : a->vq_cs * d->n_cells;
    a->ksc_bs = d->ksc_batch_stride ? d->ksc_batch_stride : a->ksc_cs * d->n_cells;
    a->vsc_bs = d->vsc_batch_stride ? d->vsc_batch_stride : a->vsc_cs * d->n_cells;
    if (a->kq_cs < 0 || a->vq_cs < 0 || a->ksc_cs < 0 || a->vsc_cs < 0 || a->kq_bs < 0 ||
        a->vq_bs < 0 || a->ksc_bs < 0 || a->vsc_bs < 0)
        return QSA_ERR_INVALID_ARG;
    if (a->kq_cs % 16 || a->vq_cs % 16 || a->kq_bs % 16 || a->vq_bs % 16 || a->ksc_cs % 2 ||
        a->vsc_cs % 2 || a->ksc_bs % 2 || a->vsc_bs % 2)
        return QSA_ERR_INVALID_ARG;
    a->B = d->batch;
    a->T = d->T;
    a->N = d->n_cells;
    a->pos0 = d->pos0;
    a->Hkv = d->Hkv;
    a->D = d->D;
    a->DI = d->d_idx;
    a->k_new = k_new;
    a->v_new = v_new;
    a->kidx_new = kidx_new;
    a->Kq = Kq;
    a->Ksc = (uint16_t*)Ksc;
    a->Vq = Vq;
    a->Vsc = (uint16_t*)Vsc;
    a->K_idx = (uint16_t*)K_idx;
    return QSA_OK;
}

size_t partial_rows(const qsa_attn_desc* d)
{
    return (size_t)d->batch * (size_t)d->T * (size_t)d->Hq * (size_t)d->P;
}

// The three descriptors of one step describe the same problems: equal T,
// batch and n_cells, the append's cells are the index tokens' positions,
// equal Hkv, D and ids_cap, equal d_idx when index keys are appended, and
// the same resolved cache strides.
bool same_step(const qsa_append_desc* pd, const qsa_index_desc* id, const qsa_attn_desc* ad,
               const qsa::AppendLaunch& ap, const qsa::AttnLaunch& at, bool with_kidx)
{
    if (pd->T != id->T || ad->T != id->T || pd->batch != id->batch || ad->batch != id->batch ||
        pd->n_cells != id->n_cells || ad->n_cells != id->n_cells || pd->pos0 != id->pos0 ||
        pd->Hkv != ad->Hkv || pd->D != ad->D || ad->ids_cap != id->ids_cap ||
        (with_kidx && pd->d_idx != id->d_idx))
        return false;
    return ap.kq_cs == at.kq_cs && ap.ksc_cs == at.ksc_cs && ap.vq_cs == at.vq_cs &&
           ap.vsc_cs == at.vsc_cs && ap.kq_bs == at.kq_bs && ap.ksc_bs == at.ksc_bs &&
           ap.vq_bs == at.vq_bs && ap.vsc_bs == at.vsc_bs;
}

// The attention and the merge run as one kernel (qsa_attend_merge).
bool merge_fuses(const qsa::AttnLaunch& at)
{
    return at.algo != QSA_ATTEND_VECTOR && (at.P == 1 || at.P == 2 || at.P == 4);
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace of qsa_step: the index workspace, then (when the merge is a
// separate kernel) the partials, 256-byte aligned.
size_t step_workspace_bytes(const qsa_index_desc* id, const qsa_attn_desc* ad,
                            const qsa::AttnLaunch& at)
{
    size_t n = round_up(qsa::index_workspace_bytes(id->batch, id->T, id->n_cells), 256);
    if (!merge_fuses(at)) {
        const size_t rows = partial_rows(ad);
        n += round_up((2 * rows + rows * (size_t)ad->D) * sizeof(float), 256);
    }
    return n;
}

}  // namespace

extern "C" {

const char* qsa_status_string(int status)
{
    switch (status) {
    case QSA_OK: return "ok";
    case QSA_ERR_INVALID_ARG: return "invalid argument";
    case QSA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case QSA_ERR_WORKSPACE: return "workspace missing or too small";
    case QSA_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
    }
}

int qsa_version(void) { return QSA_VERSION; }

size_t qsa_index_topk_workspace(const qsa_index_desc* desc)
{
    if (check_index(desc) != QSA_OK)
        return 0;
    return qsa::index_workspace_bytes(desc->batch, desc->T, desc->n_cells);
}

int qsa_index_topk(const qsa_index_desc* desc, const void* q_idx, const void* K_idx,
                   int32_t* ids, int32_t* n_sel, void* ws, size_t ws_bytes, void* stream)
{
    qsa::IndexLaunch a;
    const int st = fill_index(desc, q_idx, K_idx, ids, n_sel, &a);
    if (st != QSA_OK)
        return st;
    const size_t need = qsa::index_workspace_bytes(desc->batch, desc->T, desc->n_cells);
    if (!ws || ws_bytes < need || !aligned(ws, 16))
        return QSA_ERR_WORKSPACE;
    a.ws = ws;
    if (qsa::launch_index_topk(a, (hipStream_t)stream) != hipSuccess)
        return QSA_ERR_HIP;
    return QSA_OK;
}

int qsa_index_topk_noalloc(const qsa_index_desc* desc, const void* q_idx, const void* K_idx,
                           int32_t* ids, int32_t* n_sel, void* stream)
{
    const int st = check_index(desc);
    if (st != QSA_OK)
        return st;
    if (!q_idx || !K_idx || !ids || !n_sel)
        return QSA_ERR_INVALID_ARG;
    const size_t need = qsa::index_workspace_bytes(desc->batch, desc->T, desc->n_cells);
    if (need > (size_t)QSA_NOALLOC_WORKSPACE_BYTES)
        return QSA_ERR_WORKSPACE;
    int dev = -1;
    const hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return QSA_ERR_HIP;
    void* ws = nullptr;
    if (scratch_address(dev, &ws) != hipSuccess || !ws)
        return QSA_ERR_HIP;
    return qsa_index_topk(desc, q_idx, K_idx, ids, n_sel, ws, (size_t)QSA_NOALLOC_WORKSPACE_BYTES,
                          stream);
}

size_t qsa_partials_floats(const qsa_attn_desc* desc)
{
    qsa::AttnLaunch L;
    if (check_attn(desc, &L) != QSA_OK)
        return 0;
    const size_t rows = partial_rows(desc);
    return 2 * rows + rows * (size_t)desc->D;
}

int qsa_attend(const qsa_attn_desc* desc, const void* q, const int8_t* Kq, const void* Ksc,
               const int8_t* Vq, const void* Vsc, const int32_t* ids, const int32_t* n_sel,
               float* partials, void* stream)
{
    qsa::AttnLaunch a;
    const int st = check_attn(desc, &a);
    if (st != QSA_OK)
        return st;
    if (!q || !Kq || !Ksc || !Vq || !Vsc || !ids || !n_sel || !partials)
        return QSA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(Kq, 16) || !aligned(Ksc, 16) || !aligned(Vq, 16) ||
        !aligned(Vsc, 16) || !aligned(ids, 4) || !aligned(n_sel, 4) || !aligned(partials, 16))
        return QSA_ERR_INVALID_ARG;
    const size_t rows = partial_rows(desc);
    a.q = q;
    a.Kq = Kq;
    a.Ksc = Ksc;
    a.Vq = Vq;
    a.Vsc = Vsc;
    a.ids = ids;
    a.n_sel = n_sel;
    a.pm = partials;
    a.pl = partials + rows;
    a.po = partials + 2 * rows;
    a.out = nullptr;
    if (qsa::launch_attend(a, (hipStream_t)stream) != hipSuccess)
        return QSA_ERR_HIP;
    return QSA_OK;
}

int qsa_merge_gated(const qsa_attn_desc* desc, const float* partials, const void* gate,
                    void* out, void* stream)
{
    qsa::AttnLaunch a;
    const int st = check_attn(desc, &a);
    if (st != QSA_OK)
        return st;
    if (!partials || !out || !aligned(partials, 16) || !aligned(out, 16) ||
        (gate && !aligned(gate, 16)))
        return QSA_ERR_INVALID_ARG;
    const size_t rows = partial_rows(desc);
    a.pm = (float*)partials;
    a.pl = (float*)partials + rows;
    a.po = (float*)partials + 2 * rows;
    a.out = out;
    a.gate = gate;
    if (qsa::launch_merge(a, (hipStream_t)stream) != hipSuccess)
        return QSA_ERR_HIP;
    return QSA_OK;
}

int qsa_merge(const qsa_attn_desc* desc, const float* partials, void* out, void* stream)
{
    return qsa_merge_gated(desc, partials, nullptr, out, stream);
}

int qsa_attend_merge(const qsa_attn_desc* desc, const void* q, const int8_t* Kq, const void* Ksc,
                     const int8_t* Vq, const void* Vsc, const int32_t* ids, const int32_t* n_sel,
                     const void* gate, void* out, void* stream)
{
    qsa::AttnLaunch a;
    const int st = check_attn(desc, &a);
    if (st != QSA_OK)
        return st;
    if (!q || !Kq || !Ksc || !Vq || !Vsc || !ids || !n_sel || !out)
        return QSA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(Kq, 16) || !aligned(Ksc, 16) || !aligned(Vq, 16) ||
        !aligned(Vsc, 16) || !aligned(ids, 4) || !aligned(n_sel, 4) || !aligned(out, 16) ||
        (gate && !aligned(gate, 16)))
        return QSA_ERR_INVALID_ARG;
    // One workgroup holds four (token, chunk) items: the chunks of a token
    // must fit one workgroup.
    if (a.algo == QSA_ATTEND_VECTOR || (a.P != 1 && a.P != 2 && a.P != 4))
        return QSA_ERR_UNSUPPORTED;
    a.q = q;
    a.Kq = Kq;
    a.Ksc = Ksc;
    a.Vq = Vq;
    a.Vsc = Vsc;
    a.ids = ids;
    a.n_sel = n_sel;
    a.pm = a.pl = a.po = nullptr;
    a.out = out;
    a.gate = gate;
    if (qsa::launch_attend(a, (hipStream_t)stream) != hipSuccess)
        return QSA_ERR_HIP;
    return QSA_OK;
}

int qsa_kv_append(const qsa_append_desc* d, const float* k_new, const float* v_new,
                  const float* kidx_new, int8_t* Kq, void* Ksc, int8_t* Vq, void* Vsc,
                  void* K_idx, void* stream)
{
    qsa::AppendLaunch a;
    const int st = fill_append(d, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx, &a);
    if (st != QSA_OK)
        return st;
    if (qsa::launch_kv_append(a, (hipStream_t)stream) != hipSuccess)
        return QSA_ERR_HIP;
    return QSA_OK;
}

size_t qsa_decode_window_workspace(const qsa_index_desc* idesc, const qsa_attn_desc* adesc)
{
    qsa::AttnLaunch at;
    if (check_index(idesc) != QSA_OK || check_attn(adesc, &at) != QSA_OK)
        return 0;
    return qsa::window_workspace_bytes(idesc->batch, idesc->n_cells, adesc->Hq, adesc->P,
                                       adesc->D);
}

int qsa_decode_window(const qsa_append_desc* pdesc, const qsa_index_desc* idesc,
                      const qsa_attn_desc* adesc, const float* k_new, const float* v_new,
                      const float* kidx_new, int8_t* Kq, void* Ksc, int8_t* Vq, void* Vsc,
                      void* K_idx, const void* q_idx, const void* q, const void* gate,
                      int32_t* ids, int32_t* n_sel, void* out, void* ws, size_t ws_bytes,
                      void* stream)
{
    qsa::AppendLaunch ap;
    qsa::IndexLaunch ix;
    qsa::AttnLaunch at;
    int st = fill_append(pdesc, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx, &ap);
    if (st == QSA_OK)
        st = fill_index(idesc, q_idx, K_idx, ids, n_sel, &ix);
    if (st == QSA_OK)
        st = check_attn(adesc, &at);
    if (st != QSA_OK)
        return st;
    // One step of the same problems, read from the cache the append writes.
    if (pdesc->T != 1 || !same_step(pdesc, idesc, adesc, ap, at, kidx_new != nullptr))
        return QSA_ERR_INVALID_ARG;
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16) || (gate && !aligned(gate, 16)) ||
        !aligned(Ksc, 16) || !aligned(Vsc, 16))
        return QSA_ERR_INVALID_ARG;
    if (at.q_f16 || at.out_f16 || at.algo == QSA_ATTEND_VECTOR ||
        !qsa::window_supported(at.Hq / at.Hkv, at.D, ix.DI, at.P, ix.pos0 + 1))
        return QSA_ERR_UNSUPPORTED;
    const size_t need =
        qsa::window_workspace_bytes(idesc->batch, idesc->n_cells, adesc->Hq, adesc->P, adesc->D);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
        return QSA_ERR_WORKSPACE;
    at.q = q;
    at.Kq = Kq;
    at.Ksc = Ksc;
    at.Vq = Vq;
    at.Vsc = Vsc;
    at.ids = ids;
    at.n_sel = n_sel;
    at.out = out;
    at.gate = gate;
    if (qsa::launch_window(ap, ix, at, ws, (hipStream_t)stream) != hipSuccess)
        return QSA_ERR_HIP;
    return QSA_OK;
}

size_t qsa_step_workspace(const qsa_index_desc* idesc, const qsa_attn_desc* adesc)
{
    qsa::AttnLaunch at;
    if (check_index(idesc) != QSA_OK || check_attn(adesc, &at) != QSA_OK)
        return 0;
    return step_workspace_bytes(idesc, adesc, at);
}

int qsa_step(const qsa_append_desc* pdesc, const qsa_index_desc* idesc,
             const qsa_attn_desc* adesc, const float* k_new, const float* v_new,
             const float* kidx_new, int8_t* Kq, void* Ksc, int8_t* Vq, void* Vsc, void* K_idx,
             const void* q_idx, const void* q, const void* gate, int32_t* ids, int32_t* n_sel,
             void* out, void* ws, size_t ws_bytes, void* stream)
{
    qsa::AppendLaunch ap;
    qsa::IndexLaunch ix;
    qsa::AttnLaunch at;
    int st = fill_append(pdesc, k_new, v_new, kidx_new, Kq, Ksc, Vq, Vsc, K_idx, &ap);
    if (st == QSA_OK)
        st = fill_index(idesc, q_idx, K_idx, ids, n_sel, &ix);
    if (st == QSA_OK)
        st = check_attn(adesc, &at);
    if (st != QSA_OK)
        return st;
    if (!same_step(pdesc, idesc, adesc, ap, at, kidx_new != nullptr))
        return QSA_ERR_INVALID_ARG;
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16) || (gate && !aligned(gate, 16)) ||
        !aligned(Ksc, 16) || !aligned(Vsc, 16))
        return QSA_ERR_INVALID_ARG;
    const size_t need = step_workspace_bytes(idesc, adesc, at);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
        return QSA_ERR_WORKSPACE;
    ix.ws = ws;
    at.q = q;
    at.Kq = Kq;
    at.Ksc = Ksc;
    at.Vq = Vq;
    at.Vsc = Vsc;
    at.ids = ids;
    at.n_sel = n_sel;
    at.out = out;
    at.gate = gate;
    const hipStream_t s = (hipStream_t)stream;
    if (qsa::launch_index_topk(ix, s, &ap) != hipSuccess)
        return QSA_ERR_HIP;
    if (merge_fuses(at)) {
        at.pm = at.pl = at.po = nullptr;
        if (qsa::launch_attend(at, s) != hipSuccess)
            return QSA_ERR_HIP;
        return QSA_OK;
    }
    const size_t rows = partial_rows(adesc);
    float* part = (float*)((char*)ws + round_up(
        qsa::index_workspace_bytes(idesc->batch, idesc->T, idesc->n_cells), 256));
    at.pm = part;
    at.pl = part + rows;
    at.po = part + 2 * rows;
    if (qsa::attend_mch(at)) {
        // several chunks per wave: the kernel merges the partials it wrote
        if (qsa::launch_attend(at, s) != hipSuccess)
            return QSA_ERR_HIP;
        return QSA_OK;
    }
    void* out_keep = at.out;
    at.out = nullptr;  // qsa_attend writes the partials
    if (qsa::launch_attend(at, s) != hipSuccess)
        return QSA_ERR_HIP;
    at.out = out_keep;
    if (qsa::launch_merge(at, s) != hipSuccess)
        return QSA_ERR_HIP;
    return QSA_OK;
}

}  // extern "C"
