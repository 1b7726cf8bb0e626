/*
 * abi_driver.c -- a plain C caller of libqsa (include/qsa.h), with no
 * Python in between.
 *
 *   abi_driver host        validation and size queries only (no GPU): every
 *                          rejected call must return its documented status
 *                          and launch nothing.  Also built with
 *                          AddressSanitizer / UndefinedBehaviorSanitizer
 *                          against a host-sanitised build of the library.
 *   abi_driver run DIR     the whole path on the GPU: reads the inputs that
 *                          DIR/shape.txt describes (raw little-endian files
 *                          written by the test), copies them to device memory
 *                          it allocates itself, runs qsa_kv_append ->
 *                          qsa_index_topk -> qsa_attend -> qsa_merge_gated on
 *                          the default stream, and writes ids, n_sel, out and
 *                          the appended cache back to DIR.
 *
 * TEST INFRASTRUCTURE ONLY.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qsa.h"

static long long n_checks = 0;

#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        ++n_checks;                                                       \
        if (!(cond)) {                                                    \
            fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__);        \
            fprintf(stderr, __VA_ARGS__);                                 \
            fprintf(stderr, "\n");                                        \
            return 1;                                                     \
        }                                                                 \
    } while (0)

/* ------------------------------------------------------------ host mode --- */

static qsa_index_desc idesc(void)
{
    qsa_index_desc d = {1, 1, 8192, 128, 2048, 8191, 2051, 2051};
    return d;
}

static qsa_attn_desc adesc(void)
{
    qsa_attn_desc d;
    memset(&d, 0, sizeof d);
    d.batch = 1;
    d.T = 1;
    d.Hq = 24;
    d.Hkv = 2;
    d.D = 256;
    d.P = 4;
    d.ids_cap = 2051;
    d.n_cells = 8192;
    return d;
}

static int host_checks(void)
{
    void* const p16 = (void*)(uintptr_t)256; /* aligned, never dereferenced */
    void* const p8 = (void*)(uintptr_t)264;  /* 8-byte aligned only */
    CHECK(qsa_version() == QSA_VERSION, "version");
    CHECK(strcmp(qsa_status_string(QSA_OK), "ok") == 0, "status string of OK");
    for (int c = -4; c <= -1; ++c)
        CHECK(strcmp(qsa_status_string(c), "ok") && strcmp(qsa_status_string(c), "unknown status"),
              "status string of %d", c);
    CHECK(strcmp(qsa_status_string(7), "unknown status") == 0, "unknown status");

    /* index */
    qsa_index_desc d = idesc();
    const size_t need = qsa_index_topk_workspace(&d);
    CHECK(need >= (size_t)8192 * 4, "workspace size %zu", need);
    CHECK(qsa_index_topk(NULL, p16, p16, p16, p16, p16, need, NULL) == QSA_ERR_INVALID_ARG, "null desc");
    CHECK(qsa_index_topk(&d, NULL, p16, p16, p16, p16, need, NULL) == QSA_ERR_INVALID_ARG, "null q");
    CHECK(qsa_index_topk(&d, p8, p16, p16, p16, p16, need, NULL) == QSA_ERR_INVALID_ARG, "misaligned q");
    CHECK(qsa_index_topk(&d, p16, p16, p16, p16, NULL, need, NULL) == QSA_ERR_WORKSPACE, "null ws");
    CHECK(qsa_index_topk(&d, p16, p16, p16, p16, p16, need - 1, NULL) == QSA_ERR_WORKSPACE, "small ws");
    {
        struct { int field; int value; int code; } bad[] = {
            {0, 0, QSA_ERR_INVALID_ARG}, {1, 0, QSA_ERR_INVALID_ARG}, {4, 0, QSA_ERR_INVALID_ARG},
            {5, -1, QSA_ERR_INVALID_ARG}, {5, 8192, QSA_ERR_INVALID_ARG},
            {4, 3000, QSA_ERR_INVALID_ARG}, {6, 3000, QSA_ERR_INVALID_ARG},
            {3, 96, QSA_ERR_UNSUPPORTED}, {0, 70000, QSA_ERR_UNSUPPORTED},
        };
        for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
            qsa_index_desc e = idesc();
            ((int*)&e)[bad[i].field] = bad[i].value;
            CHECK(qsa_index_topk_workspace(&e) == 0, "workspace of bad index desc %zu", i);
            CHECK(qsa_index_topk(&e, p16, p16, p16, p16, p16, (size_t)1 << 40, NULL) == bad[i].code,
                  "bad index desc %zu", i);
        }
    }

    /* attend / merge */
    qsa_attn_desc a = adesc();
    const size_t rows = 24 * 4;
    CHECK(qsa_partials_floats(&a) == 2 * rows + rows * 256, "partials size");
    CHECK(qsa_attend(&a, NULL, p16, p16, p16, p16, p16, p16, p16, NULL) == QSA_ERR_INVALID_ARG, "null q");
    CHECK(qsa_attend(&a, p16, p16, p16, p16, p16, p16, p16, p8, NULL) == QSA_ERR_INVALID_ARG,
          "misaligned partials");
    CHECK(qsa_merge(&a, p16, NULL, NULL) == QSA_ERR_INVALID_ARG, "null out");
    CHECK(qsa_merge_gated(&a, p16, p8, p16, NULL) == QSA_ERR_INVALID_ARG, "misaligned gate");
    {
        qsa_attn_desc e = adesc();
        e.P = 65;
        CHECK(qsa_partials_floats(&e) == 0, "P=65 size");
        CHECK(qsa_attend(&e, p16, p16, p16, p16, p16, p16, p16, p16, NULL) == QSA_ERR_UNSUPPORTED, "P=65");
        e = adesc();
        e.D = 48;
        CHECK(qsa_merge(&e, p16, p16, NULL) == QSA_ERR_INVALID_ARG, "D=48");
        e = adesc();
        e.kq_cell_stride = 520;
        CHECK(qsa_attend(&e, p16, p16, p16, p16, p16, p16, p16, p16, NULL) == QSA_ERR_INVALID_ARG,
              "code stride not a multiple of 16");
        e = adesc();
        e.algo = 3;
        CHECK(qsa_attend(&e, p16, p16, p16, p16, p16, p16, p16, p16, NULL) == QSA_ERR_INVALID_ARG, "algo");
        e = adesc();
        e.scale = 1.0f / 0.0f;
        CHECK(qsa_attend(&e, p16, p16, p16, p16, p16, p16, p16, p16, NULL) == QSA_ERR_INVALID_ARG,
              "infinite scale");
    }

    /* append */
    {
        qsa_append_desc e;
        memset(&e, 0, sizeof e);
        e.batch = 2;
        e.T = 1;
        e.n_cells = 64;
        e.pos0 = 10;
        e.Hkv = 2;
        e.D = 256;
        e.d_idx = 128;
        CHECK(qsa_kv_append(&e, NULL, p16, p16, p16, p16, p16, p16, p16, NULL) == QSA_ERR_INVALID_ARG,
              "append null k");
        e.pos0 = 64;
        CHECK(qsa_kv_append(&e, p16, p16, p16, p16, p16, p16, p16, p16, NULL) == QSA_ERR_INVALID_ARG,
              "append past the cache");
        e.pos0 = 10;
        e.D = 2048;
        CHECK(qsa_kv_append(&e, p16, p16, p16, p16, p16, p16, p16, p16, NULL) == QSA_ERR_UNSUPPORTED,
              "append D=2048");
    }
    printf("host checks passed: %lld\n", n_checks);
    return 0;
}

/* ------------------------------------------------------------- GPU mode --- */

static void* read_file(const char* dir, const char* name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f)
        return NULL;
    void* p = malloc(bytes ? bytes : 1);
    const size_t got = p ? fread(p, 1, bytes, f) : 0;
    fclose(f);
    if (got != bytes) {
        free(p);
        return NULL;
    }
    return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f)
        return 1;
    const size_t put = fwrite(p, 1, bytes, f);
    fclose(f);
    return put != bytes;
}

static void* to_device(const void* host, size_t bytes)
{
    void* d = NULL;
    if (hipMalloc(&d, bytes ? bytes : 16) != hipSuccess)
        return NULL;
    if (host && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess)
        return NULL;
    return d;
}

static int gpu_run(const char* dir)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/shape.txt", dir);
    FILE* f = fopen(path, "r");
    CHECK(f != NULL, "no %s", path);
    int B, T, N, di, k, pos0, dense_max, cap, Hq, Hkv, D, P;
    const int n = fscanf(f, "%d %d %d %d %d %d %d %d %d %d %d %d", &B, &T, &N, &di, &k, &pos0,
                         &dense_max, &cap, &Hq, &Hkv, &D, &P);
    fclose(f);
    CHECK(n == 12, "shape.txt");
    const size_t nqi = (size_t)B * T * di * 2, nki = (size_t)B * N * di * 2;
    const size_t nq = (size_t)B * T * Hq * D * 4, nkv = (size_t)B * N * Hkv * D;
    const size_t nsc = nkv / 32 * 2, nnew = (size_t)B * T * Hkv * D * 4;
    const size_t nin = (size_t)B * T * di * 4, nids = (size_t)B * T * cap * 4;
    const char* names[] = {"q_idx", "K_idx", "q", "Kq", "Ksc", "Vq", "Vsc", "k_new", "v_new",
                           "kidx_new", "gate"};
    const size_t sizes[] = {nqi, nki, nq, nkv, nsc, nkv, nsc, nnew, nnew, nin, nq};
    void* host[11];
    void* dev[11];
    for (int i = 0; i < 11; ++i) {
        host[i] = read_file(dir, names[i], sizes[i]);
        CHECK(host[i] != NULL, "input %s", names[i]);
        dev[i] = to_device(host[i], sizes[i]);
        CHECK(dev[i] != NULL, "device copy of %s", names[i]);
    }
    qsa_append_desc ad;
    memset(&ad, 0, sizeof ad);
    ad.batch = B;
    ad.T = T;
    ad.n_cells = N;
    ad.pos0 = pos0;
    ad.Hkv = Hkv;
    ad.D = D;
    ad.d_idx = di;
    int st = qsa_kv_append(&ad, dev[7], dev[8], dev[9], dev[3], dev[4], dev[5], dev[6], dev[1],
                           NULL);
    CHECK(st == QSA_OK, "qsa_kv_append: %s", qsa_status_string(st));

    qsa_index_desc id = {B, T, N, di, k, pos0, dense_max, cap};
    const size_t ws_bytes = qsa_index_topk_workspace(&id);
    CHECK(ws_bytes > 0, "workspace size");
    void* ws = to_device(NULL, ws_bytes);
    void* ids = to_device(NULL, nids);
    void* n_sel = to_device(NULL, (size_t)B * T * 4);
    CHECK(ws && ids && n_sel, "device buffers");
    st = qsa_index_topk(&id, dev[0], dev[1], ids, n_sel, ws, ws_bytes, NULL);
    CHECK(st == QSA_OK, "qsa_index_topk: %s", qsa_status_string(st));

    qsa_attn_desc at;
    memset(&at, 0, sizeof at); /* scale 0: the library's default */
    at.batch = B;
    at.T = T;
    at.Hq = Hq;
    at.Hkv = Hkv;
    at.D = D;
    at.P = P;
    at.ids_cap = cap;
    at.n_cells = N;
    const size_t npart = qsa_partials_floats(&at);
    CHECK(npart > 0, "partials size");
    void* part = to_device(NULL, npart * 4);
    void* out = to_device(NULL, nq);
    CHECK(part && out, "device buffers");
    st = qsa_attend(&at, dev[2], dev[3], dev[4], dev[5], dev[6], ids, n_sel, part, NULL);
    CHECK(st == QSA_OK, "qsa_attend: %s", qsa_status_string(st));
    st = qsa_merge_gated(&at, part, dev[10], out, NULL);
    CHECK(st == QSA_OK, "qsa_merge_gated: %s", qsa_status_string(st));
    CHECK(hipDeviceSynchronize() == hipSuccess, "synchronise");

    void* h_ids = malloc(nids);
    void* h_ns = malloc((size_t)B * T * 4);
    void* h_out = malloc(nq);
    void* h_tmp = malloc(nq > nids ? nq : nids);
    CHECK(h_ids && h_ns && h_out && h_tmp, "host buffers");
    CHECK(hipMemcpy(h_ids, ids, nids, hipMemcpyDeviceToHost) == hipSuccess, "ids back");
    CHECK(hipMemcpy(h_ns, n_sel, (size_t)B * T * 4, hipMemcpyDeviceToHost) == hipSuccess, "n_sel");
    CHECK(hipMemcpy(h_out, out, nq, hipMemcpyDeviceToHost) == hipSuccess, "out back");

    /* qsa_attend_merge on the same ids: the output of the two calls, bit for
     * bit (when the split fits one workgroup). */
    if (P == 1 || P == 2 || P == 4) {
        void* out2 = to_device(NULL, nq);
        CHECK(out2 != NULL, "device buffer");
        st = qsa_attend_merge(&at, dev[2], dev[3], dev[4], dev[5], dev[6], ids, n_sel, dev[10],
                              out2, NULL);
        CHECK(st == QSA_OK, "qsa_attend_merge: %s", qsa_status_string(st));
        CHECK(hipMemcpy(h_tmp, out2, nq, hipMemcpyDeviceToHost) == hipSuccess, "out2 back");
        CHECK(memcmp(h_tmp, h_out, nq) == 0, "qsa_attend_merge differs from attend + merge");
        hipFree(out2);
        printf("attend_merge equal\n");
    }

    /* qsa_step from the original inputs: cache, ids, n_sel and output equal
     * to the four calls above, bit for bit. */
    {
        void* sdev[7];
        for (int i = 0; i < 7; ++i) {
            void* orig = read_file(dir, names[i], sizes[i]);
            CHECK(orig != NULL, "input %s", names[i]);
            sdev[i] = to_device(orig, sizes[i]);
            CHECK(sdev[i] != NULL, "device copy of %s", names[i]);
            free(orig);
        }
        const size_t sws_bytes = qsa_step_workspace(&id, &at);
        CHECK(sws_bytes > 0, "step workspace size");
        void* sws = to_device(NULL, sws_bytes);
        void* sids = to_device(NULL, nids);
        void* sns = to_device(NULL, (size_t)B * T * 4);
        void* sout = to_device(NULL, nq);
        CHECK(sws && sids && sns && sout, "device buffers");
        st = qsa_step(&ad, &id, &at, dev[7], dev[8], dev[9], sdev[3], sdev[4], sdev[5], sdev[6],
                      sdev[1], sdev[0], sdev[2], dev[10], sids, sns, sout, sws, sws_bytes, NULL);
        CHECK(st == QSA_OK, "qsa_step: %s", qsa_status_string(st));
        CHECK(hipMemcpy(h_tmp, sout, nq, hipMemcpyDeviceToHost) == hipSuccess, "step out");
        CHECK(memcmp(h_tmp, h_out, nq) == 0, "qsa_step output differs");
        CHECK(hipMemcpy(h_tmp, sids, nids, hipMemcpyDeviceToHost) == hipSuccess, "step ids");
        CHECK(memcmp(h_tmp, h_ids, nids) == 0, "qsa_step ids differ");
        CHECK(hipMemcpy(h_tmp, sns, (size_t)B * T * 4, hipMemcpyDeviceToHost) == hipSuccess,
              "step n_sel");
        CHECK(memcmp(h_tmp, h_ns, (size_t)B * T * 4) == 0, "qsa_step n_sel differs");
        for (int i = 1; i <= 6; ++i) {
            if (i == 2)
                continue;
            void* a = malloc(sizes[i]);
            void* b = malloc(sizes[i]);
            CHECK(a && b, "host buffers");
            CHECK(hipMemcpy(a, sdev[i], sizes[i], hipMemcpyDeviceToHost) == hipSuccess, "cache");
            CHECK(hipMemcpy(b, dev[i], sizes[i], hipMemcpyDeviceToHost) == hipSuccess, "cache");
            CHECK(memcmp(a, b, sizes[i]) == 0, "qsa_step cache %s differs", names[i]);
            free(a);
            free(b);
        }
        for (int i = 0; i < 7; ++i)
            hipFree(sdev[i]);
        hipFree(sws);
        hipFree(sids);
        hipFree(sns);
        hipFree(sout);
        printf("step equal\n");
    }
    CHECK(write_file(dir, "ids.out", h_ids, nids) == 0, "write ids");
    CHECK(write_file(dir, "n_sel.out", h_ns, (size_t)B * T * 4) == 0, "write n_sel");
    CHECK(write_file(dir, "out.out", h_out, nq) == 0, "write out");
    for (int i = 3; i <= 6; ++i) {
        char name[64];
        snprintf(name, sizeof name, "%s.out", names[i]);
        CHECK(hipMemcpy(host[i], dev[i], sizes[i], hipMemcpyDeviceToHost) == hipSuccess, "cache");
        CHECK(write_file(dir, name, host[i], sizes[i]) == 0, "write %s", name);
    }
    for (int i = 0; i < 11; ++i) {
        hipFree(dev[i]);
        free(host[i]);
    }
    hipFree(ws);
    hipFree(ids);
    hipFree(n_sel);
    hipFree(part);
    hipFree(out);
    free(h_ids);
    free(h_ns);
    free(h_out);
    free(h_tmp);
    printf("gpu run ok\n");
    return 0;
}

int main(int argc, char** argv)
{
    if (argc == 2 && strcmp(argv[1], "host") == 0)
        return host_checks();
    if (argc == 3 && strcmp(argv[1], "run") == 0)
        return gpu_run(argv[2]);
    fprintf(stderr, "usage: abi_driver host | abi_driver run DIR\n");
    return 2;
}
