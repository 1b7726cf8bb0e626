/*
 * oracle_patterns.c -- runs every entry point of the CPU oracle
 * (oracle/qsa_oracle.c) on five input patterns, built with AddressSanitizer
 * and UndefinedBehaviorSanitizer and without FMA contraction, following the
 * CPU-reference discipline of the "round 4 track b: mtp input and
 * hyper-connection fusion" page ("checks actually run", item 2: seeded
 * random, signed zeros, mixed powers of two, alternating signs and tiny
 * inputs; untouched padding and trailing guards checked bit for bit).
 *
 * TEST INFRASTRUCTURE ONLY (it links the oracle; nothing in the library
 * uses it).  Every output buffer is surrounded by guard words that must come
 * back untouched, and each result is checked against properties the method
 * fixes:
 *   - index: n_sel = visible cells when at most dense_max (or k) are
 *     visible, else k; kept ids ascending, visible, -1 after n_sel; every
 *     kept score >= every dropped one; equal scores at the threshold go to
 *     the lower index;
 *   - attention: the merge over P chunks equals the merge over one chunk
 *     (exact re-association, to 1e-12 relative); outputs finite; each
 *     output lies in the convex hull of the kept V rows (per element);
 *   - quantiser: codes in [-127, 127], scales non-negative, every element
 *     within half a scale step of its code (unless clamped), all-zero
 *     blocks give scale 0 and codes 0;
 *   - fp16: half -> double -> half returns every non-NaN pattern.
 * Prints "checks passed: N" and exits 0, or reports the first failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double qo_half_to_double(uint16_t h);
uint16_t qo_double_to_half(double x);
int qo_index_topk(int T, int N, int di, int k, int pos0, int dense_max, int cap,
                  const uint16_t* q_idx, const uint16_t* K_idx, int32_t* ids, int32_t* n_sel,
                  double* scores);
int qo_attend(int T, int Hq, int Hkv, int D, int P, int cap, double scale, int q_is_f16,
              const void* q, const int8_t* Kq, const uint16_t* Ksc, const int8_t* Vq,
              const uint16_t* Vsc, const int32_t* ids, const int32_t* n_sel, double* pm,
              double* pl, double* po);
int qo_merge(int T, int Hq, int P, int D, const double* pm, const double* pl, const double* po,
             double* out);
int qo_quant_row(int n, const float* x, int8_t* codes, uint16_t* scales);
int qo_kv_append(int T, int N, int Hkv, int D, int di, int pos0, const float* k_new,
                 const float* v_new, const float* kidx_new, int8_t* Kq, uint16_t* Ksc,
                 int8_t* Vq, uint16_t* Vsc, uint16_t* K_idx);

static long long n_checks = 0;

#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        ++n_checks;                                                       \
        if (!(cond)) {                                                    \
            fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__);        \
            fprintf(stderr, __VA_ARGS__);                                 \
            fprintf(stderr, "\n");                                        \
            exit(1);                                                      \
        }                                                                 \
    } while (0)

/* ------------------------------------------------------------- random --- */

static uint64_t rng_state;

static uint64_t rng_next(void) /* splitmix64 */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double rng_unit(void) { return (double)(rng_next() >> 11) * 0x1.0p-53; }

enum { PAT_RANDOM, PAT_SIGNED_ZEROS, PAT_POW2, PAT_ALT_SIGN, PAT_TINY, N_PAT };
static const char* pat_name[N_PAT] = {"seeded random", "signed zeros", "mixed powers of two",
                                      "alternating signs", "tiny"};

/* One value of pattern p at position i. */
static double pat_value(int p, size_t i)
{
    switch (p) {
    case PAT_RANDOM:
        return 4.0 * rng_unit() - 2.0;
    case PAT_SIGNED_ZEROS: {
        const uint64_t r = rng_next() % 8;
        return r < 3 ? 0.0 : r < 6 ? -0.0 : (r == 6 ? 1.0 : -0.5);
    }
    case PAT_POW2: {
        const int e = (int)(rng_next() % 24) - 12;
        return ldexp((rng_next() & 1) ? -1.0 : 1.0, e);
    }
    case PAT_ALT_SIGN:
        return ((i & 1) ? -1.0 : 1.0) * (0.25 + rng_unit());
    default: /* tiny: fp16 subnormals and the smallest normals */
        return ((rng_next() & 1) ? -1.0 : 1.0) * ldexp((double)(1 + rng_next() % 2047), -24);
    }
}

/* ------------------------------------------------------ guarded buffers --- */

#define GUARD_BYTES 64
#define GUARD_BYTE 0xA5

static void* galloc(size_t bytes)
{
    unsigned char* p = (unsigned char*)malloc(bytes + 2 * GUARD_BYTES);
    CHECK(p != NULL, "out of memory");
    memset(p, GUARD_BYTE, GUARD_BYTES);
    memset(p + GUARD_BYTES + bytes, GUARD_BYTE, GUARD_BYTES);
    memcpy(p, &bytes, sizeof bytes);
    return p + GUARD_BYTES;
}

static void gfree_checked(void* q, const char* what)
{
    unsigned char* p = (unsigned char*)q - GUARD_BYTES;
    size_t bytes;
    memcpy(&bytes, p, sizeof bytes);
    for (size_t i = sizeof bytes; i < GUARD_BYTES; ++i)
        CHECK(p[i] == GUARD_BYTE, "%s: leading guard byte %zu changed", what, i);
    for (size_t i = 0; i < GUARD_BYTES; ++i)
        CHECK(p[GUARD_BYTES + bytes + i] == GUARD_BYTE, "%s: trailing guard byte %zu changed",
              what, i);
    free(p);
}

/* ------------------------------------------------------------- checks --- */

static void check_fp16_roundtrip(void)
{
    for (uint32_t h = 0; h < 65536; ++h) {
        const double v = qo_half_to_double((uint16_t)h);
        if (isnan(v))
            continue;
        CHECK(qo_double_to_half(v) == h, "fp16 pattern %04x does not round-trip", h);
    }
}

static void check_index(int p, int T, int N, int di, int k, int pos0, int dense_max)
{
    const int cap = (k > dense_max ? k : dense_max);
    uint16_t* q = (uint16_t*)galloc(sizeof(uint16_t) * (size_t)T * di);
    uint16_t* K = (uint16_t*)galloc(sizeof(uint16_t) * (size_t)N * di);
    int32_t* ids = (int32_t*)galloc(sizeof(int32_t) * (size_t)T * cap);
    int32_t* ns = (int32_t*)galloc(sizeof(int32_t) * (size_t)T);
    double* sc = (double*)galloc(sizeof(double) * (size_t)T * N);
    for (size_t i = 0; i < (size_t)T * di; ++i)
        q[i] = qo_double_to_half(pat_value(p, i));
    for (size_t i = 0; i < (size_t)N * di; ++i)
        K[i] = qo_double_to_half(pat_value(p, i));
    CHECK(qo_index_topk(T, N, di, k, pos0, dense_max, cap, q, K, ids, ns, sc) == 0,
          "index rejected valid arguments");
    for (int t = 0; t < T; ++t) {
        const int nvis = pos0 + t + 1;
        const int want = (nvis <= dense_max || nvis <= k) ? nvis : k;
        const int32_t* row = ids + (size_t)t * cap;
        const double* s = sc + (size_t)t * N;
        CHECK(ns[t] == want, "[%s] n_sel %d, want %d", pat_name[p], ns[t], want);
        char* kept = (char*)calloc((size_t)nvis, 1);
        CHECK(kept != NULL, "out of memory");
        for (int r = 0; r < cap; ++r) {
            if (r >= ns[t]) {
                CHECK(row[r] == -1, "[%s] padding %d = %d", pat_name[p], r, row[r]);
                continue;
            }
            CHECK(row[r] >= 0 && row[r] < nvis, "[%s] id %d not visible", pat_name[p], row[r]);
            if (r)
                CHECK(row[r] > row[r - 1], "[%s] ids not ascending", pat_name[p]);
            kept[row[r]] = 1;
        }
        double lo = INFINITY;
        for (int j = 0; j < nvis; ++j)
            if (kept[j] && s[j] < lo)
                lo = s[j];
        for (int j = 0; j < nvis; ++j) {
            if (kept[j])
                continue;
            CHECK(s[j] <= lo, "[%s] dropped cell %d scores above a kept one", pat_name[p], j);
            if (s[j] == lo)
                for (int i = j + 1; i < nvis; ++i)
                    CHECK(!(kept[i] && s[i] == lo), "[%s] tie at %d kept a higher index",
                          pat_name[p], j);
        }
        for (int j = nvis; j < N; ++j)
            CHECK(isnan(s[j]), "[%s] invisible cell has a score", pat_name[p]);
        free(kept);
    }
    gfree_checked(q, "q_idx");
    gfree_checked(K, "K_idx");
    gfree_checked(ids, "ids");
    gfree_checked(ns, "n_sel");
    gfree_checked(sc, "scores");
}

static void check_attention(int p, int T, int Hq, int Hkv, int D, int P, int N, int q_f16)
{
    const int cap = N;
    const size_t nq = (size_t)T * Hq * D, nkv = (size_t)N * Hkv * D, nsc = nkv / 32;
    void* q = galloc(q_f16 ? 2 * nq : 4 * nq);
    int8_t* Kq = (int8_t*)galloc(nkv);
    int8_t* Vq = (int8_t*)galloc(nkv);
    uint16_t* Ks = (uint16_t*)galloc(2 * nsc);
    uint16_t* Vs = (uint16_t*)galloc(2 * nsc);
    int32_t* ids = (int32_t*)galloc(sizeof(int32_t) * (size_t)T * cap);
    int32_t* ns = (int32_t*)galloc(sizeof(int32_t) * (size_t)T);
    for (size_t i = 0; i < nq; ++i) {
        const double v = pat_value(p, i);
        if (q_f16)
            ((uint16_t*)q)[i] = qo_double_to_half(v);
        else
            ((float*)q)[i] = (float)v;
    }
    for (size_t i = 0; i < nkv; ++i) {
        Kq[i] = (int8_t)((int)(rng_next() % 255) - 127);
        Vq[i] = (int8_t)((int)(rng_next() % 255) - 127);
    }
    for (size_t i = 0; i < nsc; ++i) {
        Ks[i] = qo_double_to_half(fabs(pat_value(p, i)) * 0.05);
        Vs[i] = qo_double_to_half(fabs(pat_value(p, i + 1)));
    }
    /* token t keeps a random ascending subset of cells 0..N-1 (at least one) */
    for (int t = 0; t < T; ++t) {
        int n = 0;
        for (int j = 0; j < N; ++j)
            if (j == t % N || rng_unit() < 0.4)
                ids[(size_t)t * cap + n++] = j;
        for (int r = n; r < cap; ++r)
            ids[(size_t)t * cap + r] = -1;
        ns[t] = n;
    }
    const size_t rows = (size_t)T * Hq;
    double* pm = (double*)galloc(sizeof(double) * rows * P);
    double* pl = (double*)galloc(sizeof(double) * rows * P);
    double* po = (double*)galloc(sizeof(double) * rows * P * D);
    double* out = (double*)galloc(sizeof(double) * rows * D);
    double* pm1 = (double*)galloc(sizeof(double) * rows);
    double* pl1 = (double*)galloc(sizeof(double) * rows);
    double* po1 = (double*)galloc(sizeof(double) * rows * D);
    double* out1 = (double*)galloc(sizeof(double) * rows * D);
    const double scale = 1.0 / sqrt((double)D);
    CHECK(qo_attend(T, Hq, Hkv, D, P, cap, scale, q_f16, q, Kq, Ks, Vq, Vs, ids, ns, pm, pl, po)
              == 0, "attend rejected valid arguments");
    CHECK(qo_merge(T, Hq, P, D, pm, pl, po, out) == 0, "merge rejected valid arguments");
    CHECK(qo_attend(T, Hq, Hkv, D, 1, cap, scale, q_f16, q, Kq, Ks, Vq, Vs, ids, ns, pm1, pl1,
                    po1) == 0, "attend rejected valid arguments");
    CHECK(qo_merge(T, Hq, 1, D, pm1, pl1, po1, out1) == 0, "merge rejected valid arguments");
    const int G = Hq / Hkv;
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < Hq; ++h)
            for (int d = 0; d < D; ++d) {
                const size_t o = ((size_t)t * Hq + h) * D + d;
                CHECK(isfinite(out[o]), "[%s] non-finite output", pat_name[p]);
                CHECK(fabs(out[o] - out1[o]) <= 1e-12 * (1.0 + fabs(out1[o])),
                      "[%s] P=%d differs from P=1: %.17g vs %.17g", pat_name[p], P, out[o],
                      out1[o]);
                double lo = INFINITY, hi = -INFINITY;
                for (int r = 0; r < ns[t]; ++r) {
                    const size_t row = (size_t)ids[(size_t)t * cap + r] * Hkv + h / G;
                    const double v = Vq[row * D + d] * qo_half_to_double(Vs[row * (D / 32) + d / 32]);
                    lo = v < lo ? v : lo;
                    hi = v > hi ? v : hi;
                }
                const double tol = 1e-12 * (fabs(lo) + fabs(hi));
                CHECK(out[o] >= lo - tol && out[o] <= hi + tol,
                      "[%s] output outside the kept V rows' range", pat_name[p]);
            }
    gfree_checked(q, "q");
    gfree_checked(Kq, "Kq");
    gfree_checked(Vq, "Vq");
    gfree_checked(Ks, "Ksc");
    gfree_checked(Vs, "Vsc");
    gfree_checked(ids, "ids");
    gfree_checked(ns, "n_sel");
    gfree_checked(pm, "pm");
    gfree_checked(pl, "pl");
    gfree_checked(po, "po");
    gfree_checked(out, "out");
    gfree_checked(pm1, "pm1");
    gfree_checked(pl1, "pl1");
    gfree_checked(po1, "po1");
    gfree_checked(out1, "out1");
}

static void check_quantiser(int p, int T, int N, int Hkv, int D, int di)
{
    const int pos0 = N - T;
    const size_t nrow = (size_t)T * Hkv * D, nkv = (size_t)N * Hkv * D;
    float* kn = (float*)galloc(4 * nrow);
    float* vn = (float*)galloc(4 * nrow);
    float* in = (float*)galloc(4 * (size_t)T * di);
    int8_t* Kq = (int8_t*)galloc(nkv);
    int8_t* Vq = (int8_t*)galloc(nkv);
    uint16_t* Ks = (uint16_t*)galloc(2 * (nkv / 32));
    uint16_t* Vs = (uint16_t*)galloc(2 * (nkv / 32));
    uint16_t* Ki = (uint16_t*)galloc(2 * (size_t)N * di);
    for (size_t i = 0; i < nrow; ++i) {
        kn[i] = (float)(pat_value(p, i) * 3.0);
        vn[i] = (float)pat_value(p, i + 7);
    }
    for (int e = 0; e < 32 && e < (int)nrow; ++e)
        kn[e] = (e & 1) ? -0.0f : 0.0f; /* one all-zero block */
    for (size_t i = 0; i < (size_t)T * di; ++i)
        in[i] = (float)pat_value(p, i);
    memset(Kq, 0x11, nkv);
    memset(Vq, 0x11, nkv);
    memset(Ks, 0x22, 2 * (nkv / 32));
    memset(Vs, 0x22, 2 * (nkv / 32));
    memset(Ki, 0x33, 2 * (size_t)N * di);
    CHECK(qo_kv_append(T, N, Hkv, D, di, pos0, kn, vn, in, Kq, Ks, Vq, Vs, Ki) == 0,
          "append rejected valid arguments");
    for (int j = 0; j < N; ++j) {
        const int fresh = j >= pos0;
        for (int g = 0; g < Hkv; ++g)
            for (int half = 0; half < 2; ++half) {
                const int8_t* codes = (half ? Vq : Kq) + ((size_t)j * Hkv + g) * D;
                const uint16_t* sc = (half ? Vs : Ks) + ((size_t)j * Hkv + g) * (D / 32);
                if (!fresh) {
                    for (int d = 0; d < D; ++d)
                        CHECK(codes[d] == 0x11, "[%s] untouched cell %d changed", pat_name[p], j);
                    continue;
                }
                const float* x = (half ? vn : kn) + ((size_t)(j - pos0) * Hkv + g) * D;
                for (int b = 0; b < D / 32; ++b) {
                    const double s = qo_half_to_double(sc[b]);
                    CHECK(s >= 0.0 && isfinite(s), "[%s] bad scale", pat_name[p]);
                    for (int e = 0; e < 32; ++e) {
                        const int c = codes[32 * b + e];
                        CHECK(c >= -127 && c <= 127, "[%s] code out of range", pat_name[p]);
                        if (s == 0.0) {
                            CHECK(c == 0, "[%s] zero scale with a nonzero code", pat_name[p]);
                            continue;
                        }
                        const double err = fabs((double)x[32 * b + e] - c * s);
                        CHECK(err <= 0.5 * s * (1 + 1e-12) || abs(c) == 127,
                              "[%s] element off its code by %.3g scale steps", pat_name[p],
                              err / s);
                    }
                }
            }
        for (int i = 0; i < di; ++i) {
            const uint16_t h = Ki[(size_t)j * di + i];
            if (!fresh)
                CHECK(h == 0x3333, "[%s] untouched index key changed", pat_name[p]);
            else
                CHECK(h == qo_double_to_half((double)in[(size_t)(j - pos0) * di + i]),
                      "[%s] index key not rounded to nearest", pat_name[p]);
        }
    }
    if (pos0 + 0 < N) /* the all-zero block */
        CHECK(Ks[(size_t)pos0 * Hkv * (D / 32)] == 0, "[%s] all-zero block has a scale",
              pat_name[p]);
    gfree_checked(kn, "k_new");
    gfree_checked(vn, "v_new");
    gfree_checked(in, "kidx_new");
    gfree_checked(Kq, "Kq");
    gfree_checked(Vq, "Vq");
    gfree_checked(Ks, "Ksc");
    gfree_checked(Vs, "Vsc");
    gfree_checked(Ki, "K_idx");
}

int main(void)
{
    check_fp16_roundtrip();
    for (int p = 0; p < N_PAT; ++p) {
        rng_state = 1000u + (uint64_t)p;
        /* index: dense bound, k above and below the visible count, ties */
        check_index(p, 1, 1, 4, 1, 0, 0);
        check_index(p, 3, 40, 64, 5, 20, 8);
        check_index(p, 2, 200, 64, 64, 150, 67);
        check_index(p, 4, 300, 128, 128, 290, 131);
        check_index(p, 2, 70, 4, 80, 60, 83);
        /* attention + merge: GQA 4:1 and 3:1, fp32 and fp16 queries */
        check_attention(p, 2, 4, 1, 64, 3, 50, 0);
        check_attention(p, 3, 6, 2, 32, 8, 37, 1);
        check_attention(p, 1, 12, 1, 256, 4, 70, 0);
        /* quantiser */
        check_quantiser(p, 3, 9, 2, 64, 16);
        check_quantiser(p, 1, 2, 1, 256, 128);
        printf("pattern %-20s ok\n", pat_name[p]);
    }
    printf("checks passed: %lld\n", n_checks);
    return 0;
}
