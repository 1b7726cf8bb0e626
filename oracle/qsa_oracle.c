/*
 * qsa_oracle.c -- plain, slow, double-precision CPU oracle for the QSA
 * top-k sparse attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the benchmark's CPU-baseline leg do.  It shares no code, header,
 * table or helper with the HIP library: fp16 decoding/encoding, score keys,
 * selection and attention are all written out here again from their
 * definitions.
 *
 * Sources (the audit pages this method is described in):
 *   [r20]  "opus r20 track A: MTP map mlock + qsa_attn / qsa_merge decode
 *          tweaks" -- section 2 "qsa.metal" (the attention cell split, the
 *          exact max of per-lane maxima, zero padding, the merge formula) and
 *          section 3 "verification" (random int8 KV with fp16 scales,
 *          top-k-shaped ids, the pos0 sweep).
 *   [r15]  "opus r15 track A: prompt_chunk wave zipping, fused alpha|beta
 *          GEMM, QSA PSO pre-warm, 24 GB chunk 2048" -- "what changed",
 *          item 1 (qsa_score_mm / qsa_topk run only for prompts longer than
 *          2051 tokens).
 *   [r5c]  "Round 5 Track C Report: Direct FP16 qcurh in qsa_prep +
 *          PromptGemm Dead Buffer Removal & Layer-Local Aliasing" -- section 1,
 *          Target 2 (the selected-id list is 2051 words per token; q is
 *          24 heads x 256; K and V are 512 floats per token), Target 1 (fp16
 *          q on the prompt-chunk path).
 *
 * Where the pages are silent the plain reading is used (each one is named
 * at the point of use):
 *   - the index score of cell j for token t is the plain dot product of the
 *     token's index query with the cell's index key (no scale, no
 *     activation);
 *   - token t sits at position pos0+t and sees cells 0..pos0+t inclusive;
 *   - when a token sees at most dense_max cells every visible cell is kept,
 *     otherwise the min(k, visible) highest-scoring visible cells are kept,
 *     equal scores going to the lower cell index; the kept ids are listed in ascending
 *     cell order and the row is padded with -1;
 *   - query head h reads KV head h / (Hq / Hkv);
 *   - the kept ids of a token are cut into P contiguous chunks of
 *     ceil(n_sel / P) ids (the last ones may be short or empty);
 *   - each chunk yields (max logit, sum of exp, unnormalised output), and the
 *     merge rescales every chunk by exp(m_c - M).
 *
 * Everything is computed in double from the stored bytes: int8 codes times
 * their fp16 scale (one scale per 32 consecutive elements of a head row) is
 * exact in double, as is every fp16 x fp16 product.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- fp16 --- */

/* IEEE 754 binary16 bit pattern -> double (exact). */
double qo_half_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 31;
    const int frac = h & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                 /* zero or subnormal */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);  /* (1 + f/1024) 2^(e-15) */
    return sign ? -v : v;
}

/* double -> binary16, round to nearest, ties to even. */
uint16_t qo_double_to_half(double x)
{
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return 0x7e00u;
    if (isinf(x))
        return (uint16_t)(sign | 0x7c00u);            /* infinity stays infinity */
    const double a = fabs(x);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: the quantum is 2^-24 */
        const double r = nearbyint(ldexp(a, 24));     /* ties to even */
        return (uint16_t)(sign | (uint16_t)r);        /* r == 1024 is the
                                                          smallest normal */
    }
    int e2;
    frexp(a, &e2);                  /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;                 /* unbiased binary16 exponent */
    double r = nearbyint(ldexp(a, 10 - E));          /* in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        E += 1;
    }
    if (E > 15)
        return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(r - 1024.0));
}

/* ------------------------------------------------------ index + top-k --- */

typedef struct {
    double s;
    int j;
} qo_scored;

/* Order for the kept set: higher score first; equal scores -> lower index
   first (the tie rule named for the selected-id list). */
static int qo_cmp_rank(const void* pa, const void* pb)
{
    const qo_scored* a = (const qo_scored*)pa;
    const qo_scored* b = (const qo_scored*)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j < b->j) ? -1 : (a->j > b->j);
}

static int qo_cmp_int(const void* pa, const void* pb)
{
    const int a = *(const int*)pa, b = *(const int*)pb;
    return (a > b) - (a < b);
}

/*
 * Index score + top-k for one problem ([r15] item 1; [r5c] Target 2).
 *   q_idx  [T][di]  fp16 bits     K_idx [N][di] fp16 bits
 *   ids    [T][cap] out: kept cell ids ascending, then -1
 *   n_sel  [T]      out: number of kept cells
 *   scores [T][N]   optional out (NULL to skip): score of every visible
 *                   cell, NAN for cells the token cannot see.
 * Returns 0, or -1 on invalid arguments.
 */
int qo_index_topk(int T, int N, int di, int k, int pos0, int dense_max, int cap,
                  const uint16_t* q_idx, const uint16_t* K_idx,
                  int32_t* ids, int32_t* n_sel, double* scores)
{
    if (T < 1 || N < 1 || di < 1 || k < 1 || pos0 < 0 || dense_max < 0 ||
        cap < 1 || pos0 + T > N || k > cap || dense_max > cap)
        return -1;
    qo_scored* all = (qo_scored*)malloc(sizeof(qo_scored) * (size_t)N);
    int* kept = (int*)malloc(sizeof(int) * (size_t)cap);
    if (!all || !kept) {
        free(all);
        free(kept);
        return -1;
    }
    for (int t = 0; t < T; ++t) {
        const int pos = pos0 + t;
        const int nvis = pos + 1;            /* cells 0..pos inclusive */
        const uint16_t* qt = q_idx + (size_t)t * di;
        for (int j = 0; j < nvis; ++j) {
            const uint16_t* kj = K_idx + (size_t)j * di;
            double s = 0.0;
            for (int i = 0; i < di; ++i)
                s += qo_half_to_double(qt[i]) * qo_half_to_double(kj[i]);
            all[j].s = s;
            all[j].j = j;
        }
        if (scores) {
            for (int j = 0; j < N; ++j)
                scores[(size_t)t * N + j] = (j < nvis) ? all[j].s : NAN;
        }
        int n;
        if (nvis <= dense_max) {
            n = nvis;                        /* dense fallback: keep all */
            for (int j = 0; j < n; ++j)
                kept[j] = j;
        } else {
            qsort(all, (size_t)nvis, sizeof(qo_scored), qo_cmp_rank);
            n = (k < nvis) ? k : nvis;       /* fewer than k visible: all */
            for (int r = 0; r < n; ++r)
                kept[r] = all[r].j;
            qsort(kept, (size_t)n, sizeof(int), qo_cmp_int);
        }
        int32_t* row = ids + (size_t)t * cap;
        for (int r = 0; r < cap; ++r)
            row[r] = (r < n) ? kept[r] : -1;
        n_sel[t] = n;
    }
    free(all);
    free(kept);
    return 0;
}

/* ---------------------------------------------------- attend + merge --- */

/* Dequantised element: int8 code times the fp16 scale of its 32-element
   block within the (cell, KV head) row ([r20] section 3: int8 KV, fp16
   scales). */
static double qo_deq(const int8_t* codes, const uint16_t* scales, int Hkv, int D,
                     int cell, int g, int d)
{
    const size_t row = ((size_t)cell * Hkv + g);
    const double code = (double)codes[row * D + d];
    const double sc = qo_half_to_double(scales[row * (D / 32) + d / 32]);
    return code * sc;
}

/*
 * Split-KV attention partials for one problem ([r20] section 2, qsa_attn).
 *   q     [T][Hq][D]  float (q_is_f16 == 0) or fp16 bits (q_is_f16 == 1)
 *   Kq,Vq [N][Hkv][D] int8;  Ksc,Vsc [N][Hkv][D/32] fp16 bits
 *   ids   [T][cap], n_sel [T]
 *   pm, pl [T][Hq][P]; po [T][Hq][P][D]   (outputs, double)
 * For chunk c of token t: x_j = scale * <q_h, K^_j>, m = max x_j,
 * l = sum exp(x_j - m), o = sum exp(x_j - m) V^_j.  An empty chunk gives
 * m = -inf, l = 0, o = 0.
 */
int qo_attend(int T, int Hq, int Hkv, int D, int P, int cap, double scale,
              int q_is_f16, const void* q,
              const int8_t* Kq, const uint16_t* Ksc,
              const int8_t* Vq, const uint16_t* Vsc,
              const int32_t* ids, const int32_t* n_sel,
              double* pm, double* pl, double* po)
{
    if (T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 32 || D % 32 != 0 ||
        P < 1 || cap < 1)
        return -1;
    const int G = Hq / Hkv;
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    double* x = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    if (!qd || !x) {
        free(qd);
        free(x);
        return -1;
    }
    for (int t = 0; t < T; ++t) {
        const int ns = n_sel[t];
        if (ns < 0 || ns > cap) {
            free(qd);
            free(x);
            return -1;
        }
        const int S = (ns + P - 1) / P;      /* chunk length, ceil */
        const int32_t* row = ids + (size_t)t * cap;
        for (int h = 0; h < Hq; ++h) {
            const int g = h / G;             /* GQA: contiguous head groups */
            for (int d = 0; d < D; ++d) {
                const size_t qi = ((size_t)t * Hq + h) * D + d;
                qd[d] = q_is_f16 ? qo_half_to_double(((const uint16_t*)q)[qi])
                                 : (double)((const float*)q)[qi];
            }
            for (int c = 0; c < P; ++c) {
                const size_t pi = ((size_t)t * Hq + h) * P + c;
                double* oc = po + pi * D;
                const int beg = c * S;
                const int end = (beg + S < ns) ? beg + S : ns;
                if (beg >= end) {
                    pm[pi] = -INFINITY;
                    pl[pi] = 0.0;
                    for (int d = 0; d < D; ++d)
                        oc[d] = 0.0;
                    continue;
                }
                double m = -INFINITY;
                for (int i = beg; i < end; ++i) {
                    const int j = row[i];
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += qd[d] * qo_deq(Kq, Ksc, Hkv, D, j, g, d);
                    x[i] = scale * dot;
                    if (x[i] > m)
                        m = x[i];
                }
                double l = 0.0;
                for (int d = 0; d < D; ++d)
                    oc[d] = 0.0;
                for (int i = beg; i < end; ++i) {
                    const int j = row[i];
                    const double p = exp(x[i] - m);
                    l += p;
                    for (int d = 0; d < D; ++d)
                        oc[d] += p * qo_deq(Vq, Vsc, Hkv, D, j, g, d);
                }
                pm[pi] = m;
                pl[pi] = l;
            }
        }
    }
    free(qd);
    free(x);
    return 0;
}

/*
 * Merge of the P chunk partials ([r20] section 2, qsa_merge):
 *   M = max_c m_c;  e_c = exp(m_c - M);  L = sum_c l_c e_c;
 *   out[d] = (sum_c o_c[d] e_c) / L.
 * A row whose chunks are all empty (L == 0) gives 0.
 *   pm, pl [T][Hq][P]; po [T][Hq][P][D]; out [T][Hq][D]
 */
int qo_merge(int T, int Hq, int P, int D, const double* pm, const double* pl,
             const double* po, double* out)
{
    if (T < 1 || Hq < 1 || P < 1 || D < 1)
        return -1;
    for (int th = 0; th < T * Hq; ++th) {
        const double* m = pm + (size_t)th * P;
        const double* l = pl + (size_t)th * P;
        const double* o = po + (size_t)th * P * D;
        double* y = out + (size_t)th * D;
        double M = -INFINITY;
        for (int c = 0; c < P; ++c)
            if (m[c] > M)
                M = m[c];
        double L = 0.0;
        for (int d = 0; d < D; ++d)
            y[d] = 0.0;
        if (M == -INFINITY)
            continue;
        for (int c = 0; c < P; ++c) {
            if (m[c] == -INFINITY)
                continue;                    /* empty chunk: weight 0 */
            const double e = exp(m[c] - M);
            L += l[c] * e;
            for (int d = 0; d < D; ++d)
                y[d] += o[(size_t)c * D + d] * e;
        }
        for (int d = 0; d < D; ++d)
            y[d] = (L > 0.0) ? y[d] / L : 0.0;
    }
    return 0;
}

/* ------------------------------------------------- KV append (quantise) --- */

/*
 * Quantisation of a new token's K or V row into the cache format: int8
 * codes with one fp16 scale per 32 consecutive elements ([r20] section 3:
 * int8 KV with fp16 scales; the block of 32 is the one the attention reads).
 * The pages do not spell out the quantiser; the plain absmax reading is
 * used, with every rounding to nearest, ties to even, on the exact values:
 *   a = max |x| over the block,  s = fp16(a / 127),
 *   c = clamp(round(x / s), -127, 127)   (c = 0 when s = 0).
 * Both roundings are checked against their neighbours with exact products
 * (an fp16 value times 127, or a code times an fp16 scale, is exact in
 * double, and so is its difference with a float input), so the result does
 * not depend on how double division rounds.
 */

/* Value of the binary16 pattern next to h in the direction of growing
   magnitude (dir = +1) or shrinking magnitude (dir = -1), for h >= 0. */
static uint16_t qo_half_step(uint16_t h, int dir)
{
    if (dir > 0)
        return (uint16_t)(h < 0x7c00u ? h + 1 : h);
    return (uint16_t)(h > 0 ? h - 1 : 0);
}

/* fp16 nearest to a / 127 for a >= 0 (ties to the even pattern). */
static uint16_t qo_scale_of(double a)
{
    uint16_t h = qo_double_to_half(a / 127.0);
    uint16_t best = h;
    double best_err = fabs(a - 127.0 * qo_half_to_double(h));
    for (int dir = -1; dir <= 1; dir += 2) {
        const uint16_t g = qo_half_step(h, dir);
        const double err = fabs(a - 127.0 * qo_half_to_double(g));
        if (err < best_err || (err == best_err && (g & 1u) == 0 && (best & 1u) == 1)) {
            best = g;
            best_err = err;
        }
    }
    return best;
}

/* Integer nearest to x / s for s > 0 (ties to even), clamped to +-127. */
static int qo_code_of(double x, double s)
{
    const double c0 = nearbyint(x / s);
    double best = c0, best_err = fabs(x - c0 * s);
    for (int d = -1; d <= 1; d += 2) {
        const double c = c0 + d;
        const double err = fabs(x - c * s);
        if (err < best_err || (err == best_err && fmod(fabs(c), 2.0) == 0.0)) {
            best = c;
            best_err = err;
        }
    }
    if (best > 127.0)
        best = 127.0;
    if (best < -127.0)
        best = -127.0;
    return (int)best;
}

/* One row of n (a multiple of 32) floats -> n codes and n/32 scales. */
int qo_quant_row(int n, const float* x, int8_t* codes, uint16_t* scales)
{
    if (n < 32 || n % 32)
        return -1;
    for (int blk = 0; blk < n / 32; ++blk) {
        const float* xb = x + 32 * blk;
        double a = 0.0;
        for (int e = 0; e < 32; ++e)
            if (fabs((double)xb[e]) > a)
                a = fabs((double)xb[e]);
        const uint16_t h = qo_scale_of(a);
        const double s = qo_half_to_double(h);
        scales[blk] = h;
        for (int e = 0; e < 32; ++e)
            codes[32 * blk + e] = (int8_t)(s > 0.0 ? qo_code_of((double)xb[e], s) : 0);
    }
    return 0;
}

/*
 * Append T new tokens at positions pos0 .. pos0+T-1 of one problem's cache:
 *   k_new, v_new  float [T][Hkv][D]   -> Kq, Vq int8 [N][Hkv][D] and
 *                                        Ksc, Vsc fp16 [N][Hkv][D/32]
 *   kidx_new      float [T][di]       -> K_idx fp16 [N][di] (nearest, ties even)
 * Every other cell is left as it is.
 */
int qo_kv_append(int T, int N, int Hkv, int D, int di, int pos0, const float* k_new,
                 const float* v_new, const float* kidx_new, int8_t* Kq, uint16_t* Ksc,
                 int8_t* Vq, uint16_t* Vsc, uint16_t* K_idx)
{
    if (T < 1 || Hkv < 1 || D < 32 || D % 32 || di < 1 || pos0 < 0 || pos0 + T > N)
        return -1;
    for (int t = 0; t < T; ++t) {
        const size_t cell = (size_t)(pos0 + t);
        for (int g = 0; g < Hkv; ++g) {
            const size_t src = ((size_t)t * Hkv + g) * D;
            const size_t dst = (cell * Hkv + g) * D;
            const size_t sdst = (cell * Hkv + g) * (D / 32);
            qo_quant_row(D, k_new + src, Kq + dst, Ksc + sdst);
            qo_quant_row(D, v_new + src, Vq + dst, Vsc + sdst);
        }
        for (int i = 0; i < di; ++i)
            K_idx[cell * di + i] = qo_double_to_half((double)kidx_new[(size_t)t * di + i]);
    }
    return 0;
}

/* ------------------------------------------------------- gated output --- */

/*
 * Output gate ([r20] section 3 pairs the attention with a gate: random
 * "q/gate" inputs, "attention + gate" checked together; [r5c] Target 2
 * sizes q and gate together at 12288 floats per token, i.e. one gate value
 * per output element of the 24 x 256 heads).  The gate function is not
 * stated; the plain reading is an elementwise logistic sigmoid:
 *   out[t][h][d] = merge(...)[t][h][d] * 1 / (1 + exp(-gate[t][h][d])).
 *   gate [T][Hq][D] in double (from fp32 or fp16 inputs)
 */
int qo_merge_gated(int T, int Hq, int P, int D, const double* pm, const double* pl,
                   const double* po, const double* gate, double* out)
{
    const int rc = qo_merge(T, Hq, P, D, pm, pl, po, out);
    if (rc != 0)
        return rc;
    for (size_t i = 0; i < (size_t)T * Hq * D; ++i)
        out[i] *= 1.0 / (1.0 + exp(-gate[i]));
    return 0;
}
