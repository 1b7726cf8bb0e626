/*
 * qsa.h -- C ABI of the MI355X (gfx950) QSA top-k sparse attention library
 * (libqsa.so).
 *
 * QSA, as the audit pages describe it, attends each query token to a small
 * selected subset of a long KV cache:
 *   1. an indexer scores every visible cached cell against the token and
 *      keeps the top-k ("opus r15 track A: prompt_chunk wave zipping, fused
 *      alpha|beta GEMM, QSA PSO pre-warm, 24 GB chunk 2048", "what changed"
 *      item 1: qsa_score_mm / qsa_topk, used once a prompt exceeds 2051
 *      tokens; "Round 5 Track C Report: Direct FP16 qcurh in qsa_prep +
 *      PromptGemm Dead Buffer Removal & Layer-Local Aliasing", section 1
 *      Target 2: 2051 selected-id words per token);
 *   2. softmax attention over only the kept cells of an int8 KV cache with
 *      fp16 scales, split into chunks that each produce a (max, sum,
 *      unnormalised output) partial ("opus r20 track A: MTP map mlock +
 *      qsa_attn / qsa_merge decode tweaks", section 2 "qsa.metal", qsa_attn;
 *      section 3 "verification": random int8 KV with fp16 scales);
 *   3. a log-sum-exp merge of the chunk partials (same page, section 2,
 *      qsa_merge).
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates nothing and never synchronises; every call only
 *     enqueues kernels on `stream` (a hipStream_t passed as void*, NULL =
 *     the default stream) and returns.  Two calls keep device state of the
 *     library between calls: qsa_index_topk_noalloc (its fixed workspace)
 *     and qsa_decode_window (its grid barrier words); the others keep none.
 *   - Arguments are validated on the host before anything is enqueued.  An
 *     invalid call returns a negative qsa_status and enqueues nothing.  A
 *     kernel launch failure returns QSA_ERR_HIP.  There is no device-side
 *     error reporting: contents (ids out of range, NaN scores) are not
 *     checked.
 *   - Calls are thread-safe on the host.  On the device, calls of
 *     qsa_index_topk_noalloc, and calls of qsa_decode_window, must not
 *     overlap on one GPU (see there).
 *   - B = `batch` independent problems are processed by one call; problem b
 *     reads and writes the b-th slice of every tensor.
 *   - fp16 means IEEE binary16.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_VERSION 1

#if defined(__GNUC__) || defined(__clang__)
#define QSA_API __attribute__((visibility("default")))
#else
#define QSA_API
#endif

typedef enum {
    QSA_OK = 0,
    QSA_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size or shape */
    QSA_ERR_UNSUPPORTED = -2,  /* valid, but no kernel variant for it */
    QSA_ERR_WORKSPACE = -3,    /* workspace missing or too small */
    QSA_ERR_HIP = -4           /* a kernel launch failed */
} qsa_status;

typedef enum { QSA_F32 = 0, QSA_F16 = 1 } qsa_dtype;

/* Kernel family of qsa_attend (qsa_attn_desc.algo). */
typedef enum {
    QSA_ATTEND_AUTO = 0,    /* currently QSA_ATTEND_MATRIX */
    QSA_ATTEND_MATRIX = 1,  /* matrix cores (MFMA) with split fp16 operands */
    QSA_ATTEND_VECTOR = 2   /* fp32 vector FMAs */
} qsa_attend_algo;

/* Static description of a status code (never NULL). */
QSA_API const char* qsa_status_string(int status);

/* QSA_VERSION of the built library. */
QSA_API int qsa_version(void);

/* ------------------------------------------------------------------------
 * qsa_index_topk -- index score + top-k selection.
 *
 * Token t of problem b sits at position pos[t] = pos0 + t and sees the cells
 * 0..pos[t] (causal, own cell included).  Its score against visible cell j
 * is the dot product of its fp16 index query with the cell's fp16 index key,
 * accumulated in fp32 (fp16 products are exact in fp32).  If the token sees
 * at most dense_max cells, or at most k, all visible cells are kept (the
 * dense fallback below the 2051-cell bound named in the r15 audit page);
 * otherwise the k highest-scoring visible cells are kept, equal scores going
 * to the lower cell index.
 *
 * Inputs
 *   q_idx  fp16 [B][T][d_idx]      16-byte aligned
 *   K_idx  fp16 [B][N][d_idx]      16-byte aligned
 * Outputs
 *   ids    int32 [B][T][ids_cap]   kept cell ids in ascending order, then -1
 *   n_sel  int32 [B][T]            number of kept cells of each token
 * Workspace
 *   ws     device scratch of at least qsa_index_topk_workspace(desc) bytes,
 *          16-byte aligned; its contents on entry do not matter.
 *
 * Selection is exact on the fp32 scores the kernels compute: ids equal a
 * full sort by (score desc, index asc) of those scores.  Each fp32 score is
 * the sum of the exact fp16 x fp16 products, rounded in an order that
 * depends on the kernel variant (one token per call, 2..16 tokens, more),
 * so it is within gamma_d * sum_i |q_i k_i| of the exact score (gamma_d =
 * d u / (1 - d u), u = 2^-24, d = d_idx).  A kept id can therefore differ
 * from the exact-arithmetic selection only for cells whose exact score lies
 * within 2 gamma_d max_j sum_i |q_i k_ji| of the k-th exact score.  Where
 * every partial sum is exact in fp32 (e.g. inputs that are multiples of
 * 2^-5 in [-4, 4] with d_idx <= 1024) the selection is the exact one.
 *
 * Supported: d_idx in {64, 128}; 1 <= k <= ids_cap; 0 <= dense_max <=
 * ids_cap; 0 <= pos0; pos0 + T <= N <= 2^22; 1 <= batch*T <= 65535.
 * --------------------------------------------------------------------- */
typedef struct qsa_index_desc {
    int batch;      /* B */
    int T;          /* query tokens per problem */
    int n_cells;    /* N cached cells per problem */
    int d_idx;      /* index key dimension */
    int k;          /* cells kept per token */
    int pos0;       /* position of token 0 */
    int dense_max;  /* keep every visible cell while visible <= dense_max */
    int ids_cap;    /* row length of ids (>= max(k, dense_max)) */
} qsa_index_desc;

QSA_API size_t qsa_index_topk_workspace(const qsa_index_desc* desc);

QSA_API int qsa_index_topk(const qsa_index_desc* desc, const void* q_idx, const void* K_idx,
                   int32_t* ids, int32_t* n_sel, void* ws, size_t ws_bytes,
                   void* stream);

/* ------------------------------------------------------------------------
 * qsa_index_topk_noalloc -- qsa_index_topk without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops and harnesses that forbid allocation).
 *
 * The workspace is a fixed array of QSA_NOALLOC_WORKSPACE_BYTES in device
 * memory inside the library, one per GPU, held by that GPU until the
 * process ends; its address on a device is looked up once, on the first
 * call on that device.  The call allocates nothing.  Inputs, outputs,
 * results and errors are those of qsa_index_topk; a shape whose
 * qsa_index_topk_workspace(desc) exceeds QSA_NOALLOC_WORKSPACE_BYTES
 * returns QSA_ERR_WORKSPACE and enqueues nothing.
 *
 * Every call on one GPU uses that GPU's one array, and the kernels leave
 * their intermediate data in it: calls that overlap on one GPU (from several
 * streams or threads without ordering between them) race and give undefined
 * results.  Calls ordered on one stream are safe.
 * --------------------------------------------------------------------- */
#define QSA_NOALLOC_WORKSPACE_BYTES (64u << 20)

QSA_API int qsa_index_topk_noalloc(const qsa_index_desc* desc, const void* q_idx,
                                   const void* K_idx, int32_t* ids, int32_t* n_sel,
                                   void* stream);

/* ------------------------------------------------------------------------
 * qsa_attend -- split-KV attention partials over the kept cells
 * ("opus r20 ..." page, section 2, qsa_attn).
 *
 * Query head h reads KV head g = h / (Hq / Hkv).  The ids row of token t is
 * cut into P contiguous chunks of S = ceil(n_sel[t] / P) ids; chunk c covers
 * row positions [c*S, min((c+1)*S, n_sel[t])) and may be empty.  For chunk c
 * and head h, with x_j = scale * sum_d q[h][d] * Kq[j][g][d] * Ksc[j][g][d/32]:
 *   m = max_j x_j,   l = sum_j exp(x_j - m),
 *   o[d] = sum_j exp(x_j - m) * Vq[j][g][d] * Vsc[j][g][d/32]   (unnormalised)
 * An empty chunk gives m = -inf, l = 0, o = 0.  scale = desc->scale, or
 * 1/sqrt(D) when desc->scale is 0 (no scale is stated by the pages; the
 * usual softmax-attention scale is the default).
 *
 * Arithmetic.  QSA_ATTEND_VECTOR evaluates the definition with fp32 FMAs.
 * QSA_ATTEND_MATRIX (the default) runs both products on the matrix cores
 * with fp16 operands that carry the fp32 values: int8 codes are exact in
 * fp16; an fp32 query element and each weight exp(x_j - m) * Vsc are split
 * into two fp16 halves (hi + lo, 22 significant bits) whose products
 * accumulate in fp32.  Exact power-of-two shifts (per item for the query,
 * per 32-cell tile for weight x V scale) keep both halves finite and normal
 * for any finite query and any finite fp16 scale, so the results agree
 * with the fp32 definition to within about 1e-6 relative to the output
 * scale over the whole value range (tested from fp16-subnormal scales to
 * 8000 and |q| up to 1e5).  fp16 queries are used as given.
 *
 * Inputs
 *   q      [B][T][Hq][D], fp32 (q_dtype QSA_F32) or fp16 (QSA_F16), 16-byte
 *          aligned
 *   Kq,Vq  int8 codes; cell j of KV head g of problem b starts at
 *          base + b*batch_stride + j*cell_stride + g*D        (bytes)
 *   Ksc,Vsc fp16 scales, one per 32 elements; the scales of (b, j, g) start
 *          at base + b*batch_stride + j*cell_stride + g*(D/32)*2 (bytes)
 *          Dense default layouts: Kq/Vq [B][N][Hkv][D], Ksc/Vsc
 *          [B][N][Hkv][D/32]; a stride of 0 selects the dense default, so a
 *          caller may also interleave codes and scales of a cell.
 *   ids    int32 [B][T][ids_cap], n_sel int32 [B][T] (as written by
 *          qsa_index_topk, or any ids in [0, N) -- out-of-range ids are
 *          undefined behaviour).  Row entries at or beyond n_sel[t] are never
 *          read.
 * Output
 *   partials  float, qsa_partials_floats(desc) elements, 16-byte aligned:
 *             m [B][T][Hq][P] at offset 0,
 *             l [B][T][Hq][P] at offset B*T*Hq*P,
 *             o [B][T][Hq][P][D] at offset 2*B*T*Hq*P.
 *
 * Supported: D in {64, 256}; Hq % Hkv == 0 with Hq/Hkv in {1,2,4,8,12,16};
 * 1 <= P <= 64; n_sel[t] <= ids_cap; all four cache base pointers and
 * batch strides 16-byte aligned; Kq/Vq cell strides multiples of 16;
 * Ksc/Vsc cell strides multiples of D/16 (the bytes of one head's scales);
 * batch*T*Hq*P <= 2^31-1.
 * --------------------------------------------------------------------- */
typedef struct qsa_attn_desc {
    int batch;           /* B */
    int T;               /* query tokens per problem */
    int Hq;              /* query heads */
    int Hkv;             /* KV heads */
    int D;               /* head dimension */
    int P;               /* split-KV chunks per token */
    int ids_cap;         /* row length of ids */
    int n_cells;         /* N, cells per problem (sizes the default batch strides) */
    float scale;         /* softmax scale; 0 selects the default 1/sqrt(D) */
    int q_dtype;         /* qsa_dtype of q */
    int out_dtype;       /* qsa_dtype of the merged output */
    int algo;            /* qsa_attend_algo; 0 (zero-initialised) = default */
    long long kq_cell_stride, ksc_cell_stride, vq_cell_stride, vsc_cell_stride;
    long long kq_batch_stride, ksc_batch_stride, vq_batch_stride, vsc_batch_stride;
} qsa_attn_desc;

QSA_API size_t qsa_partials_floats(const qsa_attn_desc* desc);

QSA_API int qsa_attend(const qsa_attn_desc* desc, const void* q, const int8_t* Kq,
               const void* Ksc, const int8_t* Vq, const void* Vsc,
               const int32_t* ids, const int32_t* n_sel, float* partials,
               void* stream);

/* ------------------------------------------------------------------------
 * qsa_merge -- log-sum-exp merge of the P chunk partials
 * ("opus r20 ..." page, section 2, qsa_merge).
 *   M = max_c m_c;  e_c = exp(m_c - M);  L = sum_c l_c e_c  (fma, c order);
 *   out[d] = (sum_c o_c[d] e_c) / L   (fma in c order, then one division)
 * A row whose chunks are all empty writes 0.
 *
 * Input   partials as written by qsa_attend with the same desc.
 * Output  out [B][T][Hq][D], fp32 or fp16 (round to nearest even) per
 *         desc->out_dtype, 16-byte aligned.
 * Supported: as qsa_attend.
 * --------------------------------------------------------------------- */
QSA_API int qsa_merge(const qsa_attn_desc* desc, const float* partials, void* out,
              void* stream);

/* ------------------------------------------------------------------------
 * qsa_merge_gated -- qsa_merge followed by the output gate the "opus r20
 * ..." page pairs the attention with (section 3: random "q/gate" inputs,
 * "attention + gate" checked together; the "Round 5 Track C ..." page,
 * Target 2, sizes q and gate together at 12288 floats per token: one gate
 * value per output element).  The gate function is not stated; the plain
 * reading is an elementwise logistic sigmoid:
 *   out[b][t][h][d] = merged[b][t][h][d] * 1 / (1 + exp(-gate[b][t][h][d]))
 * computed in fp32 before the optional fp16 rounding of out.
 * gate: [B][T][Hq][D] in the query dtype (desc->q_dtype), 16-byte aligned;
 * NULL gives qsa_merge.  Other arguments, errors and support as qsa_merge.
 * --------------------------------------------------------------------- */
QSA_API int qsa_merge_gated(const qsa_attn_desc* desc, const float* partials, const void* gate,
                            void* out, void* stream);

/* ------------------------------------------------------------------------
 * qsa_attend_merge -- qsa_attend followed by qsa_merge_gated in ONE kernel:
 * the attention over the kept cells of the "opus r20 ..." page, section 2
 * (qsa_attn), whose chunk partials are merged by that section's qsa_merge
 * formula and gated as qsa_merge_gated describes, without writing the
 * partials to memory.
 *
 * Each workgroup of the matrix kernel computes four (token, chunk) items;
 * when P divides 4 these are all the chunks of whole tokens, so the
 * workgroup merges its own partials in on-chip memory.  The merge runs the
 * same operations in the same order as qsa_merge on the same partial
 * values, so out equals qsa_attend + qsa_merge_gated with the same
 * arguments bit for bit.
 *
 * Arguments: desc, q, Kq, Ksc, Vq, Vsc, ids, n_sel as qsa_attend; gate and
 * out as qsa_merge_gated (gate NULL: no gate).  No partials are written.
 * Supported: as qsa_attend, with P in {1, 2, 4} and algo AUTO or MATRIX
 * (else QSA_ERR_UNSUPPORTED: use the two calls).
 * --------------------------------------------------------------------- */
QSA_API int qsa_attend_merge(const qsa_attn_desc* desc, const void* q, const int8_t* Kq,
                             const void* Ksc, const int8_t* Vq, const void* Vsc,
                             const int32_t* ids, const int32_t* n_sel, const void* gate,
                             void* out, void* stream);

/* ------------------------------------------------------------------------
 * qsa_kv_append -- write T new tokens into the cache, the step that feeds
 * the path: their K and V rows become int8 codes with one fp16 scale per
 * 32 elements (the cache format of the "opus r20 ..." page, section 3:
 * random int8 KV with fp16 scales) and their index keys become fp16.
 *
 * The pages do not spell out the quantiser; the plain absmax reading is
 * used.  For every block of 32 consecutive elements x of a (token, KV head)
 * row:
 *   a = max |x|,  s = fp16(a / 127)  (saturating at 65504),
 *   c = clamp(round(x / s), -127, 127),  c = 0 when s = 0,
 * where both roundings are to nearest, ties to even, of the exact values
 * (the library decides each against its neighbours with exact products).
 * Index keys: fp16(x), to nearest, ties to even.  The results equal the
 * oracle's bit for bit.
 *
 * Token t of problem b goes to cell pos0 + t; no other cell is written.
 * Inputs (finite values)
 *   k_new, v_new  fp32 [B][T][Hkv][D], 16-byte aligned
 *   kidx_new      fp32 [B][T][d_idx], 16-byte aligned, or NULL (index keys
 *                 are then not written)
 * Outputs (the cache, in the layouts and strides qsa_attend reads: zero
 * strides select the dense defaults [B][N][Hkv][D] and [B][N][Hkv][D/32])
 *   Kq, Vq        int8 codes;  Ksc, Vsc  fp16 scales
 *   K_idx         fp16 [B][N][d_idx] (ignored when kidx_new is NULL)
 * Supported: D a multiple of 32 up to 1024; d_idx a multiple of 4;
 * 0 <= pos0, pos0 + T <= n_cells; batch*T*Hkv*D/32 <= 2^30; code pointers
 * and batch strides 16-byte aligned, code cell strides multiples of 16,
 * scale pointers 2-byte aligned and scale strides even.
 * --------------------------------------------------------------------- */
typedef struct qsa_append_desc {
    int batch;           /* B */
    int T;               /* new tokens per problem */
    int n_cells;         /* N, cells per problem */
    int pos0;            /* cell of token 0 */
    int Hkv;             /* KV heads */
    int D;               /* head dimension */
    int d_idx;           /* index key dimension */
    int reserved;        /* must be 0 */
    long long kq_cell_stride, ksc_cell_stride, vq_cell_stride, vsc_cell_stride;
    long long kq_batch_stride, ksc_batch_stride, vq_batch_stride, vsc_batch_stride;
} qsa_append_desc;

QSA_API int qsa_kv_append(const qsa_append_desc* desc, const float* k_new, const float* v_new,
                          const float* kidx_new, int8_t* Kq, void* Ksc, int8_t* Vq, void* Vsc,
                          void* K_idx, void* stream);

/* ------------------------------------------------------------------------
 * qsa_decode_window -- one decode step of the whole path in ONE kernel
 * launch: qsa_kv_append, then qsa_index_topk, qsa_attend and
 * qsa_merge_gated, each phase reading what the one before wrote.
 *
 * The "opus r20 ..." page (section 4, timings) times the QSA step of a
 * decode token as one dependent window of dispatches; with few problems the
 * gaps between separate launches cost more than their work.  Here one
 * cooperative launch (every workgroup resident at once) runs the phases,
 * separated by grid-wide barriers, with the device code of the separate
 * calls.  The results equal those of the four calls with the same
 * descriptors bit for bit: new cache codes, scales and index keys; ids and
 * n_sel; the output.  The index phase computes the fp32 scores as
 * qsa_index_topk does for batch < 128 or n_cells > 16384 and keeps the same
 * exact top-k of them; for batch >= 128 with n_cells <= 16384,
 * qsa_index_topk scores in another summation order, so ids can differ from
 * its ids, within the rounding bound stated there (never where every
 * partial sum is exact in fp32).
 *
 * Arguments are those of the four calls: pdesc/k_new/v_new/kidx_new/cache
 * as qsa_kv_append; idesc/q_idx/K_idx/ids/n_sel as qsa_index_topk; adesc/
 * q/cache/ids/n_sel as qsa_attend; gate/out as qsa_merge_gated.  The three
 * descriptors must describe the same step: T = 1 in each, equal batch and
 * n_cells, pdesc->pos0 == idesc->pos0 (the new token's cell, which its own
 * index query sees), equal Hkv and D, equal ids_cap, equal d_idx when
 * kidx_new is given, and the same resolved cache strides (else
 * QSA_ERR_INVALID_ARG).  The partials live in the workspace.  Ksc and Vsc
 * must be 16-byte aligned here.
 *
 * Workspace: at least qsa_decode_window_workspace(idesc, adesc) bytes,
 * 256-byte aligned, contents on entry irrelevant.  Its first 32-bit word is
 * 0 after a normal call; it is nonzero if a barrier wait gave up (about a
 * second per barrier; only possible if the grid could not run together,
 * which the cooperative launch excludes) -- the outputs of that call are
 * then invalid and later window calls in the process are unreliable.
 *
 * Concurrency: every call on one GPU uses the same two barrier words in
 * the library's device memory (they return to their start state after each
 * call, so calls ordered on one stream and HIP graph replays are fine).
 * Window calls that overlap on one GPU are not supported: their barriers
 * interfere, and the results are undefined (the bounded waits still end
 * every call).
 *
 * Supported: q and out fp32 (q_dtype = out_dtype = QSA_F32), algo AUTO or
 * MATRIX; (Hq/Hkv, D) in {(12, 256), (4, 64)}; d_idx in {64, 128}; P a
 * multiple of 4 up to 64; pos0 < 16384 (one workgroup selects a row from
 * registers; longer rows are faster through the separate calls); else
 * QSA_ERR_UNSUPPORTED.  QSA_ERR_HIP if the
 * device cannot launch the kernel cooperatively.
 * --------------------------------------------------------------------- */
QSA_API size_t qsa_decode_window_workspace(const qsa_index_desc* idesc,
                                           const qsa_attn_desc* adesc);

QSA_API int qsa_decode_window(const qsa_append_desc* pdesc, const qsa_index_desc* idesc,
                              const qsa_attn_desc* adesc, const float* k_new,
                              const float* v_new, const float* kidx_new, int8_t* Kq, void* Ksc,
                              int8_t* Vq, void* Vsc, void* K_idx, const void* q_idx,
                              const void* q, const void* gate, int32_t* ids, int32_t* n_sel,
                              void* out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * qsa_step -- one step of the whole path for every workload shape, in as
 * few kernel launches as the shape allows: qsa_kv_append of the T new
 * tokens, then qsa_index_topk, qsa_attend and qsa_merge_gated, each reading
 * what the one before wrote.
 *
 * Each call is its own kernel (or kernels), with its own ramp-up and drain,
 * and data passed between calls goes through memory, so the step folds
 * calls together where one workgroup already owns everything a call needs:
 *   - the append runs inside the index kernel when that kernel gives each
 *     problem one workgroup (one token per problem, batch >= 128, rows of
 *     at most 16384 cells, some token selecting): that workgroup writes its
 *     problem's new token, then scans the keys;
 *   - with one token per problem otherwise (fewer problems, or longer
 *     rows; some token selecting; Hkv * D <= 512), the append runs inside
 *     the chip-wide key scan: the workgroup whose rows end with the new cell
 *     writes the problem's new token (not for rows of 65537 to 262144 cells
 *     with k <= 4096, whose index path starts with a sampling kernel);
 *   - the merge and the gate run inside the attention kernel with the
 *     matrix kernel when P is 1, 2 or 4 (as qsa_attend_merge), and when P
 *     is a multiple of 4 above 4 with batch * T * Hkv >= 512 (the kernel then
 *     gives each (token, KV head) one workgroup, which writes its chunks'
 *     partials to the workspace and merges them itself).
 * Otherwise the calls run as their own kernels, in order.  The results
 * (new cache codes, scales and index keys; ids and n_sel; out) equal those
 * of the four calls with the same descriptors bit for bit.
 *
 * Arguments are those of the four calls: pdesc/k_new/v_new/kidx_new/cache
 * as qsa_kv_append; idesc/q_idx/K_idx/ids/n_sel as qsa_index_topk; adesc/
 * q/cache/ids/n_sel as qsa_attend; gate/out as qsa_merge_gated.  The three
 * descriptors must describe the same step: equal T, batch and n_cells,
 * pdesc->pos0 == idesc->pos0, equal Hkv and D, equal ids_cap, equal d_idx
 * when kidx_new is given, and the same resolved cache strides (else
 * QSA_ERR_INVALID_ARG).  Ksc and Vsc must be 16-byte aligned.
 *
 * Workspace: at least qsa_step_workspace(idesc, adesc) bytes (the index
 * workspace, plus room for the partials unless P is 1, 2 or 4 with the
 * matrix kernel), 256-byte aligned, contents on entry irrelevant.
 * Supported: what each of the four calls supports.
 * --------------------------------------------------------------------- */
QSA_API size_t qsa_step_workspace(const qsa_index_desc* idesc, const qsa_attn_desc* adesc);

QSA_API int qsa_step(const qsa_append_desc* pdesc, const qsa_index_desc* idesc,
                     const qsa_attn_desc* adesc, const float* k_new, const float* v_new,
                     const float* kidx_new, int8_t* Kq, void* Ksc, int8_t* Vq, void* Vsc,
                     void* K_idx, const void* q_idx, const void* q, const void* gate,
                     int32_t* ids, int32_t* n_sel, void* out, void* ws, size_t ws_bytes,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
