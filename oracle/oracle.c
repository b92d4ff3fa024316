/*
 * Reference oracle for one layer of the hybrid-head decode-attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP path.
 *
 * It is a plain, slow, obviously-correct evaluation of the definitions, in
 * double precision, parallelised only over independent (sequence, KV head)
 * pairs.  Sources (cited by title and section):
 *   [Digest]  "LycheeDecode: Accelerating Long-Context LLM Inference via
 *             Hybrid-Head Sparse Decoding" -- long-form paper digest
 *             (paper-graph-ui), section 3.4 "Detailed, Sentence-Based
 *             Technical Breakdown" (Eq. 1, Eq. 2, Eq. 3, the propagation and
 *             layer-0 rules, the complete decoding loop = Algorithm 1, and
 *             the hyper-parameter summary's GQA pooling rule).
 *   [Notes]   papernotes.org notes on the same paper, "方法详解 / 关键设计"
 *             items 1 and 2 (retrieval heads, sparse heads).
 *
 * Readings taken where the pages are silent (each one is also listed in the
 * design notes of the repository):
 *   R1  roles and critical-token sets are per KV head; all G query heads of
 *       a KV head share them (budgets on the pages are counted in KV heads).
 *   R2  the selection score of a KV head is the mean of its G query heads'
 *       pre-softmax logits (= logits of the average-pooled query), ranked
 *       descending; softmax is monotone, so this ranks A of Eq. 2.
 *   R3  ties in the selection score go to the lower token index.
 *   R4  S is stored as k int32 per (sequence, KV head), ascending; when the
 *       context n is shorter than k only min(k, n) entries are valid and
 *       the rest are -1.
 *   R5  no causal mask, no forced sink / recent tokens; rows >= n are never
 *       read; scale 1/sqrt(d) for both head kinds.
 *   R6  query head h reads KV head floor(h / G).
 *   R16 selection rules other than top-k (the digest's ablation of
 *       selection methods, section 4.4.1 / Figure 6, names them without a
 *       formula): Ratio(theta) keeps the top min(k, ceil(theta * n)) tokens
 *       (at least 1), theta * n evaluated in double; Threshold(tau) keeps the
 *       tokens whose pooled score (R2) is >= tau, the k highest of them if
 *       more.  S then holds fewer than min(k, n) valid entries, padded with
 *       -1; a sparse head skips -1 entries (an empty set gives output 0).
 *       TopP(p) keeps the shortest prefix of that ranking whose share of
 *       the softmax of the pooled scores over the whole context reaches p
 *       (the k highest if it is longer); shares are added in rank order.
 *   R17 block-granular selection (the digest's block size 64 of the kernel,
 *       with no rule for a block's score): the context is cut into blocks
 *       of bs tokens (the last one may be shorter); a block's score is the
 *       largest pooled score (R2) of its tokens; the floor(k / bs) highest
 *       blocks (score desc, block index asc; all blocks if fewer) are kept,
 *       and S lists their tokens ascending, padded with -1.
 *   R18 the multi-step loop around the step (Algorithm 1's cache append,
 *       and the Cache Correction of the digest's reasoning setup, a dense
 *       re-prefill of the last 32 decoded tokens every 32 steps): only the
 *       attention part is evaluated.  The append writes the new token's K
 *       and V rows at position n of each (sequence, KV head) and makes the
 *       context n + 1.  The correction attention gives each of the last T
 *       positions p = n - T + t (t < T) of a sequence, for every query head,
 *       dense causal attention over the cache rows 0..p (Eq. 1 with the
 *       prefill's causal mask), with that position's own query.
 *
 * Parity status: pinned (see the header of oracle/__init__.py for the list
 * of pins and the tests that hold them).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG -1
#define ORACLE_ERR_S_RANGE -2
#define ORACLE_ERR_NCTX -3
#define ORACLE_ERR_MEM -4

/* Element read: dtype 0 = IEEE fp32, dtype 1 = bfloat16 stored as uint16
 * (the upper 16 bits of an fp32).  Both convert to double exactly. */
static double elem(const void* base, int dtype, size_t i) {
    if (dtype == 0) return (double)((const float*)base)[i];
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Dot product of query row (q_off) with cache row (k_off), both of length d,
 * accumulated in double in index order. */
static double dot_row(const void* q, size_t q_off, const void* kc, size_t k_off,
                      int d, int dtype) {
    double s = 0.0;
    for (int t = 0; t < d; ++t) s += elem(q, dtype, q_off + t) * elem(kc, dtype, k_off + t);
    return s;
}

/* Ordering for top-k [Digest 3.4 Eq. 2 with reading R3]: larger score first,
 * equal scores by smaller index first.  A strict total order. */
typedef struct { double s; int32_t j; } scored;
static int cmp_desc_score_asc_index(const void* a, const void* b) {
    const scored* x = (const scored*)a;
    const scored* y = (const scored*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}
static int cmp_int_asc(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* Softmax-weighted sum over a list of rows [Digest 3.4 Eq. 1 and Eq. 3]:
 *   w_r = exp(z_r - max z),  out = sum_r (w_r / sum w) * V[row_r].
 * rows == NULL means rows 0..cnt-1. */
static void softmax_weighted_sum(const double* z, const int32_t* rows, int cnt,
                                 const void* vc, size_t v_base, int d, int dtype,
                                 double* out) {
    double m = -INFINITY;
    for (int r = 0; r < cnt; ++r) if (z[r] > m) m = z[r];
    double Z = 0.0;
    for (int r = 0; r < cnt; ++r) Z += exp(z[r] - m);
    for (int t = 0; t < d; ++t) out[t] = 0.0;
    for (int r = 0; r < cnt; ++r) {
        double p = exp(z[r] - m) / Z;
        size_t row = rows ? (size_t)rows[r] : (size_t)r;
        for (int t = 0; t < d; ++t) out[t] += p * elem(vc, dtype, v_base + row * (size_t)d + t);
    }
}

#define ORACLE_RULE_TOPK 0
#define ORACLE_RULE_RATIO 1
#define ORACLE_RULE_THRESHOLD 2
#define ORACLE_RULE_TOPP 3
#define ORACLE_RULE_BLOCK 4

/*
 * One layer of the step (the per-layer body of Algorithm 1 in [Digest 3.4],
 * attention part only), with the selection rule of reading R16 (rule, param).
 *
 *   q        [B, Hq, d]           dtype
 *   kc, vc   [B, Hkv, max_ctx, d] dtype
 *   role     [Hkv]  1 = retrieval, 0 = sparse            (reading R1)
 *   S_in     [B, Hkv, k] or NULL when every role is retrieval
 *   S_out    [B, Hkv, k]          written for every head
 *   out      [B, Hq, d]  double
 *   n_ctx    [B]        1 <= n_ctx[b] <= max_ctx
 *   scores   optional [B, Hkv, max_ctx] double: the pooled selection score of
 *            every retrieval head (reading R2); untouched for sparse heads
 *   nthreads OpenMP threads (<= 0: library default)
 * Returns ORACLE_OK or a negative error code.
 */
int oracle_layer_select(int B, int Hq, int Hkv, int d, int max_ctx, int dtype,
                        const void* q, const void* kc, const void* vc,
                        const uint8_t* role, const int32_t* S_in, int32_t* S_out,
                        double* out, const int32_t* n_ctx, int k, int rule, double param,
                        double* scores, int nthreads) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_ctx <= 0 || k <= 0) return ORACLE_ERR_ARG;
    if (rule != ORACLE_RULE_TOPK && rule != ORACLE_RULE_RATIO && rule != ORACLE_RULE_THRESHOLD &&
        rule != ORACLE_RULE_TOPP && rule != ORACLE_RULE_BLOCK)
        return ORACLE_ERR_ARG;
    if (rule == ORACLE_RULE_BLOCK && !(param >= 1.0 && param <= 4096.0 && param == floor(param) && k >= (int)param))
        return ORACLE_ERR_ARG;
    if ((rule == ORACLE_RULE_RATIO || rule == ORACLE_RULE_TOPP) && !(param > 0.0 && param <= 1.0))
        return ORACLE_ERR_ARG;
    if (Hq % Hkv != 0 || (dtype != 0 && dtype != 1)) return ORACLE_ERR_ARG;
    if (!q || !kc || !vc || !role || !S_out || !out || !n_ctx) return ORACLE_ERR_ARG;
    for (int g = 0; g < Hkv; ++g)
        if (!role[g] && !S_in) return ORACLE_ERR_ARG;
    for (int b = 0; b < B; ++b)
        if (n_ctx[b] < 1 || n_ctx[b] > max_ctx) return ORACLE_ERR_NCTX;

    const int G = Hq / Hkv;
    const double c = 1.0 / sqrt((double)d);          /* 1/sqrt(d_k), Eq. 1 and Eq. 3 */
    int status = ORACLE_OK;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
    for (int bg = 0; bg < B * Hkv; ++bg) {
        const int b = bg / Hkv, g = bg % Hkv;
        const int n = n_ctx[b];
        const int ke = k < n ? k : n;                       /* reading R4 */
        const size_t kv_base = ((size_t)b * Hkv + g) * (size_t)max_ctx * d;
        int32_t* s_out = S_out + ((size_t)b * Hkv + g) * k;

        if (role[g]) {
            /* Retrieval head: dense attention over all n tokens (Eq. 1), then
             * S^(l+1) = argsTopK(A, k) (Eq. 2) on the GQA-pooled score. */
            double* z = (double*)malloc(sizeof(double) * (size_t)n);
            double* pooled = (double*)calloc((size_t)n, sizeof(double));
            scored* order = (scored*)malloc(sizeof(scored) * (size_t)n);
            if (!z || !pooled || !order) {
                free(z); free(pooled); free(order);
#pragma omp atomic write
                status = ORACLE_ERR_MEM;
                continue;
            }
            for (int i = 0; i < G; ++i) {
                const int h = g * G + i;                    /* reading R6 */
                const size_t q_off = ((size_t)b * Hq + h) * d;
                for (int j = 0; j < n; ++j) {
                    z[j] = c * dot_row(q, q_off, kc, kv_base + (size_t)j * d, d, dtype);
                    pooled[j] += z[j];
                }
                softmax_weighted_sum(z, NULL, n, vc, kv_base, d, dtype, out + q_off);
            }
            for (int j = 0; j < n; ++j) {
                pooled[j] /= (double)G;                     /* mean of the G logits, R2 */
                order[j].s = pooled[j];
                order[j].j = j;
            }
            if (scores) {
                double* dst = scores + ((size_t)b * Hkv + g) * (size_t)max_ctx;
                memcpy(dst, pooled, sizeof(double) * (size_t)n);
            }
            if (rule == ORACLE_RULE_BLOCK) {
                /* reading R17: blocks of bs tokens, each scored by its largest
                 * pooled score; the floor(k / bs) highest blocks, their tokens
                 * listed ascending */
                const int bs = (int)param;
                const int nb = (n + bs - 1) / bs;
                const int kb = k / bs < nb ? k / bs : nb;
                int32_t* blocks = (int32_t*)malloc(sizeof(int32_t) * (size_t)(kb > 0 ? kb : 1));
                if (!blocks) {
                    free(z); free(pooled); free(order);
#pragma omp atomic write
                    status = ORACLE_ERR_MEM;
                    continue;
                }
                for (int blk = 0; blk < nb; ++blk) {
                    double m = pooled[blk * bs];
                    for (int j = blk * bs + 1; j < n && j < blk * bs + bs; ++j)
                        if (pooled[j] > m) m = pooled[j];
                    order[blk].s = m;
                    order[blk].j = blk;
                }
                qsort(order, (size_t)nb, sizeof(scored), cmp_desc_score_asc_index);
                for (int r = 0; r < kb; ++r) blocks[r] = order[r].j;
                qsort(blocks, (size_t)kb, sizeof(int32_t), cmp_int_asc);
                int w = 0;
                for (int r = 0; r < kb; ++r)
                    for (int j = blocks[r] * bs; j < n && j < blocks[r] * bs + bs; ++j) s_out[w++] = j;
                for (int r = w; r < k; ++r) s_out[r] = -1;
                free(blocks);
                free(z); free(pooled); free(order);
                continue;
            }
            qsort(order, (size_t)n, sizeof(scored), cmp_desc_score_asc_index);
            int cnt = ke;                                   /* reading R16 */
            if (rule == ORACLE_RULE_RATIO) {
                const double t = ceil(param * (double)n);
                const int kr = t < 1.0 ? 1 : (t > (double)n ? n : (int)t);
                cnt = kr < ke ? kr : ke;
            } else if (rule == ORACLE_RULE_THRESHOLD) {
                cnt = 0;
                while (cnt < ke && order[cnt].s >= param) ++cnt;
            } else if (rule == ORACLE_RULE_TOPP) {
                /* softmax of the pooled scores over all n tokens, shares added
                 * in rank order until they reach p */
                const double m = order[0].s;
                double Z = 0.0;
                for (int j = 0; j < n; ++j) Z += exp(pooled[j] - m);
                double cum = 0.0;
                for (int r = 0; r < ke; ++r) {
                    cum += exp(order[r].s - m) / Z;
                    if (cum >= param) {
                        cnt = r + 1;
                        break;
                    }
                }
            }
            for (int r = 0; r < cnt; ++r) s_out[r] = order[r].j;
            qsort(s_out, (size_t)cnt, sizeof(int32_t), cmp_int_asc);
            for (int r = cnt; r < k; ++r) s_out[r] = -1;
            free(z); free(pooled); free(order);
        } else {
            /* Sparse head: attention over the inherited rows only (Eq. 3), and
             * S^(l+1) = S^(l) unchanged. */
            const int32_t* s_in = S_in + ((size_t)b * Hkv + g) * k;
            int bad = 0, cnt = 0;
            int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)(ke > 0 ? ke : 1));
            for (int r = 0; r < ke && rows; ++r) {
                if (s_in[r] == -1) continue;                /* padding (reading R16) */
                if (s_in[r] < 0 || s_in[r] >= n) bad = 1;
                else rows[cnt++] = s_in[r];
            }
            if (bad || !rows) {
                free(rows);
#pragma omp atomic write
                status = bad ? ORACLE_ERR_S_RANGE : ORACLE_ERR_MEM;
                continue;
            }
            double* z = (double*)malloc(sizeof(double) * (size_t)(ke > 0 ? ke : 1));
            if (!z) {
                free(rows);
#pragma omp atomic write
                status = ORACLE_ERR_MEM;
                continue;
            }
            for (int i = 0; i < G; ++i) {
                const int h = g * G + i;
                const size_t q_off = ((size_t)b * Hq + h) * d;
                if (cnt == 0) {                             /* empty set: output 0 */
                    for (int t = 0; t < d; ++t) out[q_off + t] = 0.0;
                    continue;
                }
                for (int r = 0; r < cnt; ++r)
                    z[r] = c * dot_row(q, q_off, kc, kv_base + (size_t)rows[r] * d, d, dtype);
                softmax_weighted_sum(z, rows, cnt, vc, kv_base, d, dtype, out + q_off);
            }
            if (s_out != s_in) memmove(s_out, s_in, sizeof(int32_t) * (size_t)k);
            free(z);
            free(rows);
        }
    }
    return status;
}

/* The top-k rule (the product's default): oracle_layer_select with rule 0. */
int oracle_layer(int B, int Hq, int Hkv, int d, int max_ctx, int dtype,
                 const void* q, const void* kc, const void* vc,
                 const uint8_t* role, const int32_t* S_in, int32_t* S_out,
                 double* out, const int32_t* n_ctx, int k, double* scores,
                 int nthreads) {
    return oracle_layer_select(B, Hq, Hkv, d, max_ctx, dtype, q, kc, vc, role, S_in, S_out, out, n_ctx, k,
                               ORACLE_RULE_TOPK, 0.0, scores, nthreads);
}

/*
 * Algorithm 1's cache append (reading R18): row n_ctx[b] of every KV head of
 * sequence b receives k_new / v_new [B, Hkv, d] and n_ctx[b] grows by one.
 * A full cache (n_ctx[b] == max_ctx) is an error and changes nothing.
 */
int oracle_kv_append(int B, int Hkv, int d, int max_ctx, int dtype,
                     const void* k_new, const void* v_new, void* kc, void* vc, int32_t* n_ctx) {
    if (B <= 0 || Hkv <= 0 || d <= 0 || max_ctx <= 0 || (dtype != 0 && dtype != 1)) return ORACLE_ERR_ARG;
    if (!k_new || !v_new || !kc || !vc || !n_ctx) return ORACLE_ERR_ARG;
    for (int b = 0; b < B; ++b)
        if (n_ctx[b] < 0 || n_ctx[b] >= max_ctx) return ORACLE_ERR_NCTX;
    const size_t es = dtype == 1 ? 2 : 4;
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g) {
            const size_t dst = (((size_t)b * Hkv + g) * (size_t)max_ctx + (size_t)n_ctx[b]) * d * es;
            const size_t src = ((size_t)b * Hkv + g) * (size_t)d * es;
            memcpy((char*)kc + dst, (const char*)k_new + src, (size_t)d * es);
            memcpy((char*)vc + dst, (const char*)v_new + src, (size_t)d * es);
        }
        n_ctx[b] += 1;
    }
    return ORACLE_OK;
}

/*
 * Cache Correction's attention (reading R18): for the last T positions of
 * every sequence, p = n - T + t, each query head h (KV head floor(h / G))
 * attends densely and causally to cache rows 0..p with scale 1/sqrt(d):
 *   q    [B, T, Hq, d]      dtype, row t is position n - T + t
 *   out  [B, T, Hq, d]      double
 * Requires 1 <= T <= n_ctx[b] <= max_ctx.
 */
int oracle_correction_attention(int B, int T, int Hq, int Hkv, int d, int max_ctx, int dtype,
                                const void* q, const void* kc, const void* vc,
                                const int32_t* n_ctx, double* out, int nthreads) {
    if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_ctx <= 0) return ORACLE_ERR_ARG;
    if (Hq % Hkv != 0 || (dtype != 0 && dtype != 1)) return ORACLE_ERR_ARG;
    if (!q || !kc || !vc || !n_ctx || !out) return ORACLE_ERR_ARG;
    for (int b = 0; b < B; ++b)
        if (n_ctx[b] < T || n_ctx[b] > max_ctx) return ORACLE_ERR_NCTX;
    const int G = Hq / Hkv;
    const double c = 1.0 / sqrt((double)d);
    int status = ORACLE_OK;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int bt = 0; bt < B * T; ++bt) {
        const int b = bt / T, t = bt % T;
        const int pos = n_ctx[b] - T + t;                 /* this row's position */
        double* z = (double*)malloc(sizeof(double) * (size_t)(pos + 1));
        if (!z) {
#pragma omp atomic write
            status = ORACLE_ERR_MEM;
            continue;
        }
        for (int h = 0; h < Hq; ++h) {
            const int g = h / G;                          /* reading R6 */
            const size_t kv_base = ((size_t)b * Hkv + g) * (size_t)max_ctx * d;
            const size_t q_off = (((size_t)b * T + t) * Hq + h) * d;
            for (int j = 0; j <= pos; ++j) z[j] = c * dot_row(q, q_off, kc, kv_base + (size_t)j * d, d, dtype);
            softmax_weighted_sum(z, NULL, pos + 1, vc, kv_base, d, dtype, out + q_off);
        }
        free(z);
    }
    return status;
}
