/*
 * rattn_oracle.c -- TEST INFRASTRUCTURE, not part of the product library.
 *
 * Plain, slow fp64 reference ("oracle") for fused residual attention over a
 * shared base KV cache.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no code, header, table or
 * helper with the HIP library, and the HIP library never calls it.
 *
 * It computes the definition, written out, with no blocking, fusion or
 * reordering: it materialises every agent's full keys and values and then runs
 * textbook softmax attention.  The fused kernel reaches the same result because
 * the score and the weighted value sum are linear in the key and value
 * (ForkKV Guide, "Fused ResidualAttention" section 1, the AttnScore equations,
 * and the FAQ entry on accuracy: the reformulation is exact; LRAgent,
 * "Flash-LoRA-Attention": O = P V_base + (P V_lr) B).
 *
 * For agent a, query position t, query head h, with g = H_q / H_kv and
 * k = floor(h / g) (consecutive query heads share a KV head):
 *   1. gather the base rows of head k in logical token order; with a page
 *      table, logical token j lives in physical page table[j / page] at
 *      slot j % page (the bCache block pointers of the DualRadixTree lookup);
 *   2. materialise K_a = K_base + Lk_a Bk_a^(k) and V_a = V_base + Lv_a Bv_a^(k)
 *      (ForkKV Guide, "Mathematical Decomposition of LoRA KV Activations":
 *      K^(i) = K_base + dK^(i) with dK = (alpha/r) X A B; the low-rank cache
 *      holds X A, LRAgent's "LR cache"; alpha/r is folded into B; Bk^(k) is
 *      columns [k d, (k+1) d) of Bk; with a shared low-rank cache (LRAgent
 *      BaseLRShared) every agent uses Lk_0, Lv_0);
 *   3. append the agent's private tokens (full keys and values, no residual):
 *      all S of them when decoding, the first t+1 of them in a causal chunk;
 *   4. s_j = scale * q . K[j], scale = 1/sqrt(head_dim) unless given;
 *   5. p = exp(s - max s) / sum exp(s - max s);
 *   6. out = sum_j p_j V[j]; lse = max s + ln sum exp(s - max s).
 *
 * Inputs are read exactly: bf16 bit patterns and fp32 values are widened to
 * fp64 without rounding.  All arithmetic is fp64.
 *
 * ORACLE_MUTANT (compile-time, default 0) plants one deliberate mistake; the
 * test suite builds the mutants to show that its pins catch each of them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

enum { EL_F64 = 0, EL_F32 = 1, EL_BF16 = 2 };

typedef struct {
    int32_t n_agents, n_q_heads, n_kv_heads, head_dim, rank;
    int64_t prefix_len, priv_len;
    int32_t q_len, page_size;
    int64_t n_phys_pages;
    int32_t shared_lr, causal, elem;
    double sm_scale; /* <= 0: 1/sqrt(head_dim) */
} oracle_shape;

typedef struct {
    const void *q, *k_base, *v_base;
    const int32_t *block_table;
    const void *lk, *lv, *bk, *bv, *k_priv, *v_priv;
} oracle_inputs;

static double ld(const void *p, int64_t i, int elem) {
    if (elem == EL_F64) return ((const double *)p)[i];
    if (elem == EL_F32) return (double)((const float *)p)[i];
    uint32_t b = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &b, sizeof f);
    return (double)f;
}

int rattn_oracle_version(void) { return 1000 + ORACLE_MUTANT; }

/* Offset of element dd of logical base token j of KV head k. */
static int64_t base_index(const oracle_shape *s, const int32_t *table, int64_t j, int k, int dd) {
    const int64_t D = s->head_dim, H = s->n_kv_heads;
    if (s->page_size > 0) {
        const int64_t ps = s->page_size;
#if ORACLE_MUTANT == 8
        int64_t page = j / ps; /* mistake: ignores the page table */
#else
        int64_t page = table[j / ps];
#endif
        return ((page * H + k) * ps + (j % ps)) * D + dd;
    }
    return ((int64_t)k * s->prefix_len + j) * D + dd;
}

/*
 * Computes out [N, q_len, H_q, d] and lse [N, q_len, H_q] (lse may be NULL).
 * row_mask (may be NULL) selects rows (a, t, h) by flat index (a*q_len + t)*H_q + h;
 * unselected rows are left untouched.  Returns 0, or -1 on a shape error,
 * -2 on allocation failure.
 */
int rattn_oracle_attend(const oracle_shape *s, const oracle_inputs *in, const uint8_t *row_mask,
                        double *out, double *lse, int n_threads) {
    const int N = s->n_agents, HQ = s->n_q_heads, HK = s->n_kv_heads, D = s->head_dim, R = s->rank;
    const int64_t L = s->prefix_len, S = s->priv_len;
    const int QL = s->q_len, el = s->elem;
    if (N < 1 || HK < 1 || HQ % HK || D < 1 || R < 0 || L < 0 || S < 0 || QL < 1) return -1;
    if (s->causal && QL != S) return -1;
    if (L + S < 1) return -1;
    if (s->page_size > 0 && !in->block_table) return -1;
    const int g = HQ / HK;
#if ORACLE_MUTANT == 6
    const double scale = s->sm_scale > 0 ? s->sm_scale : 1.0 / (double)D; /* mistake: 1/d */
#else
    const double scale = s->sm_scale > 0 ? s->sm_scale : 1.0 / sqrt((double)D);
#endif
    const int64_t NT = L + S;
    int failed = 0;
    if (n_threads < 1) n_threads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int task = 0; task < N * HK; ++task) {
        const int a = task / HK, k = task % HK;
        /* Skip tasks with no selected row. */
        int any = 0;
        for (int t = 0; t < QL && !any; ++t)
            for (int hh = 0; hh < g && !any; ++hh) {
#if ORACLE_MUTANT == 4
                int h = hh * HK + k; /* mistake: strided GQA mapping */
#else
                int h = k * g + hh;
#endif
                if (!row_mask || row_mask[((int64_t)a * QL + t) * HQ + h]) any = 1;
            }
        if (!any) continue;

        double *K = (double *)malloc(sizeof(double) * (size_t)(NT * D));
        double *V = (double *)malloc(sizeof(double) * (size_t)(NT * D));
        double *sc = (double *)malloc(sizeof(double) * (size_t)NT);
        double *qv = (double *)malloc(sizeof(double) * (size_t)D);
        double *ov = (double *)malloc(sizeof(double) * (size_t)D);
        if (!K || !V || !sc || !qv || !ov) {
            free(K); free(V); free(sc); free(qv); free(ov);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        const int lr = s->shared_lr ? 0 : a;
        /* Steps 1-2: gather and materialise the agent's keys and values. */
        for (int64_t j = 0; j < L; ++j) {
            for (int dd = 0; dd < D; ++dd) {
                double kk = ld(in->k_base, base_index(s, in->block_table, j, k, dd), el);
                double vv = ld(in->v_base, base_index(s, in->block_table, j, k, dd), el);
                double dk = 0.0, dv = 0.0;
                for (int i = 0; i < R; ++i) {
#if ORACLE_MUTANT == 5
                    int64_t bidx = ((int64_t)a * R + i) * (HK * D) + (int64_t)dd * HK + k; /* mistake: transposed head/column */
#else
                    int64_t bidx = ((int64_t)a * R + i) * (HK * D) + (int64_t)k * D + dd;
#endif
                    dk += ld(in->lk, ((int64_t)lr * L + j) * R + i, el) * ld(in->bk, bidx, el);
                    dv += ld(in->lv, ((int64_t)lr * L + j) * R + i, el) * ld(in->bv, bidx, el);
                }
#if ORACLE_MUTANT == 1
                dk = 0.0; /* mistake: score residual dropped */
#elif ORACLE_MUTANT == 2
                dv = 0.0; /* mistake: value residual dropped */
#elif ORACLE_MUTANT == 3
                dk = -dk; /* mistake: wrong sign */
#endif
                K[j * D + dd] = kk + dk;
                V[j * D + dd] = vv + dv;
            }
        }
        /* Step 3: the agent's private tokens. */
        for (int64_t j = 0; j < S; ++j)
            for (int dd = 0; dd < D; ++dd) {
                int64_t idx = (((int64_t)a * HK + k) * S + j) * D + dd;
                K[(L + j) * D + dd] = ld(in->k_priv, idx, el);
                V[(L + j) * D + dd] = ld(in->v_priv, idx, el);
            }
        /* Steps 4-6 for every selected row of this (agent, KV head). */
        for (int t = 0; t < QL; ++t) {
            for (int hh = 0; hh < g; ++hh) {
#if ORACLE_MUTANT == 4
                const int h = hh * HK + k;
#else
                const int h = k * g + hh;
#endif
                const int64_t row = ((int64_t)a * QL + t) * HQ + h;
                if (row_mask && !row_mask[row]) continue;
#if ORACLE_MUTANT == 7
                const int64_t nk = s->causal ? L + t + 2 > NT ? NT : L + t + 2 : NT; /* mistake: sees the next token */
#else
                const int64_t nk = s->causal ? L + t + 1 : NT;
#endif
                for (int dd = 0; dd < D; ++dd) qv[dd] = ld(in->q, row * D + dd, el);
                double mx = -INFINITY;
                for (int64_t j = 0; j < nk; ++j) {
                    double dot = 0.0;
                    for (int dd = 0; dd < D; ++dd) dot += qv[dd] * K[j * D + dd];
                    sc[j] = scale * dot;
                    if (sc[j] > mx) mx = sc[j];
                }
                double sum = 0.0;
                for (int64_t j = 0; j < nk; ++j) {
                    sc[j] = exp(sc[j] - mx); /* unnormalised weight */
                    sum += sc[j];
                }
                /* o[dd] = sum_j p_j V[j][dd], each sum taken over j in order (the
                 * j loop outside walks V row by row) */
                for (int dd = 0; dd < D; ++dd) ov[dd] = 0.0;
                for (int64_t j = 0; j < nk; ++j)
                    for (int dd = 0; dd < D; ++dd) ov[dd] += sc[j] * V[j * D + dd];
                for (int dd = 0; dd < D; ++dd) out[row * D + dd] = ov[dd] / sum;
#if ORACLE_MUTANT == 9
                if (lse) lse[row] = log(sum); /* mistake: max term missing */
#else
                if (lse) lse[row] = mx + log(sum);
#endif
            }
        }
        free(K);
        free(V);
        free(sc);
        free(qv);
        free(ov);
    }
    return failed ? -2 : 0;
}
