/*
 * route_oracle.c -- plain, slow, obviously-correct CPU reference for MoE
 * routing top-k.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls it and shares no code
 * with it.
 *
 * Everything is computed in double precision, one token row at a time, in the
 * order the pages describe the method.  Sorting uses the C library qsort with
 * an explicit (score desc, index asc) comparator.
 *
 * Sources (web pages; cited by title and section):
 *   [ROUTING]  "[SGLang] MoE routing: token-to-expert assignment algorithms"
 *              (blog.secrett2633.cloud/opensource/sglang/moe-routing)
 *              sections 2 (softmax Top-K), 3 (Grouped Top-K, DeepSeek style),
 *              4 (Biased Grouped Top-K with correction_bias),
 *              5 (Fused MoE Router).
 *   [AITER]    "[sglang] SGLang MoE routing optimisation: using
 *              aiter.biased_grouped_topk on AMD GPUs"
 *              (sglang PR 23611 analysis), section "Code analysis".
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - expert ties are broken by the lower expert index, group ties by the
 *     lower group index;
 *   - the K chosen ids are emitted in (selection score desc, index asc) order;
 *   - experts of dropped groups are not candidates at all (equivalent to a
 *     -inf mask);
 *   - with a correction bias, selection uses sigmoid + bias while the emitted
 *     weight is the unbiased sigmoid score;
 *   - renormalisation divides the K weights by their plain sum.
 *
 * Parity status: every function here is pinned by the CPU tests
 * (hand-worked cases, closed forms, brute force on tiny inputs, invariants,
 * and a library matmul for the router projection).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_F64 2

#define OR_SOFTMAX 0
#define OR_SIGMOID 1

#define OR_GROUP_MAX 0     /* DeepSeek-V2 style: group score = max     */
#define OR_GROUP_TOP2SUM 1 /* DeepSeek-V3 style: sum of the top-2      */

/* Widen one logit to double.  bf16 is the upper half of an IEEE binary32,
 * so putting its 16 bits on top of 16 zero bits gives the exact value. */
static double load_logit(const void* base, int dtype, int64_t i) {
    if (dtype == OR_F32) return (double)((const float*)base)[i];
    if (dtype == OR_F64) return ((const double*)base)[i];
    {
        uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

typedef struct {
    double key;
    int idx;
} keyed_t;

/* Larger key first; equal keys by ascending index. */
static int cmp_desc_then_index(const void* a, const void* b) {
    const keyed_t* x = (const keyed_t*)a;
    const keyed_t* y = (const keyed_t*)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

/*
 * Scores of one row.
 * softmax  ([ROUTING] section 2 and the first line of section 3): the
 *          probability of expert i is exp(x_i - max x) / sum_j exp(x_j - max x),
 *          taken over all E experts.
 * sigmoid  ([ROUTING] section 4; [AITER] sigmoid scoring): 1 / (1 + exp(-x_i)).
 * The selection score adds the per-expert correction bias when one is given
 * ([ROUTING] section 4: scores_for_choice = scores + bias).
 */
int oracle_row_scores(const void* logits, int dtype, int E, const float* bias,
                      int scoring, double* s, double* c) {
    int i;
    if (E <= 0 || (scoring != OR_SOFTMAX && scoring != OR_SIGMOID)) return 1;
    if (scoring == OR_SOFTMAX) {
        double mx = load_logit(logits, dtype, 0), sum = 0.0;
        for (i = 1; i < E; ++i) {
            double x = load_logit(logits, dtype, i);
            if (x > mx) mx = x;
        }
        for (i = 0; i < E; ++i) {
            s[i] = exp(load_logit(logits, dtype, i) - mx);
            sum += s[i];
        }
        for (i = 0; i < E; ++i) s[i] = s[i] / sum;
    } else {
        for (i = 0; i < E; ++i) s[i] = 1.0 / (1.0 + exp(-load_logit(logits, dtype, i)));
    }
    for (i = 0; i < E; ++i) c[i] = s[i] + (bias ? (double)bias[i] : 0.0);
    return 0;
}

/*
 * Group scores of one row.  Groups are contiguous blocks of E/G experts, as
 * the pages' view(num_token, num_expert_group, -1) reshape implies.
 *   max rule     ([ROUTING] section 3): the largest selection score in the group.
 *   top-2 rule   ([ROUTING] section 4): the sum of the two largest selection
 *                scores in the group.
 */
int oracle_group_scores(const double* c, int E, int G, int group_rule, double* h) {
    int g, j, gs;
    keyed_t* tmp;
    if (G <= 0 || E % G != 0) return 1;
    gs = E / G;
    if (group_rule == OR_GROUP_TOP2SUM && gs < 2) return 1;
    tmp = (keyed_t*)malloc(sizeof(keyed_t) * (size_t)gs);
    if (!tmp) return 1;
    for (g = 0; g < G; ++g) {
        for (j = 0; j < gs; ++j) {
            tmp[j].key = c[g * gs + j];
            tmp[j].idx = g * gs + j;
        }
        qsort(tmp, (size_t)gs, sizeof(keyed_t), cmp_desc_then_index);
        h[g] = (group_rule == OR_GROUP_MAX) ? tmp[0].key : tmp[0].key + tmp[1].key;
    }
    free(tmp);
    return 0;
}

/*
 * Route M rows.
 *   1. scores s and selection scores c            (oracle_row_scores)
 *   2. group scores h, then keep the TG groups with the largest h
 *      ([ROUTING] section 3: topk over group scores, then a mask that keeps
 *      only the experts of the chosen groups); G == 1 keeps everything.
 *   3. the K candidates with the largest c, in (c desc, index asc) order
 *      ([ROUTING] section 3: topk over the masked scores).
 *   4. weight k = s of the chosen expert (unbiased, [ROUTING] section 4 says
 *      the bias only steers which experts are chosen); with renormalize the
 *      K weights are divided by their sum ([ROUTING] section 2).
 * Optional diagnostics per row (gaps, may be NULL), three doubles:
 *   gaps[0] = c of the K-th pick minus c of the best unpicked candidate
 *             (+inf when there is no unpicked candidate);
 *   gaps[1] = smallest difference between consecutive picks (+inf if K == 1);
 *   gaps[2] = h of the TG-th kept group minus h of the best dropped group
 *             (+inf when no group is dropped).
 * Returns 0 on success, 1 on an argument the method does not define.
 */
int oracle_route(const void* logits, int dtype, int64_t M, int E, const float* bias,
                 int scoring, int group_rule, int G, int TG, int K, int renormalize,
                 float* weights, int32_t* ids, double* gaps) {
    int64_t m;
    int rc = 0;
    double *s, *c, *h;
    keyed_t *gk, *cand;
    unsigned char* kept;
    size_t esz = (dtype == OR_F32) ? 4 : (dtype == OR_BF16) ? 2 : 8;

    if (M < 0 || E <= 0 || G <= 0 || E % G != 0 || TG < 1 || TG > G || K < 1) return 1;
    if (K > TG * (E / G)) return 1;
    if (dtype != OR_F32 && dtype != OR_BF16 && dtype != OR_F64) return 1;
    if (group_rule != OR_GROUP_MAX && group_rule != OR_GROUP_TOP2SUM) return 1;
    if (G > 1 && group_rule == OR_GROUP_TOP2SUM && E / G < 2) return 1;

    s = (double*)malloc(sizeof(double) * (size_t)E);
    c = (double*)malloc(sizeof(double) * (size_t)E);
    h = (double*)malloc(sizeof(double) * (size_t)G);
    gk = (keyed_t*)malloc(sizeof(keyed_t) * (size_t)G);
    cand = (keyed_t*)malloc(sizeof(keyed_t) * (size_t)E);
    kept = (unsigned char*)malloc((size_t)G);
    if (!s || !c || !h || !gk || !cand || !kept) {
        rc = 1;
        goto done;
    }

    for (m = 0; m < M; ++m) {
        const void* row = (const char*)logits + (size_t)m * (size_t)E * esz;
        int g, i, k, n = 0, gs = E / G;
        double wsum = 0.0;

        if (oracle_row_scores(row, dtype, E, bias, scoring, s, c)) { rc = 1; goto done; }

        /* group selection */
        if (G > 1) {
            if (oracle_group_scores(c, E, G, group_rule, h)) { rc = 1; goto done; }
            for (g = 0; g < G; ++g) { gk[g].key = h[g]; gk[g].idx = g; kept[g] = 0; }
            qsort(gk, (size_t)G, sizeof(keyed_t), cmp_desc_then_index);
            for (g = 0; g < TG; ++g) kept[gk[g].idx] = 1;
        } else {
            kept[0] = 1;
        }

        /* candidates = experts of kept groups, sorted (c desc, index asc) */
        for (i = 0; i < E; ++i) {
            if (!kept[i / gs]) continue;
            cand[n].key = c[i];
            cand[n].idx = i;
            ++n;
        }
        qsort(cand, (size_t)n, sizeof(keyed_t), cmp_desc_then_index);

        for (k = 0; k < K; ++k) wsum += s[cand[k].idx];
        for (k = 0; k < K; ++k) {
            double w = s[cand[k].idx];
            if (renormalize) w = w / wsum;
            weights[m * K + k] = (float)w;
            ids[m * K + k] = (int32_t)cand[k].idx;
        }

        if (gaps) {
            double og = INFINITY;
            gaps[m * 3 + 0] = (n > K) ? cand[K - 1].key - cand[K].key : INFINITY;
            for (k = 0; k + 1 < K; ++k) {
                double d = cand[k].key - cand[k + 1].key;
                if (d < og) og = d;
            }
            gaps[m * 3 + 1] = og;
            gaps[m * 3 + 2] = (G > 1 && TG < G) ? gk[TG - 1].key - gk[TG].key : INFINITY;
        }
    }

done:
    free(s);
    free(c);
    free(h);
    free(gk);
    free(cand);
    free(kept);
    return rc;
}

/*
 * Router projection of the fused router ([ROUTING] section 5): the logit of
 * expert e for token m is the dot product of the token's hidden vector with
 * the expert's router weights, accumulated in high precision.  Both operands
 * are bf16 (raw 16-bit patterns); each product of two bf16 values is exact in
 * double and the sum runs over h in ascending order.  The router weight is
 * stored [H, E] (row h holds the weights of every expert for hidden unit h).
 */
int oracle_router_logits(const uint16_t* hidden, const uint16_t* w, int64_t M, int H,
                         int E, double* logits) {
    int64_t m;
    int e, hh;
    if (M < 0 || H <= 0 || E <= 0) return 1;
    for (m = 0; m < M; ++m) {
        for (e = 0; e < E; ++e) {
            double acc = 0.0;
            for (hh = 0; hh < H; ++hh) {
                double a = load_logit(hidden, OR_BF16, m * (int64_t)H + hh);
                double b = load_logit(w, OR_BF16, (int64_t)hh * E + e);
                acc += a * b;
            }
            logits[m * E + e] = acc;
        }
    }
    return 0;
}

/*
 * Expert-sorted dispatch metadata of a routing result.  The routing page
 * ([ROUTING], section "output format") names a kernel-oriented output made of
 * routing data, a gather index and a scatter index, without defining their
 * fields.  The reading taken here is the plainest one: the M*K (token, slot)
 * assignments, numbered a = m*K + k, are put in order of expert id, and
 * assignments of the same expert keep their order a (a stable counting sort):
 *   counts[e]   number of assignments to expert e;
 *   offsets[e]  where expert e's run starts (exclusive prefix sum of counts;
 *               offsets[E] = number of valid assignments);
 *   gather[p]   the assignment at sorted position p (-1 past offsets[E]);
 *   scatter[a]  the sorted position of assignment a (its inverse), or -1 when
 *               ids[a] is outside [0, E) (such an assignment is dropped);
 *   sorted_w[p] weights[gather[p]] (0 past offsets[E]); weights may be NULL.
 */
int oracle_dispatch(const int32_t* ids, const float* weights, int64_t n, int E,
                    int32_t* counts, int32_t* offsets, int32_t* gather, int32_t* scatter,
                    float* sorted_w) {
    int64_t a, p;
    int e;
    int32_t* cursor;
    if (n < 0 || E <= 0) return 1;
    for (e = 0; e < E; ++e) counts[e] = 0;
    for (a = 0; a < n; ++a)
        if (ids[a] >= 0 && ids[a] < E) counts[ids[a]] += 1;
    offsets[0] = 0;
    for (e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor) return 2;
    for (e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (p = 0; p < n; ++p) {
        gather[p] = -1;
        if (sorted_w) sorted_w[p] = 0.0f;
    }
    for (a = 0; a < n; ++a) {
        const int32_t id = ids[a];
        if (id < 0 || id >= E) {
            scatter[a] = -1;
            continue;
        }
        p = cursor[id]++;
        gather[p] = (int32_t)a;
        scatter[a] = (int32_t)p;
        if (sorted_w) sorted_w[p] = weights ? weights[a] : 0.0f;
    }
    free(cursor);
    return 0;
}

/*
 * Shared-expert slot ([ROUTING] section 6): with fused shared experts the
 * last of a row's K slots is handed to a shared expert.  The page draws its
 * id at random from [E, E + num_shared); here the draw is an input
 * (shared_ids[m]), so that the result is reproducible.  When a routed
 * scaling factor is given (rsf != 0), the slot's weight becomes the sum of
 * the row's other K-1 weights divided by it; otherwise the weight is left as
 * it was.  The other slots are untouched.  Applied in place.
 */
int oracle_fuse_shared_expert(float* weights, int32_t* ids, int64_t M, int K,
                              const int32_t* shared_ids, double rsf) {
    int64_t m;
    int k;
    if (M < 0 || K < 2) return 1;
    for (m = 0; m < M; ++m) {
        ids[m * K + (K - 1)] = shared_ids[m];
        if (rsf != 0.0) {
            double s = 0.0;
            for (k = 0; k < K - 1; ++k) s += (double)weights[m * K + k];
            weights[m * K + (K - 1)] = (float)(s / rsf);
        }
    }
    return 0;
}

/*
 * Ascending id order: each row's K (id, weight) pairs reordered by expert id,
 * lowest first (equal ids keep their slot order).  Routing emits ids in score
 * order; some consumers want them by expert, as the page on MiniMax-M3's
 * decode top-k ("[sglang] MiniMax-M3 ... FP8 Attention GEMM", section 1)
 * orders its block ids.  Applied in place; insertion sort per row.
 */
int oracle_sort_ids(float* weights, int32_t* ids, int64_t M, int K) {
    int64_t m;
    int i, j;
    if (M < 0 || K < 1) return 1;
    for (m = 0; m < M; ++m) {
        float* w = weights + m * K;
        int32_t* d = ids + m * K;
        for (i = 1; i < K; ++i) {
            const int32_t di = d[i];
            const float wi = w[i];
            for (j = i - 1; j >= 0 && d[j] > di; --j) {
                d[j + 1] = d[j];
                w[j + 1] = w[j];
            }
            d[j + 1] = di;
            w[j + 1] = wi;
        }
    }
    return 0;
}

/*
 * Router logit soft-capping ([ROUTING] section 5): with a non-zero cap the
 * fused router replaces each logit l by cap * tanh(l / cap) before scoring
 * (a cap of 0 leaves the logits as they are).  In place, in double.
 */
int oracle_softcap(double* logits, int64_t n, double cap) {
    int64_t i;
    if (n < 0) return 1;
    if (cap == 0.0) return 0;
    for (i = 0; i < n; ++i) logits[i] = cap * tanh(logits[i] / cap);
    return 0;
}
