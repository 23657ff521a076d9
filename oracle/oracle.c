/*
 * CPU oracle for the routed-expert int4 SwiGLU hot path of "The Other Half of
 * the Memory Wall: Serving 35B MoEs from SSD with Trained Routing Prediction"
 * (arXiv 2609.18063), as the four web pages about it describe it.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg. Plain loops, double precision, no blocking, no
 * fusion. Every function names the passage it restates. Page names used below:
 *   [koala]   koala.ai.kr walkthrough of the report
 *   [pytorch] discuss.pytorch.kr summary of the project README
 *   [jaehun]  jaehun.me review of the report (cites the report's sections)
 *   [xyznot]  xyznot.com summary with the English abstract
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* IEEE binary16 -> double (exact). */
double orc_half(uint16_t h)
{
    int sign = h >> 15, ex = (h >> 10) & 31, man = h & 1023;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man | 1024), ex - 25);
    return sign ? -v : v;
}

/* int4 affine group-64 weight: w = scale * q + bias, one fp16 scale and one
 * fp16 bias per 64 consecutive elements of a row ([koala] "the tiers" table:
 * int4 affine g64; [pytorch] streaming section: 4-bit affine, group size 64). */
static double weight_at(const orc_mat *m, int cols, int r, int c)
{
    uint32_t word = m->q[(size_t)r * (cols / 8) + c / 8];
    int q = (int)((word >> (4 * (c % 8))) & 15u);
    size_t g = (size_t)r * (cols / 64) + c / 64;
    return orc_half(m->s[g]) * (double)q + orc_half(m->b[g]);
}

void orc_dequant(const orc_mat *m, int rows, int cols, double *out)
{
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c)
            out[(size_t)r * cols + c] = weight_at(m, cols, r, c);
}

/* out[rows] = W v, W int4 g64 [rows][cols]. */
static void qmatvec(const orc_mat *m, int rows, int cols, const double *v, double *out)
{
    for (int r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (int c = 0; c < cols; ++c)
            acc += weight_at(m, cols, r, c) * v[c];
        out[r] = acc;
    }
}

/* out[rows] = W v, W fp16 [rows][cols]. */
static void hmatvec(const uint16_t *w, int rows, int cols, const double *v, double *out)
{
    for (int r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (int c = 0; c < cols; ++c)
            acc += orc_half(w[(size_t)r * cols + c]) * v[c];
        out[r] = acc;
    }
}

/* The layer's own gate: one logit per expert, a dot product of the hidden
 * state with that expert's router row ([koala] prediction-as-routing: the
 * MoE layer's "original router"). Rounded to fp32, the precision in which the
 * logits are handed to the routing step. */
void orc_router_logits(const uint16_t *x, const uint16_t *wr, int T, int E, int d, float *logits)
{
    double *xv = malloc(sizeof(double) * d);
    double *o = malloc(sizeof(double) * E);
    for (int t = 0; t < T; ++t) {
        for (int i = 0; i < d; ++i)
            xv[i] = orc_half(x[(size_t)t * d + i]);
        hmatvec(wr, E, d, xv, o);
        for (int e = 0; e < E; ++e)
            logits[(size_t)t * E + e] = (float)o[e];
    }
    free(xv);
    free(o);
}

/* Index of the largest v[i] over i with allowed[i], ties to the lower index. */
static int argmax_masked(const double *v, const unsigned char *allowed, int n)
{
    int best = -1;
    for (int i = 0; i < n; ++i)
        if (allowed[i] && (best < 0 || v[i] > v[best]))
            best = i;
    return best;
}

/* Softmax-top-K, renormalised ([jaehun] routing math, report Appx. A):
 *   g = softmax(l);  inds = top-k(g, K);  w = g[inds] / sum_{inds} g.
 * Softmax is strictly increasing in the logit, so top-k of g is top-k of l;
 * the selection is made on l so that no rounding of g can make a tie that the
 * logits do not have. Indices come out in descending score, ties to the lower
 * expert id. */
void orc_softmax_topk(const float *logits, int T, int E, int K, int32_t *idx, double *w)
{
    double *l = malloc(sizeof(double) * E);
    double *g = malloc(sizeof(double) * E);
    unsigned char *allowed = malloc(E);
    for (int t = 0; t < T; ++t) {
        double mx = -INFINITY, z = 0.0;
        for (int e = 0; e < E; ++e) {
            l[e] = logits[(size_t)t * E + e];
            if (l[e] > mx)
                mx = l[e];
        }
        for (int e = 0; e < E; ++e)
            z += exp(l[e] - mx);
        for (int e = 0; e < E; ++e)
            g[e] = exp(l[e] - mx) / z;
        memset(allowed, 1, E);
        double gs = 0.0;
        for (int k = 0; k < K; ++k) {
            int e = argmax_masked(l, allowed, E);
            allowed[e] = 0;
            idx[(size_t)t * K + k] = e;
            gs += g[e];
        }
        for (int k = 0; k < K; ++k)
            w[(size_t)t * K + k] = g[idx[(size_t)t * K + k]] / gs;
    }
    free(l);
    free(g);
    free(allowed);
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Group scores of one row: sum of the two largest sigmoid scores in each
 * contiguous group of E/n experts, in fp32 (the precision the GPU decides in). */
static void group_scores(const double *l, int E, int n_groups, float *gsc)
{
    int per = E / n_groups;
    for (int gi = 0; gi < n_groups; ++gi) {
        int a = -1, b = -1;
        for (int e = gi * per; e < (gi + 1) * per; ++e) {
            if (a < 0 || l[e] > l[a]) {
                b = a;
                a = e;
            } else if (b < 0 || l[e] > l[b]) {
                b = e;
            }
        }
        float sa = (float)sigmoid(l[a]);
        float sb = per > 1 ? (float)sigmoid(l[b]) : 0.0f;
        gsc[gi] = sa + sb;
    }
}

/* Sigmoid-group routing ([jaehun] routing math, report Appx. A; 8B tier
 * "sigmoid-group(8x4, x2.5)" in the report's Tab. 1):
 *   sigma = sigmoid(l); keep the top-G of the n groups, each scored by the sum
 *   of its two largest sigma; inds = top-k(sigma over kept experts, K);
 *   w = s * sigma[inds] / (sum sigma[inds] + eps).
 * Groups are contiguous blocks of E/n ids. Within a group and among kept
 * experts the order of sigma is the order of l (sigmoid is increasing), so
 * those choices are made on l; group scores are sums of two values and are
 * compared in fp32. */
int orc_sigmoid_group(const float *logits, int T, int E, int K, int n_groups, int topk_groups,
                      double scale, double eps, int32_t *idx, double *w)
{
    if (n_groups <= 0 || E % n_groups || topk_groups > n_groups || K > topk_groups * (E / n_groups))
        return 1;
    double *l = malloc(sizeof(double) * E);
    float *gsc = malloc(sizeof(float) * n_groups);
    double *gd = malloc(sizeof(double) * n_groups);
    unsigned char *gallow = malloc(n_groups), *allowed = malloc(E);
    int per = E / n_groups;
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e)
            l[e] = logits[(size_t)t * E + e];
        group_scores(l, E, n_groups, gsc);
        for (int gi = 0; gi < n_groups; ++gi)
            gd[gi] = gsc[gi];
        memset(gallow, 1, n_groups);
        memset(allowed, 0, E);
        for (int j = 0; j < topk_groups; ++j) {
            int gi = argmax_masked(gd, gallow, n_groups);
            gallow[gi] = 0;
            for (int e = gi * per; e < (gi + 1) * per; ++e)
                allowed[e] = 1;
        }
        double ssum = 0.0;
        for (int k = 0; k < K; ++k) {
            int e = argmax_masked(l, allowed, E);
            allowed[e] = 0;
            idx[(size_t)t * K + k] = e;
            ssum += sigmoid(l[e]);
        }
        for (int k = 0; k < K; ++k)
            w[(size_t)t * K + k] = scale * sigmoid(l[idx[(size_t)t * K + k]]) / (ssum + eps);
    }
    free(l);
    free(gsc);
    free(gd);
    free(gallow);
    free(allowed);
    return 0;
}

static int cmp_desc(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x < y) - (x > y);
}

/* Smallest gap among the K+1 largest logits of any row (the decisions of
 * softmax-top-K: the order of the K selected and the K-th against the next). */
double orc_softmax_topk_margin(const float *logits, int T, int E, int K)
{
    double m = INFINITY;
    double *v = malloc(sizeof(double) * E);
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e)
            v[e] = logits[(size_t)t * E + e];
        qsort(v, E, sizeof(double), cmp_desc);
        int lim = K < E ? K + 1 : K;
        for (int i = 0; i + 1 < lim; ++i)
            if (v[i] - v[i + 1] < m)
                m = v[i] - v[i + 1];
    }
    free(v);
    return m;
}

/* Smallest gap of any decision of sigmoid-group: the G-th group score against
 * the next (fp64 of the fp32 scores), and the K+1 largest logits among the
 * kept experts (order and boundary). */
double orc_sigmoid_group_margin(const float *logits, int T, int E, int K, int n_groups, int topk_groups)
{
    double m = INFINITY;
    int per = E / n_groups;
    double *l = malloc(sizeof(double) * E), *v = malloc(sizeof(double) * E);
    float *gsc = malloc(sizeof(float) * n_groups);
    double *gd = malloc(sizeof(double) * n_groups), *gs = malloc(sizeof(double) * n_groups);
    unsigned char *gallow = malloc(n_groups);
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e)
            l[e] = logits[(size_t)t * E + e];
        group_scores(l, E, n_groups, gsc);
        for (int gi = 0; gi < n_groups; ++gi)
            gs[gi] = gd[gi] = gsc[gi];
        qsort(gs, n_groups, sizeof(double), cmp_desc);
        if (topk_groups < n_groups && gs[topk_groups - 1] - gs[topk_groups] < m)
            m = gs[topk_groups - 1] - gs[topk_groups];
        memset(gallow, 1, n_groups);
        int nv = 0;
        for (int j = 0; j < topk_groups; ++j) {
            int gi = argmax_masked(gd, gallow, n_groups);
            gallow[gi] = 0;
            for (int e = gi * per; e < (gi + 1) * per; ++e)
                v[nv++] = l[e];
        }
        qsort(v, nv, sizeof(double), cmp_desc);
        int lim = K < nv ? K + 1 : K;
        for (int i = 0; i + 1 < lim; ++i)
            if (v[i] - v[i + 1] < m)
                m = v[i] - v[i + 1];
    }
    free(l);
    free(v);
    free(gsc);
    free(gd);
    free(gs);
    free(gallow);
    return m;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* The math contract every execution path shares ([jaehun] report 3.1;
 * [koala] execution paths): down(silu(gate(x)) * up(x)). */
void orc_expert_ffn(const orc_expert *e, int d, int f, const uint16_t *x, double *y)
{
    double *xv = malloc(sizeof(double) * d);
    double *g = malloc(sizeof(double) * f), *u = malloc(sizeof(double) * f), *h = malloc(sizeof(double) * f);
    for (int i = 0; i < d; ++i)
        xv[i] = orc_half(x[i]);
    qmatvec(&e->gate, f, d, xv, g);
    qmatvec(&e->up, f, d, xv, u);
    for (int i = 0; i < f; ++i)
        h[i] = silu(g[i]) * u[i];
    qmatvec(&e->down, d, f, h, y);
    free(xv);
    free(g);
    free(u);
    free(h);
}

/* Weighted contribution of pair (t, k) into contrib[(t*K + k)*d ..]. */
static void pair_contrib(const orc_expert *e, int d, int f, const uint16_t *x, double wk, double *out)
{
    orc_expert_ffn(e, d, f, x, out);
    for (int i = 0; i < d; ++i)
        out[i] *= wk;
}

/* y[t] = sum over k = 0..K-1, in that order, of contrib[t][k]. */
static void sum_in_k_order(const double *contrib, int T, int K, int d, double *y)
{
    for (int t = 0; t < T; ++t)
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += contrib[((size_t)t * K + k) * d + i];
            y[(size_t)t * d + i] = acc;
        }
}

/* Path "exact" ([jaehun] report 3.1; [koala] paths table): build the
 * deduplicated set of routed experts, then run each on the tokens routed to
 * it. The weighted combine is y_t = sum_k w_tk * FFN_{idx_tk}(x_t). */
int orc_moe_exact(const orc_expert *experts, int E, int d, int f, int T, int K, const uint16_t *x,
                  const int32_t *idx, const double *w, double *y)
{
    int err = 0;
    double *contrib = calloc((size_t)T * K * d, sizeof(double));
    unsigned char *used = calloc(E, 1);
    for (int p = 0; p < T * K; ++p) {
        if (idx[p] < 0 || idx[p] >= E)
            err |= 1;
        else
            used[idx[p]] = 1;
    }
    for (int e = 0; e < E; ++e) {
        if (!used[e])
            continue;
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k)
                if (idx[t * K + k] == e)
                    pair_contrib(&experts[e], d, f, x + (size_t)t * d, w[t * K + k],
                                 contrib + ((size_t)t * K + k) * d);
    }
    sum_in_k_order(contrib, T, K, d, y);
    free(contrib);
    free(used);
    return err;
}

/* Path "staged" ([koala] paths table; [jaehun] report 3.1): routed ids go
 * through the slot table (id -> slot) and the weights are read from the fixed
 * slot pool. An id that is out of range (bit 1) or not resident (bit 2)
 * contributes nothing. */
int orc_moe_staged(const orc_expert *pool, int S, const int32_t *slot_of, int E, int d, int f, int T,
                   int K, const uint16_t *x, const int32_t *idx, const double *w, double *y)
{
    int err = 0;
    double *contrib = calloc((size_t)T * K * d, sizeof(double));
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int e = idx[t * K + k];
            if (e < 0 || e >= E) {
                err |= 1;
                continue;
            }
            int s = slot_of[e];
            if (s < 0 || s >= S) {
                err |= 2;
                continue;
            }
            pair_contrib(&pool[s], d, f, x + (size_t)t * d, w[t * K + k], contrib + ((size_t)t * K + k) * d);
        }
    sum_in_k_order(contrib, T, K, d, y);
    free(contrib);
    return err;
}

/* Path "whole-layer" ([jaehun] report 3.1; [pytorch] paths table: all of a
 * layer's experts loaded, then a sorted gather): count the (t, k) pairs per
 * expert, take the exclusive prefix sum, place the pairs stably by expert,
 * then visit them in that order. perm_out (optional) receives the pair order
 * (t*K + k). */
int orc_moe_sorted(const orc_expert *experts, int E, int d, int f, int T, int K, const uint16_t *x,
                   const int32_t *idx, const double *w, double *y, int32_t *perm_out)
{
    int err = 0, n = T * K;
    int *cnt = calloc(E + 1, sizeof(int)), *pos = calloc(E + 1, sizeof(int));
    int32_t *perm = malloc(sizeof(int32_t) * (n ? n : 1));
    double *contrib = calloc((size_t)n * d, sizeof(double));
    for (int p = 0; p < n; ++p) {
        if (idx[p] < 0 || idx[p] >= E)
            err |= 1;
        else
            cnt[idx[p]]++;
    }
    for (int e = 0, acc = 0; e < E; ++e) {
        pos[e] = acc;
        acc += cnt[e];
    }
    int m = 0;
    for (int p = 0; p < n; ++p)
        if (idx[p] >= 0 && idx[p] < E) {
            perm[pos[idx[p]]++] = p;
            ++m;
        }
    for (int i = 0; i < m; ++i) {
        int p = perm[i], t = p / K;
        pair_contrib(&experts[idx[p]], d, f, x + (size_t)t * d, w[p], contrib + (size_t)p * d);
    }
    sum_in_k_order(contrib, T, K, d, y);
    if (perm_out)
        memcpy(perm_out, perm, sizeof(int32_t) * m);
    free(cnt);
    free(pos);
    free(perm);
    free(contrib);
    return err;
}

static int contains(const int32_t *v, int n, int32_t x)
{
    for (int i = 0; i < n; ++i)
        if (v[i] == x)
            return 1;
    return 0;
}

/* Staged slots, changed experts only ([koala] paths table and Appx. B note:
 * fixed double-buffered slots, incr_stack rewrites only the changed experts in
 * place; [xyznot] glossary "incremental sticky-slot stack"). Rule:
 *  1. an expert of the next set already resident stays where it is;
 *  2. each missing expert, in ascending id, takes the lowest-index slot whose
 *     occupant is in neither the next set nor the in-use set (or is empty);
 *  3. its bytes are copied there and both tables are set, the evicted
 *     expert's entry cleared. */
int orc_slot_update(int E, int S, const int32_t *want, int n_want, const int32_t *keep, int n_keep,
                    int32_t *slot_of, int32_t *expert_of, int32_t *copy_slot, int32_t *copy_expert,
                    int32_t *n_copies)
{
    int nc = 0;
    for (int e = 0; e < E; ++e) {
        if (!contains(want, n_want, e) || slot_of[e] >= 0)
            continue;
        int s = 0;
        for (; s < S; ++s) {
            int o = expert_of[s];
            if (o < 0 || (!contains(want, n_want, o) && !contains(keep, n_keep, o)))
                break;
        }
        if (s == S) {
            *n_copies = nc;
            return 4;
        }
        if (expert_of[s] >= 0)
            slot_of[expert_of[s]] = -1;
        expert_of[s] = e;
        slot_of[e] = s;
        copy_slot[nc] = s;
        copy_expert[nc] = e;
        ++nc;
    }
    *n_copies = nc;
    return 0;
}

/* Head input: the hidden state followed by two top-K one-hot vectors, the
 * owner layer's routing at this token and at the previous token ([xyznot]
 * head architecture: dim = d_model + 2E; [jaehun] report 3.2 toy example:
 * concat(h, one_hot_now, one_hot_prev)). Each one-hot has a 1 at every routed
 * id; a missing previous token gives zeros. */
void orc_head_feature(const uint16_t *h, int d, int E, const int32_t *cur, const int32_t *prev, int K,
                      double *feat)
{
    for (int i = 0; i < d; ++i)
        feat[i] = orc_half(h[i]);
    for (int i = d; i < d + 2 * E; ++i)
        feat[i] = 0.0;
    for (int k = 0; k < K; ++k) {
        if (cur && cur[k] >= 0 && cur[k] < E)
            feat[d + cur[k]] = 1.0;
        if (prev && prev[k] >= 0 && prev[k] < E)
            feat[d + E + prev[k]] = 1.0;
    }
}

static double gelu_erf(double a) { return 0.5 * a * (1.0 + erf(a / sqrt(2.0))); }

/* Prerouter head ([xyznot] head architecture: head(x) = fc2(erf-gelu(fc1(x)))
 * + l(x), l a linear residual warm-started from the next layer's router;
 * [pytorch] prerouter section: fc1, erf-based gelu, fc2, plus linear_init).
 * The residual reads the hidden part of the feature (the next router acts on
 * a hidden state). */
void orc_head_logits(const orc_head *hd, int d, int E, int hid, const uint16_t *h, const int32_t *cur,
                     const int32_t *prev, int K, double *o)
{
    int din = d + 2 * E;
    double *feat = malloc(sizeof(double) * din);
    double *a = malloc(sizeof(double) * hid), *lin = malloc(sizeof(double) * E);
    orc_head_feature(h, d, E, cur, prev, K, feat);
    hmatvec(hd->fc1_w, hid, din, feat, a);
    for (int j = 0; j < hid; ++j)
        a[j] = gelu_erf(a[j] + (hd->fc1_b ? orc_half(hd->fc1_b[j]) : 0.0));
    hmatvec(hd->fc2_w, E, hid, a, o);
    hmatvec(hd->lin_w, E, d, feat, lin);
    for (int e = 0; e < E; ++e)
        o[e] += (hd->fc2_b ? orc_half(hd->fc2_b[e]) : 0.0) + lin[e];
    free(feat);
    free(a);
    free(lin);
}

/* Projection with an unmerged low-rank delta ([xyznot] adapter execution:
 * y = W_int4(x) + (alpha/r) B A x; [jaehun] report 3.3). */
static void proj_lora(const orc_mat *m, const orc_lora *lo, int r, double aor, int rows, int cols,
                      const double *v, double *out)
{
    qmatvec(m, rows, cols, v, out);
    if (!lo)
        return;
    double *av = malloc(sizeof(double) * r), *bav = malloc(sizeof(double) * rows);
    hmatvec(lo->a, r, cols, v, av);
    hmatvec(lo->b, rows, r, av, bav);
    for (int i = 0; i < rows; ++i)
        out[i] += aor * bav[i];
    free(av);
    free(bav);
}

/* Shared expert of a layer: the same SwiGLU contract, each of gate, up and
 * down carrying its own unmerged delta (LoRA sits on the shared-expert
 * projections, not on the routed experts: [koala] training phase 2; [xyznot]
 * student-path SFT). */
void orc_shared_lora(const orc_expert *e, const orc_lora *lora, int r, double alpha_over_r, int d, int f,
                     const uint16_t *x, double *y)
{
    double *xv = malloc(sizeof(double) * d);
    double *g = malloc(sizeof(double) * f), *u = malloc(sizeof(double) * f), *h = malloc(sizeof(double) * f);
    for (int i = 0; i < d; ++i)
        xv[i] = orc_half(x[i]);
    proj_lora(&e->gate, lora ? &lora[0] : NULL, r, alpha_over_r, f, d, xv, g);
    proj_lora(&e->up, lora ? &lora[1] : NULL, r, alpha_over_r, f, d, xv, u);
    for (int i = 0; i < f; ++i)
        h[i] = silu(g[i]) * u[i];
    proj_lora(&e->down, lora ? &lora[2] : NULL, r, alpha_over_r, d, f, h, y);
    free(xv);
    free(g);
    free(u);
    free(h);
}

typedef struct {
    const orc_expert *pools;
    int S;
    const int32_t *slot_of;
    int L, E, d, f, B, K;
    const uint16_t *x;
    const int32_t *idx;
    const double *w;
    double *y;
    int l0, l1, err;
} decode_job;

static void *decode_worker(void *arg)
{
    decode_job *j = arg;
    for (int l = j->l0; l < j->l1; ++l)
        j->err |= orc_moe_staged(j->pools + (size_t)l * j->S, j->S, j->slot_of + (size_t)l * j->E, j->E, j->d,
                                 j->f, j->B, j->K, j->x + (size_t)l * j->B * j->d,
                                 j->idx + (size_t)l * j->B * j->K, j->w + (size_t)l * j->B * j->K,
                                 j->y + (size_t)l * j->B * j->d);
    return NULL;
}

int orc_decode_layers(const orc_expert *pools, int S, const int32_t *slot_of, int L, int E, int d, int f,
                      int B, int K, const uint16_t *x, const int32_t *idx, const double *w, double *y,
                      int n_threads)
{
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > L)
        n_threads = L;
    decode_job *jobs = calloc(n_threads, sizeof(decode_job));
    pthread_t *th = calloc(n_threads, sizeof(pthread_t));
    int err = 0;
    for (int i = 0; i < n_threads; ++i) {
        decode_job j = {pools, S, slot_of, L, E, d, f, B, K, x, idx, w, y, L * i / n_threads,
                        L * (i + 1) / n_threads, 0};
        jobs[i] = j;
        if (n_threads > 1)
            pthread_create(&th[i], NULL, decode_worker, &jobs[i]);
        else
            decode_worker(&jobs[i]);
    }
    for (int i = 0; i < n_threads; ++i) {
        if (n_threads > 1)
            pthread_join(th[i], NULL);
        err |= jobs[i].err;
    }
    free(jobs);
    free(th);
    return err;
}

/* Round a double to the nearest IEEE binary16 value, ties to even (the
 * conversion the fp16 activations of the path go through). Written from the
 * format: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; values
 * below 2^-14 are subnormal multiples of 2^-24; overflow gives infinity. */
uint16_t orc_to_half(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7e00u);
    if (a >= 65520.0) /* 65504 + half an ulp rounds up to infinity */
        return (uint16_t)(sign | 0x7c00u);
    int e;
    frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
    int ex = e - 1; /* a in [2^ex, 2^(ex+1)) */
    if (a == 0.0 || ex < -14)
        ex = -14; /* subnormal range: spacing 2^-24 */
    double ulp = ldexp(1.0, ex - 10);
    double n = a / ulp; /* exact: a scaled by a power of two */
    double r = nearbyint(n); /* current rounding mode: to nearest, ties to even */
    uint32_t units = (uint32_t)r; /* multiples of ulp, at most 2048 */
    uint32_t bits;
    if (units >= 2048) { /* rounded up into the next binade */
        ex += 1;
        units >>= 1;
    }
    if (units < 1024) /* subnormal (only possible at ex == -14) */
        bits = units;
    else
        bits = ((uint32_t)(ex + 15) << 10) | (units - 1024);
    return (uint16_t)(sign | bits);
}

/* Chained batch-1 decode over L layers: the MoE input of layer l is the RMS
 * norm of the residual stream, scaled by the layer's norm weight and rounded
 * to fp16, and the layer's output is added back to the residual:
 *   x_l = fp16( r_l / sqrt(mean(r_l^2) + eps) * g_l ),  y_l = MoE_l(x_l),
 *   r_{l+1} = r_l + y_l.
 * MoE_l is the staged path of layer l (pool layer l, slot_of row l). The
 * pages run one token through the stacked layers with the next layers'
 * weights staged ahead ([koala] Fig. 1 and its timeline); attention is not
 * part of this path, so a layer here is norm + routed experts + residual.
 * pools [L][S]; slot_of [L][E]; r0, g [L][d] (g fp16); idx, w [L][K];
 * y, r_out [L][d] (r_out[l] = r_{l+1}). */
int orc_chain_decode(const orc_expert *pools, int S, const int32_t *slot_of, int L, int E, int d, int f, int K,
                     const double *r0, const uint16_t *g, double eps, const int32_t *idx, const double *w,
                     double *y, double *r_out)
{
    int err = 0;
    double *r = malloc(sizeof(double) * d);
    uint16_t *x = malloc(sizeof(uint16_t) * d);
    for (int i = 0; i < d; ++i)
        r[i] = r0[i];
    for (int l = 0; l < L; ++l) {
        double ss = 0.0;
        for (int i = 0; i < d; ++i)
            ss += r[i] * r[i];
        double inv = 1.0 / sqrt(ss / d + eps);
        for (int i = 0; i < d; ++i)
            x[i] = orc_to_half(r[i] * inv * orc_half(g[(size_t)l * d + i]));
        double *yl = y + (size_t)l * d;
        err |= orc_moe_staged(pools + (size_t)l * S, S, slot_of + (size_t)l * E, E, d, f, 1, K, x,
                              idx + (size_t)l * K, w + (size_t)l * K, yl);
        for (int i = 0; i < d; ++i) {
            r[i] += yl[i];
            r_out[(size_t)l * d + i] = r[i];
        }
    }
    free(r);
    free(x);
    return err;
}
