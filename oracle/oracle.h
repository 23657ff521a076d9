/*
 * CPU oracle for the routed-expert int4 SwiGLU hot path ("The Other Half of
 * the Memory Wall: Serving 35B MoEs from SSD with Trained Routing
 * Prediction", arXiv 2609.18063).
 *
 * TEST INFRASTRUCTURE ONLY. This is a plain, slow, obviously-correct
 * restatement of what the method computes, in double precision. It is used by
 * the test-suite, by the smoke check and by the benchmark's CPU-baseline leg,
 * and by nothing else. It shares no code with the GPU library and includes
 * none of its headers.
 *
 * Conventions of this file (its own, written from the pages):
 *  - fp16 values travel as IEEE binary16 bit patterns (uint16_t).
 *  - An int4 group-64 matrix W[rows][cols] is three arrays: codes q as uint32
 *    words [rows][cols/8] (code c of a row at bits 4*(c%8) of word c/8),
 *    scales s and biases b as fp16 [rows][cols/64]; W[r][c] = s*q + b.
 *  - Expert: gate [f][d], up [f][d], down [d][f].
 *  - Return value of the int-returning calls: 0 ok, nonzero error bits.
 */
#ifndef E0_ORACLE_H
#define E0_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    const uint32_t *q;
    const uint16_t *s;
    const uint16_t *b;
} orc_mat;

typedef struct {
    orc_mat gate, up, down;
} orc_expert;

/* Unmerged low-rank delta on one projection: P'(v) = W v + alpha_over_r * B (A v). */
typedef struct {
    const uint16_t *a; /* fp16 [r][in]  */
    const uint16_t *b; /* fp16 [out][r] */
} orc_lora;

typedef struct {
    const uint16_t *fc1_w; /* fp16 [hid][d + 2E] */
    const uint16_t *fc1_b; /* fp16 [hid] or NULL */
    const uint16_t *fc2_w; /* fp16 [E][hid]      */
    const uint16_t *fc2_b; /* fp16 [E] or NULL   */
    const uint16_t *lin_w; /* fp16 [E][d]        */
} orc_head;

double orc_half(uint16_t h);
void orc_dequant(const orc_mat *m, int rows, int cols, double *out);

/* Router logits (a plain GEMV), rounded to fp32: logits[t][e] = x[t] . Wr[e]. */
void orc_router_logits(const uint16_t *x, const uint16_t *wr, int T, int E, int d, float *logits);

/* Routing. logits fp32 [T][E] -> idx [T][K] (descending score, ties to the
 * lower id) and weights w [T][K] (fp64). */
void orc_softmax_topk(const float *logits, int T, int E, int K, int32_t *idx, double *w);
int orc_sigmoid_group(const float *logits, int T, int E, int K, int n_groups, int topk_groups,
                      double scale, double eps, int32_t *idx, double *w);
/* Smallest score gap that decides any selection of the rows (fp64 scores). */
double orc_softmax_topk_margin(const float *logits, int T, int E, int K);
double orc_sigmoid_group_margin(const float *logits, int T, int E, int K, int n_groups, int topk_groups);

/* One expert's SwiGLU: y[d] = down(silu(gate x) * up x), fp64. */
void orc_expert_ffn(const orc_expert *e, int d, int f, const uint16_t *x, double *y);

/* One MoE layer over T tokens, three orderings. experts/pool: arrays of
 * orc_expert. Output y [T][d] fp64 = sum over k, in k order, of w[t][k] * FFN. */
int orc_moe_exact(const orc_expert *experts, int E, int d, int f, int T, int K, const uint16_t *x,
                  const int32_t *idx, const double *w, double *y);
int orc_moe_staged(const orc_expert *pool, int S, const int32_t *slot_of, int E, int d, int f, int T,
                   int K, const uint16_t *x, const int32_t *idx, const double *w, double *y);
int orc_moe_sorted(const orc_expert *experts, int E, int d, int f, int T, int K, const uint16_t *x,
                   const int32_t *idx, const double *w, double *y, int32_t *perm_out);

/* Slot update of one layer. want[n_want] = next routed ids, keep[n_keep] = ids
 * in use by the in-flight step. Tables are updated in place; copies are listed
 * as (dst slot, expert). Returns 0, or 4 when no slot is free. */
int orc_slot_update(int E, int S, const int32_t *want, int n_want, const int32_t *keep, int n_keep,
                    int32_t *slot_of, int32_t *expert_of, int32_t *copy_slot, int32_t *copy_expert,
                    int32_t *n_copies);

/* Prerouter head feature [h | Khot(cur) | Khot(prev)] (prev may be NULL). */
void orc_head_feature(const uint16_t *h, int d, int E, const int32_t *cur, const int32_t *prev, int K,
                      double *feat);
/* Head logits o[E] = fc2 gelu(fc1 feat + b1) + b2 + lin h (fp64). */
void orc_head_logits(const orc_head *hd, int d, int E, int hid, const uint16_t *h, const int32_t *cur,
                     const int32_t *prev, int K, double *o);

/* Shared expert with unmerged LoRA on gate, up, down. lora may be NULL. */
void orc_shared_lora(const orc_expert *e, const orc_lora *lora /*[3] or NULL*/, int r,
                     double alpha_over_r, int d, int f, const uint16_t *x, double *y);

/* Staged decode over L independent layers with B tokens each, split over
 * n_threads threads by layer. pools: [L][S]; slot_of [L][E]; x [L][B][d];
 * idx, w [L][B][K]; y [L][B][d]. */
int orc_decode_layers(const orc_expert *pools, int S, const int32_t *slot_of, int L, int E, int d, int f,
                      int B, int K, const uint16_t *x, const int32_t *idx, const double *w, double *y,
                      int n_threads);

/* Nearest IEEE binary16 of v, ties to even. */
uint16_t orc_to_half(double v);

/* Chained batch-1 decode: x_l = fp16(r_l / rms(r_l) * g_l), y_l = staged MoE
 * of layer l on x_l, r_{l+1} = r_l + y_l. pools [L][S]; slot_of [L][E];
 * r0 [d]; g fp16 [L][d]; idx, w [L][K]; y, r_out [L][d]. */
int orc_chain_decode(const orc_expert *pools, int S, const int32_t *slot_of, int L, int E, int d, int f, int K,
                     const double *r0, const uint16_t *g, double eps, const int32_t *idx, const double *w,
                     double *y, double *r_out);

#ifdef __cplusplus
}
#endif
#endif
