/*
 * e0.h — C ABI of the MI355X (gfx950) routed-expert int4 SwiGLU hot path.
 *
 * The method is the one of "The Other Half of the Memory Wall: Serving 35B
 * MoEs from SSD with Trained Routing Prediction" (arXiv 2609.18063), as four
 * web pages describe it (cited below by site):
 *   koala.ai.kr walkthrough, discuss.pytorch.kr summary of the project README,
 *   jaehun.me review (cites the report's sections), xyznot.com summary.
 *
 * Five calls cover the path: e0_route, e0_prerouter, e0_moe_staged_decode,
 * e0_moe_sorted_prefill, e0_slot_update.
 *
 * Common rules
 *  - Ownership: the caller allocates and owns every buffer (inputs, outputs,
 *    workspace, the device error word) and every stream. The library never
 *    allocates, frees or synchronises; it keeps no state between calls
 *    (except e0_moe_staged_decode_noalloc's fixed workspace array and its
 *    per-device address).
 *  - A workspace serves one call at a time: calls that may be in flight
 *    together (on different streams) need separate workspaces.
 *  - Pointers named "device" must point to device (HBM) memory; structs and
 *    sizes are read on the host during the call only.
 *  - Every call validates its arguments on the host first. On any error it
 *    returns a nonzero e0_status and enqueues nothing. On success the work is
 *    only enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *    null stream) and the call returns without waiting.
 *  - Data errors found on the device (a routed id out of range, an id that is
 *    not resident in the slot table, no free slot) OR a bit into *dev_err
 *    (E0_DEV_*); the offending contribution is skipped and nothing is read
 *    or written out of bounds. dev_err is never cleared by the library.
 *  - fp16 tensors are IEEE binary16 bit patterns (uint16_t).
 *  - int4 group-64 matrix W[rows][cols] (koala.ai.kr "two tiers" table: int4
 *    affine g64; discuss.pytorch.kr streaming section: 4-bit affine, group
 *    size 64): codes q as uint32 words [rows][cols/8], code c of a row at bits
 *    4*(c%8) of word c/8; scales s and biases b fp16, stored in tiles of 8
 *    rows as [rows/8][cols/64][8] (the scale of row r, group g at element
 *    ((r/8)*(cols/64) + g)*8 + r%8: a tile's 8 rows of one group are 16
 *    contiguous bytes, and the tile's groups follow each other);
 *    W[r][c] = s(r, c/64) * q + b(r, c/64). Groups run along the input
 *    (reduction) dimension. gate and up are [d_ff][d_model], down is
 *    [d_model][d_ff].
 */
#ifndef E0_H
#define E0_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define E0_ABI_VERSION 1

typedef int32_t e0_status;
enum {
    E0_OK = 0,
    E0_ERR_INVALID_ARG = 1,       /* null pointer, negative size, bad mode */
    E0_ERR_UNSUPPORTED_SHAPE = 2, /* d or f not a multiple of 64, K > E, groups that do not divide E, ... */
    E0_ERR_CAPACITY = 3,          /* workspace too small, S too small, size over a kernel limit */
    E0_ERR_HIP = 4                /* a HIP launch of this call failed (hipGetLastError; a status left
                                     pending by the caller's earlier runtime calls is cleared on entry) */
};

/* Bits of the device error word. */
enum {
    E0_DEV_BAD_ID = 1,       /* routed id < 0 or >= E */
    E0_DEV_NOT_RESIDENT = 2, /* routed id has no slot in the slot table */
    E0_DEV_NO_SLOT = 4,      /* slot update found no free slot for a missing expert */
    E0_DEV_SYNC_TIMEOUT = 8  /* an in-launch wait between workgroups expired (outputs invalid) */
};

/* Routing math (jaehun.me review, report Appx. A; the same math routes both
 * the layer's own router logits and the prerouter's predicted logits,
 * koala.ai.kr prerouter section):
 *  mode 0, softmax-top-K: g = softmax(l); inds = top-k(g, K); w = g[inds] / sum g[inds].
 *  mode 1, sigmoid-group: sigma = sigmoid(l); keep the top `topk_groups` of
 *    `n_groups` contiguous groups of E/n_groups experts, each scored by the
 *    sum of its two largest sigma; inds = top-k(sigma over kept experts, K);
 *    w = scale * sigma[inds] / (sum sigma[inds] + eps).
 * Indices come out in descending score, ties to the lower id. */
typedef struct {
    int32_t mode;
    int32_t k;
    int32_t n_groups;    /* mode 1 only */
    int32_t topk_groups; /* mode 1 only */
    float scale;         /* mode 1 only */
    float eps;           /* mode 1 only */
} e0_route_params;

/* Shape of an expert FFN. */
typedef struct {
    int32_t d_model; /* multiple of 64, <= 8192 */
    int32_t d_ff;    /* multiple of 64, <= 4096 */
    int32_t n_experts;
    int32_t top_k;
} e0_moe_dims;

/* One of the nine per-layer stacked tensors ({gate, up, down} x {q, s, b};
 * jaehun.me report 3.1: nine stacked tensors per layer). Slot i of layer l
 * starts at ptr + l * layer_stride + i * slot_stride (bytes). A
 * bundle-contiguous layout (all nine parts of one expert adjacent) and nine
 * separate stacked tensors are both expressible. */
typedef struct {
    const void *ptr;
    int64_t slot_stride;
    int64_t layer_stride;
} e0_part;

/* Index: part[3 * matrix + kind], matrix 0 gate, 1 up, 2 down; kind 0 q, 1 s, 2 b. */
typedef struct {
    e0_part part[9];
} e0_stack;

/* Shared expert with an unmerged low-rank delta on each projection
 * (xyznot.com adapter execution: y = W_int4 x + (alpha/r) B A x; LoRA sits on
 * the shared-expert projections and not on the routed experts: koala.ai.kr
 * training phase 2). Slot 0 of `w` is the layer's shared expert (slot_stride
 * unused). lora_a[p]: fp16 [r][in_p]; lora_b[p]: fp16 [out_p][r]; p = 0 gate,
 * 1 up, 2 down; each with a per-layer stride in bytes. lora_rank 0 = no delta.
 * The shared expert's output is added to the routed combine with weight 1. */
typedef struct {
    e0_stack w;
    int32_t d_ff;
    int32_t lora_rank; /* 0 or 1..32 */
    float lora_scale;  /* alpha / r */
    int32_t pad_;
    const uint16_t *lora_a[3];
    int64_t lora_a_layer_stride[3];
    const uint16_t *lora_b[3];
    int64_t lora_b_layer_stride[3];
} e0_shared;

/* Prerouter heads, one per staged layer, each an fp16 tensor at ptr + j *
 * stride (bytes) for head j (xyznot.com head architecture; jaehun.me report
 * 3.2). fc1_w [hidden][d + 2E], fc1_b [hidden] (nullable), fc2_w [E][hidden],
 * fc2_b [E] (nullable), lin_w [E][d] (the linear residual, warm-started from
 * the next layer's router). */
typedef struct {
    const uint16_t *fc1_w;
    int64_t fc1_w_stride;
    const uint16_t *fc1_b;
    int64_t fc1_b_stride;
    const uint16_t *fc2_w;
    int64_t fc2_w_stride;
    const uint16_t *fc2_b;
    int64_t fc2_b_stride;
    const uint16_t *lin_w;
    int64_t lin_w_stride;
    int32_t hidden; /* fc1 output width; multiple of 64, <= 2048 */
    int32_t pad_;
} e0_prerouter_heads;

int32_t e0_abi_version(void);
const char *e0_status_string(e0_status s);

/* Operation ids for e0_workspace_bytes. */
enum {
    E0_OP_ROUTE = 0,
    E0_OP_PREROUTER = 1,
    E0_OP_STAGED_DECODE = 2,
    E0_OP_SORTED_PREFILL = 3,
    E0_OP_SLOT_UPDATE = 4,
    E0_OP_CHAINED_DECODE = 5
};

/* Workspace bytes the call `op` needs. n = layers (decode, chained decode, slot update),
 * tokens (prefill, route) or heads (prerouter); b = tokens per layer (decode,
 * slot update, prerouter), ignored otherwise; s = slots per layer (slot
 * update) or the shared expert's LoRA rank (decode; 0 = no LoRA), ignored
 * otherwise. For the prerouter, dims->d_ff is the head's hidden width. E0_OP_ROUTE
 * needs no workspace (0). Returns 0 for an invalid request. */
size_t e0_workspace_bytes(int32_t op, const e0_moe_dims *dims, int32_t n, int32_t b, int32_t s);

/*
 * e0_route — routing for n_layers x T tokens.
 *  logits:     device [L][T][E], fp16 if logits_fp16 else fp32; or NULL, then
 *              logits[l][t][e] = x[l][t] . w_router[l][e] (the layer's own
 *              router, computed in fp32 from fp16 x [L][T][d] and fp16
 *              w_router [L][E][d]; d a multiple of 64, <= 8192).
 *  idx, w:     device outputs int32 / fp32 [L][T][K].
 *  logits_out: device fp32 [L][T][E], the logits routed on; required when
 *              logits is NULL (the router writes there), optional otherwise.
 *  Limits: E <= 1024, K <= 32, K <= E; mode 1: E % n_groups == 0,
 *  n_groups <= 64, K <= topk_groups * E / n_groups.
 */
e0_status e0_route(const e0_route_params *p, int32_t n_layers, int32_t T, int32_t E, const void *logits,
                   int32_t logits_fp16, const uint16_t *x, const uint16_t *w_router, int32_t d, int32_t *idx,
                   float *w, float *logits_out, void *stream);

/*
 * e0_prerouter — every head of a step in one call (the one-token lead lets
 * all staged layers be predicted in a single flush per step: koala.ai.kr
 * prerouter section; jaehun.me report 3.2). Head j at token b reads
 *   x = [ h[j][b] (d) | K-hot(cur_idx[j][b]) (E) | K-hot(prev_idx[j][b]) (E) ],
 *   o = fc2 gelu_erf(fc1 x + fc1_b) + fc2_b + lin_w h,
 * and routes o with `p` (prediction-as-routing: the prediction is the
 * routing, koala.ai.kr and xyznot.com). A K-hot vector has a 1 at each id of
 * the row; ids < 0 are skipped; prev_idx NULL means no previous token.
 *  h: device fp16 [n_heads][B][d]; cur_idx, prev_idx: device int32
 *  [n_heads][B][K]; next_idx, next_w: device [n_heads][B][K]; logits_out:
 *  optional device fp32 [n_heads][B][E].
 *  ws: device workspace of e0_workspace_bytes(E0_OP_PREROUTER, dims, n_heads, B, 0)
 *  bytes (dims: d_model = d, n_experts = E, top_k = p->k; d_ff = heads->hidden).
 *  Limits: B <= 64, d multiple of 64 and <= 8192, E <= 1024.
 */
e0_status e0_prerouter(const e0_prerouter_heads *heads, int32_t n_heads, int32_t B, int32_t d, int32_t E,
                       const uint16_t *h, const int32_t *cur_idx, const int32_t *prev_idx,
                       const e0_route_params *p, int32_t *next_idx, float *next_w, float *logits_out, void *ws,
                       size_t ws_bytes, void *stream);

/*
 * e0_moe_staged_decode — the staged path (koala.ai.kr paths table; jaehun.me
 * report 3.1) over L independent layers of B tokens each:
 *   y[l][t] = sum_k w[l][t][k] * down(silu(gate(x)) * up(x)) of expert
 *             idx[l][t][k], whose weights are read from slot
 *             slot_of[l][idx] of the pool (the slot table keeps routing ids
 *             on the GPU), plus the shared expert if `shared` is not NULL.
 * Experts are deduplicated per layer: each routed expert's weights are read
 * once per call and applied to all of its tokens.
 *  x: device fp16 [L][B][d]; idx, w: device [L][B][K]; slot_of: device int32
 *  [L][E]; pool: S slots per layer; y: device fp32 [L][B][d] (overwritten).
 *  ws: device workspace, e0_workspace_bytes(E0_OP_STAGED_DECODE, dims, L, B, r),
 *  r the shared expert's LoRA rank (0 without shared expert or LoRA).
 *  dev_err: device int32, OR-ed with E0_DEV_BAD_ID / E0_DEV_NOT_RESIDENT.
 *  Limits: B <= 64, K <= 32.
 *  Numeric range: x is taken as fp16 and half of its values are scaled by
 *  1/16 in fp16 inside the kernels (the nibble dot product), so inputs below
 *  2^-10 in magnitude lose relative precision as fp16 subnormals; at B > 1
 *  the hidden h = silu(gate x) * up x of each (expert, token) is carried as
 *  an fp16 high/low pair, so |h| must stay below 65504. Inputs of unit scale
 *  (the synthetic N(0,1) activations) are far from both limits.
 *  Concurrency: the workspace belongs to one call at a time. Calls that may
 *  run concurrently (different streams) need separate workspaces; at B = 1
 *  the single-launch kernel keeps its in-launch hand-off flags and h blocks
 *  there, tagged with a per-call epoch.
 */
e0_status e0_moe_staged_decode(const e0_moe_dims *dims, int32_t L, int32_t B, const uint16_t *x,
                               const int32_t *idx, const float *w, const int32_t *slot_of, int32_t S,
                               const e0_stack *pool, const e0_shared *shared, float *y, void *ws, size_t ws_bytes,
                               int32_t *dev_err, void *stream);

/*
 * e0_moe_staged_decode_noalloc — e0_moe_staged_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, kernels and results as
 * e0_moe_staged_decode, without ws / ws_bytes: the workspace is a fixed device
 * array of E0_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU,
 * held until the process ends. The call allocates nothing.
 *  Sizes whose workspace (e0_workspace_bytes(E0_OP_STAGED_DECODE, ...)) is
 *  larger than the array return E0_ERR_CAPACITY before anything is enqueued.
 *  The first call on a device looks up the array's address on that device
 *  (hipGetSymbolAddress; a failure returns E0_ERR_HIP); later calls reuse it.
 *  All calls on one GPU share the array: calls that may run at the same time
 *  on one GPU (other streams, other host threads) race and must not overlap.
 */
#define E0_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
e0_status e0_moe_staged_decode_noalloc(const e0_moe_dims *dims, int32_t L, int32_t B, const uint16_t *x,
                                       const int32_t *idx, const float *w, const int32_t *slot_of, int32_t S,
                                       const e0_stack *pool, const e0_shared *shared, float *y, int32_t *dev_err,
                                       void *stream);

/*
 * e0_moe_sorted_prefill — the whole-layer path (jaehun.me report 3.1;
 * discuss.pytorch.kr paths table: a layer's experts all resident, then a
 * sorted gather): the T*K (token, k) pairs are grouped by expert (the order
 * of the rows inside an expert's group is unspecified; no result depends on
 * it: repeated calls on the same inputs give the same bytes), each active
 * expert runs as one grouped GEMM over its rows (matrix cores; fp16 operands,
 * the dequantised weight rounded to fp16 once, fp32 accumulation; an expert
 * with at most 16 rows multiplies the codes themselves and applies its scales
 * and biases in fp32), and the weighted results are summed back per token in
 * k order:
 *   y[t] = sum_k w[t][k] * down(silu(gate(x_t)) * up(x_t)) of expert idx[t][k].
 *  x: device fp16 [T][d]; idx, w: device [T][K]; layer: slot e = expert e
 *  (layer_stride unused); y: device fp32 [T][d] (overwritten).
 *  ws: device workspace, e0_workspace_bytes(E0_OP_SORTED_PREFILL, dims, T, 0, 0).
 *  dev_err: device int32, OR-ed with E0_DEV_BAD_ID.
 *  Limits: d_model, d_ff multiples of 128; E <= 1024; K <= 32; T*K <= 2^24.
 */
e0_status e0_moe_sorted_prefill(const e0_moe_dims *dims, int32_t T, const uint16_t *x, const int32_t *idx,
                                const float *w, const e0_stack *layer, float *y, void *ws, size_t ws_bytes,
                                int32_t *dev_err, void *stream);

/*
 * e0_slot_update — fixed double-buffered slots updated in place for changed
 * experts only (koala.ai.kr paths table, "staged"; Appx. B incr_stack;
 * xyznot.com glossary "incremental sticky-slot stack"). Per layer l:
 *   U' = ids in next_idx[l] (the set the next step routes to),
 *   U  = ids in cur_idx[l] (in use by the step in flight; NULL = none).
 *   An expert of U' already resident stays where it is. Each missing expert
 *   of U', in ascending id, takes the lowest-index slot whose occupant is in
 *   neither U' nor U (or is empty); its nine parts are copied there from the
 *   store, expert_of[l][slot] and slot_of[l][id] are set and the evicted
 *   expert's slot_of entry becomes -1. With S >= 2 * (max distinct ids per
 *   step) a free slot always exists and no slot read by the step in flight is
 *   written, so this may run on a side stream concurrently with that step.
 *  next_idx, cur_idx: device int32 [L][B][K]; slot_of: device [L][E];
 *  expert_of: device [L][S] (-1 = empty); store: slot e = expert e, in device
 *  memory or in pinned host memory mapped for the device (hipHostMalloc; the
 *  copy then reads it over the host link: the store outside HBM with the pool
 *  as its cache, the pages' own setting with the SSD replaced by host DRAM);
 *  each part's address is resolved with hipPointerGetAttributes and a part the
 *  device cannot reach fails the call with E0_ERR_INVALID_ARG before anything
 *  is enqueued; pool: S slots in device memory. n_copied: optional device
 *  int32 [L], experts copied per layer.
 *  ws: device workspace, e0_workspace_bytes(E0_OP_SLOT_UPDATE, dims, L, B, S).
 *  dev_err: OR-ed with E0_DEV_BAD_ID, E0_DEV_NO_SLOT (then the experts that
 *  found a slot are still placed, the others are not).
 *  Limits: E <= 4096, S <= 4096, B*K <= 4096.
 */
e0_status e0_slot_update(const e0_moe_dims *dims, int32_t L, int32_t B, int32_t S, const int32_t *next_idx,
                         const int32_t *cur_idx, int32_t *slot_of, int32_t *expert_of, const e0_stack *store,
                         const e0_stack *pool, int32_t *n_copied, void *ws, size_t ws_bytes, int32_t *dev_err,
                         void *stream);

/*
 * e0_slot_update_lru — e0_slot_update with the pool kept as a per-layer
 * least-recently-used hot set of the store: an HBM budget of S slots per
 * layer, larger than one step needs and smaller than the store, that keeps
 * the experts used most recently (koala.ai.kr on the hot path of resident
 * experts; jaehun.me review, report 3.2 on whole-layer residency). Same
 * arguments and limits as e0_slot_update, plus:
 *  last_use: device int32 [L][S], the last step at which each slot's expert
 *  was wanted (-1 = never; initialise to -1 with the tables); step: this
 *  update's step number, >= 0, increasing from call to call.
 * Rule per layer: every expert of U' already resident stays and its slot's
 * last_use becomes `step` (a hit); the i-th missing expert of U' in
 * ascending id takes the i-th candidate slot (empty, or holding an expert in
 * neither U' nor U) in ascending (last_use, slot) order, and that slot's
 * last_use becomes `step` (a miss: the expert least recently used is
 * evicted). Every wanted expert is resident afterwards, so the decode stays
 * exact; only the copy count depends on the policy. n_copied counts the
 * misses. Errors as e0_slot_update; E0_ERR_INVALID_ARG also for a null
 * last_use or a negative step.
 */
e0_status e0_slot_update_lru(const e0_moe_dims *dims, int32_t L, int32_t B, int32_t S, const int32_t *next_idx,
                             const int32_t *cur_idx, int32_t *slot_of, int32_t *expert_of, int32_t *last_use,
                             int32_t step, const e0_stack *store, const e0_stack *pool, int32_t *n_copied, void *ws,
                             size_t ws_bytes, int32_t *dev_err, void *stream);

/*
 * e0_moe_chained_decode — one token through L stacked layers in one call, the
 * input of each layer computed from the output of the one before (the pages
 * stage the next layers' experts ahead so that their weight reads overlap the
 * current layer's compute: koala.ai.kr Fig. 1 and its timeline; the
 * dependency that forces it, layer l+1's experts known only from layer l's
 * output, is stated in the same page's problem section). A layer here is norm
 * + routed experts + residual (attention is outside this path):
 *   x_l = fp16( r_l / sqrt(mean_i r_l[i]^2 + eps) * g_l ),   r_0 = r_in,
 *   y_l = sum_k w[l][k] * down(silu(gate(x_l)) * up(x_l)) of expert idx[l][k]
 *         read through slot_of[l] from the pool (as e0_moe_staged_decode),
 *   r_{l+1} = r_l + y_l.
 * The routing of every layer is given up front (the staged prediction). The
 * weights of later layers are requested while earlier layers compute.
 *  r_in: device fp32 [d]; norm_w: device fp16 [L][d] (g_l); eps >= 0;
 *  idx, w: device [L][K]; slot_of: device int32 [L][E]; pool: S slots per
 *  layer; y: device fp32 [L][d], the MoE output of each layer; r_out: device
 *  fp32 [L][d], r_out[l] = r_{l+1} (the last row is the stack's output). All
 *  pointers 16-byte aligned except idx, w, slot_of, y.
 *  ws: device workspace, e0_workspace_bytes(E0_OP_CHAINED_DECODE, dims, L, 0, 0)
 *  (0 when the shape is unsupported).
 *  dev_err: device int32, OR-ed with E0_DEV_BAD_ID / E0_DEV_NOT_RESIDENT (that
 *  expert's contribution skipped) and E0_DEV_SYNC_TIMEOUT (an in-launch wait
 *  of more than 50 ms; results then undefined).
 *  Limits: d_model 2048; d_ff 256, 512 or 1024 (1024 with K <= 4); K <= 8;
 *  E <= 1024. The caller owns every buffer; nothing is allocated or freed.
 */
e0_status e0_moe_chained_decode(const e0_moe_dims *dims, int32_t L, const float *r_in, const uint16_t *norm_w,
                                float eps, const int32_t *idx, const float *w, const int32_t *slot_of, int32_t S,
                                const e0_stack *pool, float *y, float *r_out, void *ws, size_t ws_bytes,
                                int32_t *dev_err, void *stream);

/*
 * e0_lora_merge_requant — a LoRA delta merged into an int4 group-64 matrix and
 * requantised: the alternative the pages weigh against serving the recovery
 * LoRA unmerged (jaehun.me review, the paragraph on not merging, citing the
 * report's section 3.3 and its retention measure 1 - |U - M| / |U - B|;
 * xyznot.com FAQ on why the recovery LoRA stays unmerged: deltas of RMS about
 * 1e-3 sit below one 4-bit step, so requantisation erases most of them).
 * Per row i and column c, in fp32 with every operation rounded to nearest
 * (no fused multiply-add):
 *   w = s[i][g] * q[i][c] + b[i][g]                       (g = c / 64)
 *   t = sum over k = 0 .. r-1, in order, of B[i][k] * A[k][c]
 *   w' = w + alpha_over_r * t
 * then per (row, group), with lo/hi the group's least/largest w':
 *   s' = fp16((hi - lo) / 15),  b' = fp16(lo),
 *   q' = s' == 0 ? 0 : min(15, max(0, round_half_even((w' - b') / s'))).
 * The definition is exact arithmetic; computed in fp32 as above, a code (or
 * an fp16 scale or bias) can differ from the exact one by one step only where
 * the exact value lies within the fp32 rounding error of a rounding flip.
 *  rows, cols: rows % 8 == 0, cols % 64 == 0, rows * cols < 2^31; r in 1 .. 64.
 *  q, q_out: device uint32 [rows][cols/8] (code c at bits 4*(c%8) of word
 *  c/8); s, b, s_out, b_out: device fp16 bit patterns in the stacks' 8-row
 *  tiles ([rows/8][cols/64][8], as in e0_stack); lora_b: device fp16
 *  [rows][r]; lora_a: device fp16 [r][cols]. All pointers 16-byte aligned;
 *  outputs must not overlap the inputs. One launch on `stream`; nothing is
 *  allocated. Errors: E0_ERR_INVALID_ARG / E0_ERR_UNSUPPORTED_SHAPE before
 *  any launch, E0_ERR_HIP on a launch failure.
 */
e0_status e0_lora_merge_requant(int32_t rows, int32_t cols, const uint32_t *q, const uint16_t *s, const uint16_t *b,
                                const uint16_t *lora_b, const uint16_t *lora_a, int32_t r, float alpha_over_r,
                                uint32_t *q_out, uint16_t *s_out, uint16_t *b_out, void *stream);

/*
 * Measurement probes (not part of the method): what this GPU sustains, for
 * roofline fractions against measured as well as published peaks.
 *  e0_probe_stream_read: reads `bytes` (multiple of 16, src 16-byte aligned)
 *    of device memory once with 16-byte streaming loads on 4096 workgroups;
 *    sink: device uint32 (practically never written).
 *  e0_probe_mfma: `blocks` workgroups of four wavefronts, each running `iters`
 *    rounds of eight independent v_mfma_f32_32x32x16_f16; *flop (host, may be
 *    NULL) receives the dense FLOP count of the launch.
 * Both only enqueue on `stream`; E0_ERR_INVALID_ARG on bad arguments.
 */
e0_status e0_probe_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);
e0_status e0_probe_mfma(int32_t blocks, int32_t iters, uint32_t *sink, double *flop, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* E0_H */
