// Staged decode on gfx950: routed experts read through the slot table from a
// fixed slot pool, int4 group-64 dequantised in registers, gate and up fused
// in one pass, SiLU, down, weighted combine; optional shared expert with an
// unmerged LoRA delta.
//
// Method (arXiv 2609.18063 as described on the pages):
//  - the math contract every path shares: down(silu(gate(x)) * up(x))
//    (jaehun.me review, report 3.1; koala.ai.kr execution paths);
//  - "staged": fixed double-buffered slots, routing ids mapped through a slot
//    table so indices never leave the GPU (koala.ai.kr paths table; jaehun.me
//    report 3.1);
//  - weighted combine over the top-K routed experts (jaehun.me report Appx. A
//    routing weights);
//  - shared expert with the recovery LoRA kept unmerged,
//    y = W_int4 x + (alpha/r) B A x (xyznot.com adapter execution; jaehun.me
//    report 3.3), LoRA on the shared-expert projections only (koala.ai.kr
//    training phase 2).
//
// Kernels (one call = up to four launches on the caller's stream):
//  1. prep   (grid L, B > 1 only): per layer, a stable counting sort of the
//     (token, k) pairs by expert (the deduplicated expert set and each
//     expert's tokens).
//     lora   (shared expert with LoRA only): the down-projections A x, one
//     wavefront per dot product.
//  2. gateup (grid L x experts x row-chunks): each workgroup streams a block
//     of gate and up rows of one expert once and applies them to all of its
//     tokens: h = silu(gate x) * up x, written as fp32.
//  3. down   (grid L x row-chunks): each workgroup owns a block of output
//     rows of one layer and walks the layer's experts in a fixed order,
//     accumulating w * (down h) per token; y is written once, no atomics.
//
// The int4 dot product: each lane holds 32 consecutive inputs of a row (one
// 16-byte load of codes). Codes become fp16 16+q by bit placement
// (exact), and v_dot2_f32_f16 accumulates (16+q) x in fp32; per lane and
// group, s * acc + (b - 16 s) * sum(x) equals sum((s q + b) x). Row sums are
// finished with a register reduce-scatter across the lanes of a row.
#include "e0_internal.h"

#include <math.h>

#include <type_traits>

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxB = 64;
constexpr int kMaxK = 32;
constexpr int kMaxE = 1024;
constexpr int kMaxR = 32;
constexpr int kDownRows = 64;  // output rows per down workgroup
constexpr int kGuGroups = 8;         // row groups streamed per batched gate/up block
constexpr int kHChunkFloats = 4096;  // h floats staged in LDS per chunk of pairs (batched down)

struct DecodeArgs {
    int L, B, K, E, S, d, f;
    const uint16_t *x;
    const int32_t *idx;
    const float *w;
    const int32_t *slot_of;
    Stack pool;
    int has_shared;
    Stack sh;
    int r;
    float lscale;
    const uint16_t *la[3];
    int64_t la_ls[3];
    const uint16_t *lb[3];
    int64_t lb_ls[3];
    float *y;
    int32_t *err;
    int has_plan;
    int umax;
    int32_t *ucnt;   // [L]
    int32_t *uexp;   // [L][umax]
    int32_t *uslot;  // [L][umax]
    int32_t *uoff;   // [L][umax + 1]
    int32_t *pairs;  // [L][B*K]
    int32_t *pslot;  // [L][B*K] slot of the expert of each sorted pair (-1: not resident)
    float *pwt;      // [L][B*K] routing weight of each sorted pair
    float *hbuf;     // [L][B*K + B][f]: B == 1 k order; B > 1 sorted pair order; then the shared expert's
    float *lora_a;   // [L][B][3][r]
    uint32_t *hblk;  // [L][units][d_ff / 32][kBlk] (single-launch batch-1 path)
    // single-launch batch-1 path
    uint64_t *flags;  // [L] lora items, then [L][units][nch] gate/up items
    uint64_t epoch;
    int units;        // K + (shared expert ? 1 : 0)
    int nch;          // h half blocks (flags) per unit: d_ff / 16
    int n_lora;       // lora items (L * lora_parts with LoRA, else 0)
    int lora_parts;   // lora items per layer: 8 of the 2r dot products each
    int n_gu;         // gate/up items per layer (units * d_ff / 64)
    int n_dn;         // down items per layer
    int lag;          // the down items of layer l follow the gate/up items of layer l + lag
    // chained decode (batch 1): the input of layer l is the normed residual,
    // and layer l's down items add its output to the residual
    int chain;
    const float *r_in;       // [d] residual entering layer 0
    float *r_out;            // [L][d] residual after each layer
    const uint16_t *norm_w;  // [L][d] fp16 norm gains
    float norm_eps;
    uint64_t *dflags;        // [L][n_dn] down items of the chain
};

E0_DEV int pairs_per_layer(const DecodeArgs &a) { return a.B * a.K + a.B; }

E0_DEV float *hrow(const DecodeArgs &a, int l, int p) {
    return a.hbuf + ((int64_t)l * pairs_per_layer(a) + p) * a.f;
}

E0_DEV float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of one int per thread (256 threads).
// ---------------------------------------------------------------------------
E0_DEV int block_exclusive_scan(int v, int *lds4, int &total) {
    const int lane = threadIdx.x & 63, wv = wave_id();
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    if (lane == 63) lds4[wv] = inc;
    __syncthreads();
    int base = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        int t = lds4[i];
        if (i < wv) base += t;
        total += t;
    }
    __syncthreads();
    return base + inc - v;
}

// ---------------------------------------------------------------------------
// 1. prep: dedup plan (B > 1); LoRA A x for the shared expert (own kernel).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void decode_prep_kernel(DecodeArgs a) {
    __shared__ int s_cnt[kMaxE];
    __shared__ int s_base[kMaxE];
    __shared__ int s_ids[kMaxB * kMaxK];
    __shared__ int s_slot[kMaxE];
    __shared__ int s_scan[kWaves];
    const int l = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = a.B * a.K;

    if (a.has_plan) {
        for (int e = tid; e < a.E; e += kThreads) s_cnt[e] = 0;
        __syncthreads();
        for (int p = tid; p < n; p += kThreads) {
            int e = a.idx[(int64_t)l * n + p];
            if (e < 0 || e >= a.E) {
                set_err(a.err, E0_DEV_BAD_ID);
                e = -1;
            } else {
                atomicAdd(&s_cnt[e], 1);
            }
            s_ids[p] = e;
        }
        __syncthreads();
        // Each thread owns E/256 consecutive experts (E <= 1024 -> up to 4).
        const int per = (a.E + kThreads - 1) / kThreads;
        const int e0 = tid * per;
        int nu = 0, np = 0;
        for (int e = e0; e < e0 + per && e < a.E; ++e) {
            nu += s_cnt[e] > 0;
            np += s_cnt[e];
        }
        int utot, ptot;
        int ubase = block_exclusive_scan(nu, s_scan, utot);
        int pbase = block_exclusive_scan(np, s_scan, ptot);
        int32_t *uexp = a.uexp + (int64_t)l * a.umax;
        int32_t *uslot = a.uslot + (int64_t)l * a.umax;
        int32_t *uoff = a.uoff + (int64_t)l * (a.umax + 1);
        for (int e = e0; e < e0 + per && e < a.E; ++e) {
            s_base[e] = pbase;
            if (s_cnt[e] > 0) {
                uexp[ubase] = e;
                uoff[ubase] = pbase;
                int s = a.slot_of[(int64_t)l * a.E + e];
                if (s < 0 || s >= a.S) {
                    set_err(a.err, E0_DEV_NOT_RESIDENT);
                    s = -1;
                }
                uslot[ubase] = s;
                s_slot[e] = s;
                ++ubase;
                pbase += s_cnt[e];
            }
        }
        if (tid == 0) {
            a.ucnt[l] = utot;
            uoff[utot] = ptot;
        }
        __syncthreads();
        // Stable placement: a pair's rank among earlier pairs of its expert.
        int32_t *pairs = a.pairs + (int64_t)l * n;
        for (int p = tid; p < n; p += kThreads) {
            const int e = s_ids[p];
            if (e < 0) continue;
            int rank = 0;
            for (int q = 0; q < p; ++q) rank += s_ids[q] == e;
            pairs[s_base[e] + rank] = p;
            a.pslot[(int64_t)l * n + s_base[e] + rank] = s_slot[e];
            a.pwt[(int64_t)l * n + s_base[e] + rank] = a.w[(int64_t)l * n + p];
        }
    }

}

// LoRA down-projections of the shared expert's inputs:
// lora_a[l][t][p][i] = A_p[i] . x_t for gate and up (p = 0, 1); one wavefront
// per dot product, spread over the whole grid.
__global__ __launch_bounds__(kThreads) void decode_lora_kernel(DecodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int job = blockIdx.x * kWaves + wave_id();
    const int per_layer = a.B * 2 * a.r;
    if (job >= a.L * per_layer) return;
    const int l = job / per_layer, rem = job % per_layer;
    const int t = rem / (2 * a.r), p = (rem / a.r) % 2, i = rem % a.r;
    const uint16_t *arow = a.la[p] + (int64_t)l * (a.la_ls[p] / 2) + (int64_t)i * a.d;
    const uint16_t *xt = a.x + ((int64_t)l * a.B + t) * a.d;
    float acc = 0.0f;
    for (int c = lane * 8; c < a.d; c += 512) {
        const u32x4 av = *reinterpret_cast<const u32x4 *>(arow + c);
        const u32x4 xv = *reinterpret_cast<const u32x4 *>(xt + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_fdot2(as_h2(av[j]), as_h2(xv[j]), acc, false);
    }
    acc = wave_sum(acc);
    if (lane == 0) a.lora_a[(((int64_t)l * a.B + t) * 3 + p) * a.r + i] = acc;
}

// Group reduce-scatter over aligned groups of G lanes (G a power of two).
// N values per lane. After: if N >= G, lane holds N/G totals, index
// (lane % G) * (N / G) + j, in v[0 .. N/G); else it holds one total in v[0],
// index (lane % G) / (G / N). Stages are unrolled at compile time (M = the
// lane distance, n = the live value count), so every register index is static.
template <int N, int M, int n>
struct ReduceStage {
    static E0_DEV void run(float (&v)[N], int lane) {
        if constexpr (n == 1) {
            v[0] += __shfl_xor(v[0], M);
        } else {
            constexpr int h = n / 2;
            const bool hi = (lane & M) != 0;
#pragma unroll
            for (int i = 0; i < h; ++i) {
                const float keep = hi ? v[i + h] : v[i];
                const float send = hi ? v[i] : v[i + h];
                v[i] = keep + __shfl_xor(send, M);
            }
        }
        if constexpr (M > 1) ReduceStage<N, M / 2, (n > 1 ? n / 2 : 1)>::run(v, lane);
    }
};

template <int N, int G>
E0_DEV void group_reduce_scatter(float (&v)[N]) {
    if constexpr (G > 1) ReduceStage<N, G / 2, N>::run(v, threadIdx.x & 63);
}

// fp16 pairs (x_j, x_{j+4}) of 8 consecutive fp16 values held as 4 dwords.
E0_DEV void x_pairs(const u32x4 v, uint32_t (&o)[4]) {
    o[0] = __builtin_amdgcn_perm(v[2], v[0], 0x05040100u);
    o[1] = __builtin_amdgcn_perm(v[2], v[0], 0x07060302u);
    o[2] = __builtin_amdgcn_perm(v[3], v[1], 0x05040100u);
    o[3] = __builtin_amdgcn_perm(v[3], v[1], 0x07060302u);
}

// (a & m) | c, selected as one v_and_or_b32. gfx9 VOP3 instructions take at
// most one scalar or literal operand, so the two constants live in VGPRs:
// the callers take them from nibble_consts(), whose values
// the compiler cannot see, which keeps it from splitting the operation.
E0_DEV uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) { return (a & m) | c; }

// Constants of the nibble-to-fp16 placement, kept in VGPRs.
struct NibbleConsts {
    uint32_t mask, one6;
};
E0_DEV NibbleConsts nibble_consts() {
    NibbleConsts k;
    __asm__("v_mov_b32 %0, 0x03c003c0" : "=v"(k.mask));
    __asm__("v_mov_b32 %0, 0x4c004c00" : "=v"(k.one6));
    return k;
}

// sum over the 8 codes of `w` of (16 + q_c) * x_c, x given as pairs
// (x_j, x_{j+4}); code pair (q_j, q_{j+4}) lands at bits 6..9 of each half.
E0_DEV float dot_word(uint32_t w, const uint32_t (&xp)[4], float acc, NibbleConsts k) {
    const uint32_t t0 = and_or(w << 6, k.mask, k.one6);
    const uint32_t t1 = and_or(w << 2, k.mask, k.one6);
    const uint32_t t2 = and_or(w >> 2, k.mask, k.one6);
    const uint32_t t3 = and_or(w >> 6, k.mask, k.one6);
    acc = __builtin_amdgcn_fdot2(as_h2(t0), as_h2(xp[0]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(t1), as_h2(xp[1]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(t2), as_h2(xp[2]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(t3), as_h2(xp[3]), acc, false);
    return acc;
}
E0_DEV float dot_word(uint32_t w, const uint32_t (&xp)[4], float acc) { return dot_word(w, xp, acc, nibble_consts()); }

// Nibbles as fp16 denormals: w & 0x000F000F puts the codes at bits 0..3 of
// each half, which read as fp16 are q * 2^-24; w & 0x00F000F0 (bits 4..7)
// reads as q * 2^-20. v_dot2_f32_f16 takes denormal inputs exactly, so with
// the inputs v of the second kind pre-scaled by 1/16 every product is
// q * v * 2^-24, exact in fp32. One shift, four single-source ANDs (full rate,
// unlike a three-register and-or) and four dot2 per 8 codes.
constexpr float kDenormScale = 16777216.0f;  // 2^24

// Over the 8 codes of `w`: 2^-24 * sum(q_c v_c), v given as the pairs
// (v0, v4), (v1/16, v5/16), (v2, v6), (v3/16, v7/16).
E0_DEV float dot_word_m(uint32_t w, const uint32_t *vp, float acc) {
    const uint32_t w8 = w >> 8;
    acc = __builtin_amdgcn_fdot2(as_h2(w & 0x000F000Fu), as_h2(vp[0]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(w & 0x00F000F0u), as_h2(vp[1]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(w8 & 0x000F000Fu), as_h2(vp[2]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(w8 & 0x00F000F0u), as_h2(vp[3]), acc, false);
    return acc;
}

// The same with v split in two fp16 parts, vh + vl (hi = fp16(v), lo =
// fp16(v - hi)), for fp32 inputs.
E0_DEV float dot_word_m2(uint32_t w, const uint32_t *vh, const uint32_t *vl, float acc) {
    const uint32_t w8 = w >> 8;
    const uint32_t t0 = w & 0x000F000Fu, t1 = w & 0x00F000F0u, t2 = w8 & 0x000F000Fu, t3 = w8 & 0x00F000F0u;
    acc = __builtin_amdgcn_fdot2(as_h2(t0), as_h2(vh[0]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(t0), as_h2(vl[0]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(t1), as_h2(vh[1]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(t1), as_h2(vl[1]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(t2), as_h2(vh[2]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(t2), as_h2(vl[2]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(t3), as_h2(vh[3]), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(t3), as_h2(vl[3]), acc, false);
    return acc;
}

// Pairs (v0, v4), (v1/16, v5/16), (v2, v6), (v3/16, v7/16) of 8 consecutive
// fp16 inputs (4 dwords), and their plain sum.
E0_DEV void x_pairs_m(const u32x4 v, uint32_t (&o)[4], float &sum) {
    x_pairs(v, o);
    const f16x2 k16 = {(f16)0.0625f, (f16)0.0625f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f16x2 hv = as_h2(o[j]);
        sum += (float)hv[0] + (float)hv[1];
        if (j & 1) o[j] = __builtin_bit_cast(uint32_t, hv * k16);
    }
}

// ---------------------------------------------------------------------------
// 2. gateup. Template: LPR lanes per row pass (d = 32 * LPR * NP), TC tokens
// per register chunk, RB rows per lane group per iteration.
// ---------------------------------------------------------------------------
template <int LPR, int NP, int TC, int RB, int G>
__global__ __launch_bounds__(kThreads) void decode_gateup_kernel(DecodeArgs a) {
    constexpr int RPI = kWave / LPR;          // rows per wave instruction
    constexpr int ROWS_W = RPI * RB;          // rows per wave
    constexpr int ROWS_B = ROWS_W * kWaves;   // rows per block
    constexpr int NV = 2 * RB * TC;           // partial values per lane
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int gl = lane % LPR, grp = lane / LPR;
    const int l = blockIdx.x, u = blockIdx.y;
    const bool is_shared = a.has_shared && u == a.umax;

    // Which expert, which slot, which pairs.
    const Stack *st = is_shared ? &a.sh : &a.pool;
    int slot = 0, p_begin = 0, p_count = 0;
    const int32_t *plist = nullptr;
    if (is_shared) {
        p_begin = 0;
        p_count = a.B;
    } else if (a.has_plan) {
        if (u >= a.ucnt[l]) return;
        slot = a.uslot[(int64_t)l * a.umax + u];
        if (slot < 0) return;
        const int32_t *uoff = a.uoff + (int64_t)l * (a.umax + 1);
        p_begin = uoff[u];
        p_count = uoff[u + 1] - p_begin;
        plist = a.pairs + (int64_t)l * a.B * a.K;
    } else {
        // B == 1: expert k of token 0.
        const int e = a.idx[(int64_t)l * a.K + u];
        if (e < 0 || e >= a.E) {
            if (blockIdx.z == 0 && threadIdx.x == 0) set_err(a.err, E0_DEV_BAD_ID);
            return;
        }
        slot = a.slot_of[(int64_t)l * a.E + e];
        if (slot < 0 || slot >= a.S) {
            if (blockIdx.z == 0 && threadIdx.x == 0) set_err(a.err, E0_DEV_NOT_RESIDENT);
            return;
        }
        p_begin = u;
        p_count = 1;
    }
    const int row_base = blockIdx.z * ROWS_B * G + wv * ROWS_W;
    if (row_base >= a.f) return;

    const int d = a.d;
    const int ngrp = d / kGroup;
    rsrc_t qr[2], sr[2], br[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        qr[m] = make_rsrc(part_at(st->p[3 * m + 0], l, slot), (uint32_t)a.f * d / 2);
        sr[m] = make_rsrc(part_at(st->p[3 * m + 1], l, slot), (uint32_t)a.f * ngrp * 2);
        br[m] = make_rsrc(part_at(st->p[3 * m + 2], l, slot), (uint32_t)a.f * ngrp * 2);
    }

    if constexpr (G > 1) {
        // Blocks of G groups of ROWS_B rows: the expert's tokens go in chunks
        // of 4, 2 or 1 (as many as remain, so few slots compute padding); for
        // each chunk the block streams its G groups, the weight rows of group
        // gi + 1 requested before group gi is computed.
        struct Wb {
            u32x4 qv[RB][2][NP];
            float sv[RB][2][NP], bv[RB][2][NP];
        };
        auto load_rows = [&](int rb_base, Wb &W) {
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
                const int row = min(rb_base + rr * RPI + grp, a.f - 1);  // clamped: in-bounds, never written
#pragma unroll
                for (int m = 0; m < 2; ++m) {
#pragma unroll
                    for (int np = 0; np < NP; ++np) {
                        const uint32_t col = (uint32_t)(np * LPR + gl);
                        const uint32_t g = col / 2;
                        W.qv[rr][m][np] = ld128_once(qr[m], (uint32_t)row * (d / 2) + col * 16);
                        W.sv[rr][m][np] = h2f(ld16(sr[m], sb_index((uint32_t)row, g, ngrp) * 2));
                        W.bv[rr][m][np] = h2f(ld16(br[m], sb_index((uint32_t)row, g, ngrp) * 2));
                    }
                }
            }
        };
        auto chunk = [&](auto tcc, int c0) {
            constexpr int TCc = decltype(tcc)::value;
            constexpr int NVc = 2 * RB * TCc;
            int tok[TCc], pid[TCc];
            uint32_t xp[TCc][NP][4][4];
            float xs[TCc][NP];
#pragma unroll
            for (int t = 0; t < TCc; ++t) {
                const int ci = c0 + t;
                int p = -1, tk = -1;
                if (ci < p_count) {
                    if (is_shared) {
                        tk = ci;
                        p = a.B * a.K + ci;
                    } else {
                        tk = plist[p_begin + ci] / a.K;
                        p = p_begin + ci;  // a batch keeps its h rows in sorted pair order
                    }
                }
                tok[t] = tk;
                pid[t] = p;
                const int tl = tk >= 0 ? tk : 0;  // a padding slot reads token 0; never written
#pragma unroll
                for (int np = 0; np < NP; ++np) {
                    float sm = 0.0f;
#pragma unroll
                    for (int wd = 0; wd < 4; ++wd) {
                        const uint16_t *xr = a.x + ((int64_t)l * a.B + tl) * d + (np * LPR + gl) * 32 + wd * 8;
                        x_pairs_m(*reinterpret_cast<const u32x4 *>(xr), xp[t][np][wd], sm);
                    }
                    xs[t][np] = sm;
                }
            }
            // Two register stages used in turn (group gi computes from one
            // while group gi + 1's rows land in the other), so no copy.
            Wb W0, W1;
            load_rows(row_base, W0);
            auto group = [&](int gi, const Wb &Wc, Wb &Wn) {
                const int rbase = row_base + gi * ROWS_B;
                if (gi + 1 < G) load_rows(rbase + ROWS_B, Wn);
                float acc[NVc];
#pragma unroll
                for (int i = 0; i < NVc; ++i) acc[i] = 0.0f;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
#pragma unroll
                        for (int np = 0; np < NP; ++np) {
                            const float sc = Wc.sv[rb][m][np] * kDenormScale;
                            const float bi = Wc.bv[rb][m][np];
#pragma unroll
                            for (int t = 0; t < TCc; ++t) {
                                float dacc = 0.0f;
#pragma unroll
                                for (int wd = 0; wd < 4; ++wd) dacc = dot_word_m(Wc.qv[rb][m][np][wd], xp[t][np][wd], dacc);
                                acc[(m * RB + rb) * TCc + t] += sc * dacc + bi * xs[t][np];
                            }
                        }
                    }
                }
                group_reduce_scatter<NVc, LPR>(acc);
                // Gate values in the lower half of a row group, up values in
                // the upper half (partner lane ^ LPR/2).
                constexpr int PER = NVc >= LPR ? NVc / LPR : 1;
                constexpr int DUP = NVc >= LPR ? 1 : LPR / NVc;
#pragma unroll
                for (int j = 0; j < PER; ++j) {
                    const int vi = NVc >= LPR ? gl * PER + j : gl / DUP;  // value index
                    const int m = vi / (RB * TCc);
                    const int rb = (vi / TCc) % RB;
                    const int t = vi % TCc;
                    float val = acc[j];
                    const int row = rbase + rb * RPI + grp;
                    if (is_shared && a.r > 0 && row < a.f && tok[t] >= 0) {
                        const uint16_t *brow = a.lb[m] + (int64_t)l * (a.lb_ls[m] / 2) + (int64_t)row * a.r;
                        const float *av = a.lora_a + (((int64_t)l * a.B + tok[t]) * 3 + m) * a.r;
                        float dl = 0.0f;
                        for (int i = 0; i < a.r; ++i) dl += h2f(brow[i]) * av[i];
                        val += a.lscale * dl;
                    }
                    const float other = __shfl_xor(val, LPR / 2);
                    if (m == 0 && (NVc >= LPR || gl % DUP == 0) && row < a.f && tok[t] >= 0)
                        hrow(a, l, pid[t])[row] = silu(val) * other;
                }
            };
            static_assert(G % 2 == 0, "groups are taken in pairs");
            for (int gi = 0; gi < G; gi += 2) {
                if (row_base + gi * ROWS_B >= a.f) break;
                group(gi, W0, W1);
                if (row_base + (gi + 1) * ROWS_B >= a.f) break;
                group(gi + 1, W1, W0);
            }
        };
        for (int c0 = 0; c0 < p_count;) {
            const int rem = p_count - c0;
            if (rem >= 3) {
                chunk(std::integral_constant<int, 4>{}, c0);
                c0 += 4;
            } else if (rem == 2) {
                chunk(std::integral_constant<int, 2>{}, c0);
                c0 += 2;
            } else {
                chunk(std::integral_constant<int, 1>{}, c0);
                c0 += 1;
            }
        }
        return;
    }
    for (int c0 = 0; c0 < p_count; c0 += TC) {
        // Token chunk: x slices as pairs, and their sums per pass.
        int tok[TC];
        int pid[TC];
        uint32_t xp[TC][NP][4][4];
        float xs[TC][NP];
#pragma unroll
        for (int t = 0; t < TC; ++t) {
            const int ci = c0 + t;
            int p = -1, tk = -1;
            if (ci < p_count) {
                if (is_shared) {
                    tk = ci;
                    p = a.B * a.K + ci;
                } else if (plist) {
                    tk = plist[p_begin + ci] / a.K;
                    p = p_begin + ci;  // a batch keeps its h rows in sorted pair order
                } else {
                    p = p_begin;
                    tk = 0;
                }
            }
            tok[t] = tk;
            pid[t] = p;
            const int tl = tk >= 0 ? tk : 0;  // padding tokens read token 0; never written
#pragma unroll
            for (int np = 0; np < NP; ++np) {
                float s = 0.0f;
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    const uint16_t *xr = a.x + ((int64_t)l * a.B + tl) * d + (np * LPR + gl) * 32 + wd * 8;
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(xr);
                    x_pairs(v, xp[t][np][wd]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        f16x2 hv = as_h2(v[j]);
                        s += (float)hv[0] + (float)hv[1];
                    }
                }
                xs[t][np] = s;
            }
        }

        float acc[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i] = 0.0f;
        // Rows in batches of RBB: the batch's code loads are issued together,
        // then consumed; the scheduling fence keeps the compiler from hoisting
        // every batch's loads at once (register pressure).
        constexpr int RBB = RB < 4 ? RB : 4;
#pragma unroll
        for (int rb0 = 0; rb0 < RB; rb0 += RBB) {
            u32x4 qv[RBB][2][NP];
            float sv[RBB][2][NP], bv[RBB][2][NP];
#pragma unroll
            for (int rr = 0; rr < RBB; ++rr) {
                // Rows past the end are clamped to the last row (in-bounds
                // loads, results never written) so the loads stay unconditional.
                const int row = min(row_base + (rb0 + rr) * RPI + grp, a.f - 1);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
#pragma unroll
                    for (int np = 0; np < NP; ++np) {
                        const uint32_t col = (uint32_t)(np * LPR + gl);  // 32-element column block
                        const uint32_t g = col / 2;                           // its group
                        qv[rr][m][np] = ld128_once(qr[m], (uint32_t)row * (d / 2) + col * 16);
                        sv[rr][m][np] = h2f(ld16(sr[m], sb_index((uint32_t)row, g, ngrp) * 2));
                        bv[rr][m][np] = h2f(ld16(br[m], sb_index((uint32_t)row, g, ngrp) * 2));
                    }
                }
            }
#pragma unroll
            for (int rr = 0; rr < RBB; ++rr) {
                const int rb = rb0 + rr;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
#pragma unroll
                    for (int np = 0; np < NP; ++np) {
                        const float s = sv[rr][m][np];
                        const float b16 = bv[rr][m][np] - 16.0f * s;
#pragma unroll
                        for (int t = 0; t < TC; ++t) {
                            float dacc = 0.0f;
#pragma unroll
                            for (int wd = 0; wd < 4; ++wd) dacc = dot_word(qv[rr][m][np][wd], xp[t][np][wd], dacc);
                            acc[(m * RB + rb) * TC + t] += s * dacc + b16 * xs[t][np];
                        }
                    }
                }
            }
            __asm__ __volatile__("" ::: "memory");  // keep batches apart (register pressure)
        }

        group_reduce_scatter<NV, LPR>(acc);

        // Each lane now holds totals; gate values in the lower half of a row
        // group, up values in the upper half (partner lane ^ LPR/2).
        constexpr int PER = NV >= LPR ? NV / LPR : 1;
        constexpr int DUP = NV >= LPR ? 1 : LPR / NV;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int vi = NV >= LPR ? gl * PER + j : gl / DUP;  // value index
            const int m = vi / (RB * TC);
            const int rb = (vi / TC) % RB;
            const int t = vi % TC;
            float val = acc[j];
            const int row = row_base + rb * RPI + grp;
            if (is_shared && a.r > 0 && row < a.f && tok[t] >= 0) {
                const uint16_t *brow = a.lb[m] + (int64_t)l * (a.lb_ls[m] / 2) + (int64_t)row * a.r;
                const float *av = a.lora_a + (((int64_t)l * a.B + tok[t]) * 3 + m) * a.r;
                float dl = 0.0f;
                for (int i = 0; i < a.r; ++i) dl += h2f(brow[i]) * av[i];
                val += a.lscale * dl;
            }
            const float other = __shfl_xor(val, LPR / 2);
            if (m == 0 && (NV >= LPR || gl % DUP == 0) && row < a.f && tok[t] >= 0)
                hrow(a, l, pid[t])[row] = silu(val) * other;
        }
    }
}

// ---------------------------------------------------------------------------
// 3. down + weighted combine. LPR lanes per row (f = 32 * LPR), RPI rows per
// wave instruction, IT instructions per wave (kDownRows rows per block).
// ---------------------------------------------------------------------------
template <int LPR>
struct DownCfg {
    static constexpr int RPI = kWave / LPR;
    static constexpr int IT = kDownRows / (kWaves * RPI) > 0 ? kDownRows / (kWaves * RPI) : 1;
};

// Partial dot of one row pass: sum over the lane's 32 columns of (s q + b) h.
E0_DEV float down_dot(const u32x4 qv, float s, float b, const float (&h)[32], float hsum) {
    float acc = 0.0f;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
        const uint32_t w = qv[wd];
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc += (float)((lo >> (8 * k)) & 0xFFu) * h[wd * 8 + 2 * k];
            acc += (float)((hi >> (8 * k)) & 0xFFu) * h[wd * 8 + 2 * k + 1];
        }
    }
    return s * acc + b * hsum;
}

template <int LPR>
__global__ __launch_bounds__(kThreads, LPR <= 16 ? 3 : 1) void decode_down_kernel(DecodeArgs a) {
    constexpr int RPI = DownCfg<LPR>::RPI;
    constexpr int IT = DownCfg<LPR>::IT;
    __shared__ float s_acc[kMaxB][kDownRows];
    __shared__ float s_lora[kMaxB][kMaxR];
    __shared__ __attribute__((aligned(16))) float s_h[kHChunkFloats];  // staged h rows (B > 1)
    __shared__ int s_pid[kHChunkFloats / 128 + 1], s_pslot[kHChunkFloats / 128 + 1];
    __shared__ float s_pw[kHChunkFloats / 128 + 1];
    __shared__ __attribute__((aligned(16))) float s_hs[kHChunkFloats / 8];  // partial h sums (B > 1)
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int gl = lane % LPR, grp = lane / LPR;
    const int l = blockIdx.x;
    const int row0 = blockIdx.y * kDownRows;
    const int f = a.f, d = a.d;
    const int fgrp = f / kGroup;
    const int col0 = gl * 32;
    const int g = col0 / kGroup;
    int rows[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) rows[it] = row0 + (wv * IT + it) * RPI + grp;

    // Shared-expert LoRA: a_d[t] = A_down h_shared[t] (r values per token).
    const bool lora = a.has_shared && a.r > 0;
    if (lora) {
        const int jobs = a.B * a.r;
        for (int job = wv; job < jobs; job += kWaves) {
            const int t = job / a.r, i = job % a.r;
            const uint16_t *arow = a.la[2] + (int64_t)l * (a.la_ls[2] / 2) + (int64_t)i * f;
            const float *hs = hrow(a, l, a.B * a.K + t);
            float acc = 0.0f;
            for (int c = lane; c < f; c += kWave) acc += h2f(arow[c]) * hs[c];
            acc = wave_sum(acc);
            if (lane == 0) s_lora[t][i] = acc;
        }
        __syncthreads();
    }

    // One expert's contribution to this lane's rows for pair p, weight wk.
    auto expert_rows = [&](const Stack &st, int slot, int p, float wk, float (&out)[IT]) {
        const rsrc_t qb = make_rsrc(part_at(st.p[6], l, slot), (uint32_t)d * f / 2);
        const rsrc_t sb = make_rsrc(part_at(st.p[7], l, slot), (uint32_t)d * fgrp * 2);
        const rsrc_t bb = make_rsrc(part_at(st.p[8], l, slot), (uint32_t)d * fgrp * 2);
        const float *hp = hrow(a, l, p) + col0;
        float h[32];
        float hsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            f32x4 v = *reinterpret_cast<const f32x4 *>(hp + 4 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h[4 * i + j] = v[j];
                hsum += v[j];
            }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const uint32_t row = (uint32_t)min(rows[it], d - 1);  // clamped: in-bounds, never written
            const u32x4 qv = ld128_once(qb, row * (f / 2) + gl * 16);
            const float s = h2f(ld16(sb, sb_index(row, (uint32_t)g, (uint32_t)fgrp) * 2));
            const float b = h2f(ld16(bb, sb_index(row, (uint32_t)g, (uint32_t)fgrp) * 2));
            out[it] += wk * down_dot(qv, s, b, h, hsum);
        }
    };

    if (!a.has_plan) {
        // B == 1: experts in k order, then the shared expert.
        float acc[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) acc[it] = 0.0f;
        for (int k = 0; k < a.K; ++k) {
            const int e = a.idx[(int64_t)l * a.K + k];
            if (e < 0 || e >= a.E) continue;
            const int slot = a.slot_of[(int64_t)l * a.E + e];
            if (slot < 0 || slot >= a.S) continue;
            expert_rows(a.pool, slot, k, a.w[(int64_t)l * a.K + k], acc);
        }
        if (a.has_shared) expert_rows(a.sh, 0, a.K, 1.0f, acc);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            float v = group_sum(acc[it], LPR);
            const int row = rows[it];
            if (lora && row < d) {
                const uint16_t *brow = a.lb[2] + (int64_t)l * (a.lb_ls[2] / 2) + (int64_t)row * a.r;
                float dl = 0.0f;
                for (int i = 0; i < a.r; ++i) dl += h2f(brow[i]) * s_lora[0][i];
                v += a.lscale * dl;
            }
            if (gl == 0 && row < d) a.y[(int64_t)l * d + row] = v;
        }
        return;
    }

    // B > 1: the layer's pairs in sorted order (unique experts ascending, an
    // expert's pairs in token order), each pair's contribution folded into the
    // block's per-token accumulators in that order. The h rows of a chunk of
    // pairs are staged in LDS by one cooperative load (their latencies
    // overlap). An expert's pairs form one run: its weight rows are loaded
    // once for the run, and the next expert's rows are requested when a run
    // starts, so their latency hides behind the whole run.
    for (int i = threadIdx.x; i < a.B * kDownRows; i += kThreads) s_acc[i / kDownRows][i % kDownRows] = 0.0f;
    __syncthreads();
    const int nu = a.ucnt[l];
    const int32_t *uoff = a.uoff + (int64_t)l * (a.umax + 1);
    const int32_t *plist = a.pairs + (int64_t)l * a.B * a.K;
    auto fold = [&](float (&part)[IT], int t) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const float v = group_sum(part[it], LPR);
            const int row = rows[it];
            if (gl == 0 && row < d) s_acc[t][row - row0] += v;
        }
    };
    struct Wrows {
        u32x4 q[IT];
        float s[IT], b[IT];
    };
    auto load_w = [&](int slot, Wrows &wr) {
        const rsrc_t qb = make_rsrc(part_at(a.pool.p[6], l, slot), (uint32_t)d * f / 2);
        const rsrc_t sb = make_rsrc(part_at(a.pool.p[7], l, slot), (uint32_t)d * fgrp * 2);
        const rsrc_t bb = make_rsrc(part_at(a.pool.p[8], l, slot), (uint32_t)d * fgrp * 2);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const uint32_t row = (uint32_t)min(rows[it], d - 1);  // clamped: in-bounds, never written
            wr.q[it] = ld128_once(qb, row * (f / 2) + gl * 16);
            wr.s[it] = h2f(ld16(sb, sb_index(row, (uint32_t)g, (uint32_t)fgrp) * 2));
            wr.b[it] = h2f(ld16(bb, sb_index(row, (uint32_t)g, (uint32_t)fgrp) * 2));
        }
    };
    const int npairs = nu > 0 ? cload(uoff, nu) : 0;
    const int chunk = kHChunkFloats / f;  // pairs per LDS chunk (f <= 2048: at least 2)
    const int32_t *pslot = a.pslot + (int64_t)l * a.B * a.K;
    const float *wl = a.w + (int64_t)l * a.B * a.K;
    const int32_t *uslot = a.uslot + (int64_t)l * a.umax;
    auto uslot_at = [&](int u) {
        const int sl = cload(uslot, u);
        return sl < 0 ? 0 : sl;  // a non-resident expert's pairs are skipped below; its load reads slot 0
    };
    Wrows wc, wn;
    int u_cur = 0, run_end = 0;  // the current run's expert and the pair after its run
    if (nu > 0) {
        load_w(uslot_at(0), wc);
        run_end = cload(uoff, 1);
        if (nu > 1) load_w(uslot_at(1), wn);
    }
    for (int c0 = 0; c0 < npairs; c0 += chunk) {
        const int cn = min(chunk, npairs - c0);
        __syncthreads();  // the previous chunk's LDS reads are done
        // Per pair of the chunk: pair index, slot and routing weight (plus the
        // slot of the first pair after the chunk); h rows in the layout
        // [pair][i][gl] of 16-byte chunks, lane gl's i-th chunk of its 32
        // columns, so the lanes of a row read consecutive chunks.
        if (threadIdx.x <= cn && c0 + threadIdx.x < npairs) {
            const int pi = c0 + threadIdx.x;
            s_pslot[threadIdx.x] = pslot[pi];
            if ((int)threadIdx.x < cn) {
                const int p = plist[pi];
                s_pid[threadIdx.x] = p;
                s_pw[threadIdx.x] = wl[p];
            }
        }
        // h of the chunk's pairs in the form dot_word_m2 takes: per lane group
        // gl (32 columns) and word wd (8 columns), 4 dwords of fp16 hi pairs
        // (element j with j + 4, odd j scaled by 1/16) and 4 of lo pairs
        // (the rounding remainders), at [pair][2 wd + part][gl]; and the four
        // partial sums of the group's h at [pair][gl][wd].
        uint32_t *s_hq = reinterpret_cast<uint32_t *>(s_h);
        for (int v = threadIdx.x; v < cn * LPR * 4; v += kThreads) {
            const int pc = v / (LPR * 4), gq = (v / 4) % LPR, wd = v % 4;
            const float *src = hrow(a, l, c0 + pc) + gq * 32 + wd * 8;
            const f32x4 lo4 = *reinterpret_cast<const f32x4 *>(src), hi4 = *reinterpret_cast<const f32x4 *>(src + 4);
            u32x4 qh, ql;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float sc = (j & 1) ? 0.0625f : 1.0f;
                const float va = lo4[j] * sc, vb = hi4[j] * sc;
                const f16 ha = (f16)va, hb = (f16)vb;
                const f16 la = (f16)(va - (float)ha), lb = (f16)(vb - (float)hb);
                qh[j] = (uint32_t)__builtin_bit_cast(uint16_t, ha) | (uint32_t)__builtin_bit_cast(uint16_t, hb) << 16;
                ql[j] = (uint32_t)__builtin_bit_cast(uint16_t, la) | (uint32_t)__builtin_bit_cast(uint16_t, lb) << 16;
            }
            *reinterpret_cast<u32x4 *>(&s_hq[((pc * 8 + 2 * wd) * LPR + gq) * 4]) = qh;
            *reinterpret_cast<u32x4 *>(&s_hq[((pc * 8 + 2 * wd + 1) * LPR + gq) * 4]) = ql;
            s_hs[(pc * LPR + gq) * 4 + wd] = (lo4[0] + lo4[1]) + (lo4[2] + lo4[3]) + ((hi4[0] + hi4[1]) + (hi4[2] + hi4[3]));
        }
        __syncthreads();
        for (int pc = 0; pc < cn; ++pc) {
            const int pi = c0 + pc;
            if (pi == run_end && u_cur + 1 < nu) {
                // The next expert's run starts: its rows were requested a run ago.
                ++u_cur;
                wc = wn;
                run_end = cload(uoff, u_cur + 1);
                if (u_cur + 1 < nu) load_w(uslot_at(u_cur + 1), wn);
            }
            if (s_pslot[pc] >= 0) {
                uint32_t hh[16], hl[16];
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    const u32x4 vh = *reinterpret_cast<const u32x4 *>(&s_hq[((pc * 8 + 2 * wd) * LPR + gl) * 4]);
                    const u32x4 vl = *reinterpret_cast<const u32x4 *>(&s_hq[((pc * 8 + 2 * wd + 1) * LPR + gl) * 4]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        hh[4 * wd + j] = vh[j];
                        hl[4 * wd + j] = vl[j];
                    }
                }
                const f32x4 hs4 = *reinterpret_cast<const f32x4 *>(&s_hs[(pc * LPR + gl) * 4]);
                const float hsum = (hs4[0] + hs4[1]) + (hs4[2] + hs4[3]);
                const float wk = s_pw[pc];
                float part[IT];
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    float dacc = 0.0f;
#pragma unroll
                    for (int wd = 0; wd < 4; ++wd) dacc = dot_word_m2(wc.q[it][wd], hh + 4 * wd, hl + 4 * wd, dacc);
                    part[it] = wk * ((wc.s[it] * kDenormScale) * dacc + wc.b[it] * hsum);
                }
                fold(part, s_pid[pc] / a.K);
            }
        }
    }
    if (a.has_shared) {
        for (int t = 0; t < a.B; ++t) {
            float part[IT];
#pragma unroll
            for (int it = 0; it < IT; ++it) part[it] = 0.0f;
            expert_rows(a.sh, 0, a.B * a.K + t, 1.0f, part);
            fold(part, t);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < a.B * kDownRows; i += kThreads) {
        const int t = i / kDownRows, rr = i % kDownRows, row = row0 + rr;
        if (row >= d) continue;
        float v = s_acc[t][rr];
        if (lora) {
            const uint16_t *brow = a.lb[2] + (int64_t)l * (a.lb_ls[2] / 2) + (int64_t)row * a.r;
            float dl = 0.0f;
            for (int j = 0; j < a.r; ++j) dl += h2f(brow[j]) * s_lora[t][j];
            v += a.lscale * dl;
        }
        a.y[((int64_t)l * a.B + t) * d + row] = v;
    }
}

// ---------------------------------------------------------------------------
// 3b. down for B > 1 on the matrix cores (v_mfma_f32_16x16x32_f16), d_ff of
// 128, 256 or 512. A block owns kDownRows output rows of a layer, 16 per wavefront, and
// walks the layer's experts in sorted order, then the shared expert. The MFMA
// rows are a window of 16 consecutive sorted pairs, staged in LDS as fp16
// hi + lo parts of h in the order of the denormal-nibble product (pairs
// (h_j, h_j+4) per code word, odd j scaled by 1/16); the columns are the
// wavefront's 16 output rows, with their code words as fp16 denormals
// (q 2^-24, exact); each product is exact in fp32. Per quantisation group g
// (64 inputs: two K = 32 slices, hi and lo) P_g = 2^-24 sum q h, and the
// group adds s 2^24 P_g + b sum_g h. A pass computes all 16 rows of the
// window and folds those of the current expert, times their routing weight,
// into the block's per-token accumulators in LDS in sorted order (y written
// once, no atomics). The experts' weight rows (16 code bytes per lane per two
// groups, and the wavefront's scales and biases, 8 rows of one group per
// lane, in one 16-byte load) sit in a ring of kDmRing register stages: expert
// u + kDmRing - 1 is requested before expert u is computed.
// Lane (n = lane % 16, kq = lane / 16): A row n = window slot n, B column
// n = output row n, over inputs 32 (kq & 1) + 8 (kq >> 1) + 16 s .. + 7 of
// group g for the slices s = 0, 1; C rows 4 kq .. 4 kq + 3 (window slots) of
// column n.
// ---------------------------------------------------------------------------
constexpr int kDmSlots = 16;  // window slots (MFMA rows)
constexpr int kDmRing = 4;    // weight stages in flight

typedef _Float16 h8mf __attribute__((ext_vector_type(8)));
typedef float f4mf __attribute__((ext_vector_type(4)));

template <int FG>
struct DmStage {
    u32x4 w[FG / 2];  // chunk c: 16 code bytes of output row n at byte 64 c + 16 kq (group 2 c + kq / 2)
    u32x4 sb;         // lane i < 2 FG: scales of 8 rows of one group; lane 32 + i: the biases
};

// Dynamic LDS of the kernel (bytes): accumulators, LoRA A h, h window, group
// sums of the window, each wavefront's scale/bias table, and the layer's run
// table (first pair of each expert's run, and its slot).
__host__ __device__ inline int dm_slot_dwords(int fg) { return fg * 64 + 4; }  // + 16 B: slots start on different banks
__host__ __device__ inline size_t dm_lds_bytes(int B, int r, int fg, int umax) {
    return (size_t)4 * (B * kDownRows + ((B * r + 3) & ~3) + kDmSlots * dm_slot_dwords(fg) + fg * kDmSlots) +
           (size_t)kWaves * 512 + (size_t)4 * (2 * umax + 1);
}
constexpr size_t kDmMaxLds = 64 * 1024 - 256;  // dynamic LDS cap, leaving room for the static arrays

// Every global load of the expert loop is unconditional and the same for
// every expert (the ring's tail re-reads the last expert), so the compiler
// can count the loads issued after a stage and wait for that stage alone
// instead of for all loads in flight.
template <int FG>
__global__ __launch_bounds__(kThreads, 3) void decode_down_mfma_kernel(DecodeArgs a) {
    extern __shared__ __attribute__((aligned(16))) float dm_lds[];
    __shared__ int s_tok[kDmSlots];
    __shared__ float s_wt[kDmSlots];
    const int lane = threadIdx.x & 63, wv = wave_id(), tid = threadIdx.x;
    const int nl = lane & 15, kq = lane >> 4;
    const int l = blockIdx.x, row0 = blockIdx.y * kDownRows;
    const int d = a.d, f = FG * kGroup, B = a.B;
    constexpr int slot_dw = FG * 64 + 4;
    float *s_acc = dm_lds;                      // [B][kDownRows]
    float *s_lora = s_acc + B * kDownRows;      // [B][r]
    uint32_t *s_hw = reinterpret_cast<uint32_t *>(s_lora + ((B * a.r + 3) & ~3));  // [slot][g][kq][hi w0, hi w1, lo w0, lo w1]
    float *s_hs = reinterpret_cast<float *>(s_hw + kDmSlots * slot_dw);          // [g][slot]
    uint16_t *s_sb0 = reinterpret_cast<uint16_t *>(s_hs + FG * kDmSlots);
    uint16_t *s_sb = s_sb0 + wv * 256;  // [s|b][octet][g][8 rows]
    int32_t *s_uoff = reinterpret_cast<int32_t *>(s_sb0 + kWaves * 256);  // [umax + 1]
    int32_t *s_uslot = s_uoff + a.umax + 1;                               // [umax]

    // Shared-expert LoRA: a_d[t] = A_down h_shared[t] (r values per token).
    const bool lora = a.has_shared && a.r > 0;
    if (lora) {
        const int jobs = B * a.r;
        for (int job = wv; job < jobs; job += kWaves) {
            const int t = job / a.r, i = job % a.r;
            const uint16_t *arow = a.la[2] + (int64_t)l * (a.la_ls[2] / 2) + (int64_t)i * f;
            const float *hs = hrow(a, l, B * a.K + t);
            float acc = 0.0f;
            for (int c = lane; c < f; c += kWave) acc += h2f(arow[c]) * hs[c];
            acc = wave_sum(acc);
            if (lane == 0) s_lora[t * a.r + i] = acc;
        }
    }
    for (int i = tid; i < B * kDownRows; i += kThreads) s_acc[i] = 0.0f;

    const int row = row0 + wv * 16 + nl;
    const uint32_t rowc = (uint32_t)min(row, d - 1);  // clamped: in-bounds, never written
    const int nu = a.ucnt[l];
    const int nrun = nu + (a.has_shared ? 1 : 0);
    const int32_t *uoff = a.uoff + (int64_t)l * (a.umax + 1);
    const int32_t *uslot = a.uslot + (int64_t)l * a.umax;
    const int32_t *plist = a.pairs + (int64_t)l * B * a.K;
    const float *pwt = a.pwt + (int64_t)l * B * a.K;
    const int npairs = nu > 0 ? cload(uoff, nu) : 0;
    // The run table in LDS: the expert loop reads it in a few cycles where a
    // scalar load from memory would put a round trip in front of every run.
    for (int i = tid; i <= nu; i += kThreads) s_uoff[i] = uoff[i];
    for (int i = tid; i < nu; i += kThreads) s_uslot[i] = uslot[i];
    const int ntot = npairs + (a.has_shared ? B : 0);
    // This lane's 16-byte chunk of the wavefront's scale (lanes 0-31) or bias
    // (lanes 32-63) rows: octet oct0 + i / FG, group i % FG (i = lane mod
    // 2 FG; the lanes past 2 FG repeat a chunk and are not used).
    const int li = lane & 31;
    const int sbi = li % (2 * FG);
    const uint32_t sb_off = (uint32_t)((min((row0 + wv * 16) / 8 + sbi / FG, d / 8 - 1) * FG + sbi % FG) * 16);

    auto load_stage = [&](int u, DmStage<FG> &S) {
        u = min(u, nrun - 1);
        const bool shx = u >= nu;
        int slot = 0;
        if (!shx) {
            slot = __builtin_amdgcn_readfirstlane(s_uslot[u]);
            slot = slot < 0 ? 0 : slot;  // a non-resident expert is skipped; its stage reads slot 0
        }
        const Part pq = shx ? a.sh.p[6] : a.pool.p[6];
        const Part ps = shx ? a.sh.p[7] : a.pool.p[7];
        const Part pb = shx ? a.sh.p[8] : a.pool.p[8];
        const rsrc_t qb = make_rsrc(part_at(pq, l, slot), (uint32_t)d * f / 2);
        // Each load reads 64 contiguous bytes (two groups) of each of the 16
        // rows: a probe of this grid streams that pattern at the full read
        // rate, and 32 bytes of 16 rows per load at three quarters of it.
        // One offset register for the stage's loads (the chunk goes in the
        // instruction's immediate offset), not one per chunk held by the
        // loop. Plain loads: with the nontemporal hint the wavefronts stalled
        // about twice as long issuing them.
        uint32_t qoff = rowc * (f / 2) + kq * 16;
        __asm__ volatile("" : "+v"(qoff));
#pragma unroll
        for (int c = 0; c < FG / 2; ++c) S.w[c] = __builtin_amdgcn_raw_buffer_load_b128(qb, (int)(qoff + c * 64), 0, 0);
        const char *sbp = lane < 32 ? part_at(ps, l, slot) : part_at(pb, l, slot);
        S.sb = *reinterpret_cast<const u32x4 *>(sbp + sb_off);
    };

    // Window c: slots c * 16 .. c * 16 + 15 of the sorted pairs (then the
    // shared expert's B rows). Every wavefront takes part. The window's rows
    // and routing data are requested before the barrier that frees the LDS,
    // so the two waits overlap.
    constexpr int kItems = kDmSlots * FG * 4;  // (slot, group, quarter): 16 h values each
    constexpr int kIpt = (kItems + kThreads - 1) / kThreads;
    int cur = -1;
    auto stage_window = [&](int c) {
        float v[kIpt][16];
#pragma unroll
        for (int k = 0; k < kIpt; ++k) {
            const int it = tid + k * kThreads;
            const int q4 = it & 3, g = (it >> 2) % FG, sl = (it >> 2) / FG;
            const int pi = c * kDmSlots + sl;
            if (it < kItems && pi < ntot) {
                const int hp = pi < npairs ? pi : B * a.K + (pi - npairs);
                // the inputs lane kq = q4 takes in the pass: 8 at 32 (q4 & 1) +
                // 8 (q4 >> 1) + 16 s of the group, s = 0, 1
                const float *src = hrow(a, l, hp) + g * kGroup + 32 * (q4 & 1) + 8 * (q4 >> 1);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 t = *reinterpret_cast<const f32x4 *>(src + 16 * (j >> 1) + 4 * (j & 1));
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[k][4 * j + e] = t[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) v[k][e] = 0.0f;
            }
        }
        int tk = -1;
        float wt = 0.0f;
        if (tid < kDmSlots) {
            const int pi = c * kDmSlots + tid;
            if (pi < npairs) {
                tk = plist[pi] / a.K;
                wt = pwt[pi];
            } else if (pi < ntot) {
                tk = pi - npairs;
                wt = 1.0f;
            }
        }
        __syncthreads();  // every wavefront is done with the previous window
#pragma unroll
        for (int k = 0; k < kIpt; ++k) {
            const int it = tid + k * kThreads;
            if (it < kItems) {
                const int q4 = it & 3, g = (it >> 2) % FG, sl = (it >> 2) / FG;
                u32x4 hv[2], lv[2];
                float sum = 0.0f;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float sc = (e & 1) ? 0.0625f : 1.0f;
                        const float va = v[k][8 * j + e] * sc, vb = v[k][8 * j + e + 4] * sc;
                        const f16 ha = (f16)va, hb = (f16)vb;
                        const f16 la = (f16)(va - (float)ha), lb = (f16)(vb - (float)hb);
                        hv[j][e] = (uint32_t)__builtin_bit_cast(uint16_t, ha) | (uint32_t)__builtin_bit_cast(uint16_t, hb) << 16;
                        lv[j][e] = (uint32_t)__builtin_bit_cast(uint16_t, la) | (uint32_t)__builtin_bit_cast(uint16_t, lb) << 16;
                        sum += v[k][8 * j + e] + v[k][8 * j + e + 4];
                    }
                }
                u32x4 *dst = reinterpret_cast<u32x4 *>(s_hw + sl * slot_dw + (g * 4 + q4) * 16);
                dst[0] = hv[0];
                dst[1] = hv[1];
                dst[2] = lv[0];
                dst[3] = lv[1];
                // the four quarters of a group are four consecutive lanes
                sum += __shfl_xor(sum, 1);
                sum += __shfl_xor(sum, 2);
                if (q4 == 0) s_hs[g * kDmSlots + sl] = sum;
            }
        }
        if (tid < kDmSlots) {
            s_tok[tid] = tk;
            s_wt[tid] = wt;
        }
        __syncthreads();
    };

    // One expert against window slots [sa, sb).
    auto pass = [&](const DmStage<FG> &S, int sa, int sb) {
        if (li < 2 * FG) *reinterpret_cast<u32x4 *>(s_sb + (((lane >> 5) * 2 + li / FG) * 8 + li % FG) * 8) = S.sb;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint32_t *hb = s_hw + nl * slot_dw + kq * 16;
        const int so = (nl >> 3) * 64 + (nl & 7);
        // The nibble masks and shift pass through an empty asm so that the
        // code words' masks are formed in this pass, group by group, not
        // hoisted out of the expert's passes (that would hold 64 more
        // registers).
        uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, sh8 = 8;
        __asm__ volatile("" : "+v"(m_lo), "+v"(m_hi), "+v"(sh8));
        f4mf totp = {0.0f, 0.0f, 0.0f, 0.0f}, totb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int g = 0; g < FG; ++g) {
            const u32x4 *hq = reinterpret_cast<const u32x4 *>(hb + g * 64);
            // words (s = 0, 1) of group g: word 2 s + (g & 1) of the swapped chunk
            const u32x4 W = S.w[g >> 1];
            // a code word w (8 codes) as the B operand: (q0, q4, 16 q1, 16 q5,
            // q2, q6, 16 q3, 16 q7) x 2^-24 as fp16 denormals
            const uint32_t w0 = W[g & 1], w1 = W[2 + (g & 1)], w08 = w0 >> sh8, w18 = w1 >> sh8;
            const h8mf b0 = __builtin_bit_cast(h8mf, u32x4{w0 & m_lo, w0 & m_hi, w08 & m_lo, w08 & m_hi});
            const h8mf b1 = __builtin_bit_cast(h8mf, u32x4{w1 & m_lo, w1 & m_hi, w18 & m_lo, w18 & m_hi});
            f4mf P = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8mf, hq[0]), b0,
                                                           f4mf{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            P = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8mf, hq[1]), b1, P, 0, 0, 0);
            P = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8mf, hq[2]), b0, P, 0, 0, 0);
            P = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8mf, hq[3]), b1, P, 0, 0, 0);
            // s P_g and b sum_g h kept apart (the 2^24 of the products is
            // applied once, below), each with the fp16 factor taken as is
            const float sc = h2f(s_sb[so + g * 8]), bi = h2f(s_sb[128 + so + g * 8]);
            const f4mf hs4 = *reinterpret_cast<const f4mf *>(s_hs + g * kDmSlots + 4 * kq);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                totp[i] = __builtin_fmaf(sc, P[i], totp[i]);
                totb[i] = __builtin_fmaf(bi, hs4[i], totb[i]);
            }
            // formed here, group by group: sunk into the fold's branches, the
            // sums would hold every group's products and operands at once
            __asm__("" : "+v"(totp), "+v"(totb));
        }
        f4mf tot;
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[i] = __builtin_fmaf(kDenormScale, totp[i], totb[i]);
        if (row < d) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sl = 4 * kq + i;
                if (sl >= sa && sl < sb) s_acc[s_tok[sl] * kDownRows + (row - row0)] += s_wt[sl] * tot[i];
            }
        }
        __builtin_amdgcn_wave_barrier();  // the table is rewritten by the next pass
    };

    // Chunk c holds group 2 c in lanes 0-31 and group 2 c + 1 in lanes 32-63.
    // Swapping the upper lanes of words 0 and 2 with the lower lanes of words
    // 1 and 3 leaves words 0 and 2 holding only group 2 c (codes 32 (kq & 1) +
    // 8 (kq >> 1) + 16 s, s = 0, 1) and words 1 and 3 only group 2 c + 1, in
    // the same lane order. Done once per expert, in place (the stage is not
    // read again until it is reloaded).
    auto swap_stage = [&](const DmStage<FG> &S) {
        DmStage<FG> T;
#pragma unroll
        for (int c = 0; c < FG / 2; ++c) {
            const auto r01 = __builtin_amdgcn_permlane32_swap(S.w[c][0], S.w[c][1], false, false);
            const auto r23 = __builtin_amdgcn_permlane32_swap(S.w[c][2], S.w[c][3], false, false);
            T.w[c] = u32x4{r01[0], r01[1], r23[0], r23[1]};
        }
        T.sb = S.sb;
        return T;
    };

    auto run = [&](int u, const DmStage<FG> &S0_) {
        const DmStage<FG> S = swap_stage(S0_);
        const int p0 = u < nu ? __builtin_amdgcn_readfirstlane(s_uoff[u]) : npairs;
        const int p1 = u < nu ? __builtin_amdgcn_readfirstlane(s_uoff[u + 1]) : ntot;
        const bool ok = u >= nu || __builtin_amdgcn_readfirstlane(s_uslot[u]) >= 0;
        for (int p = p0; p < p1;) {
            const int c = p / kDmSlots;
            while (cur < c) stage_window(++cur);
            const int q = min(p1, (c + 1) * kDmSlots);
            if (ok) pass(S, p - c * kDmSlots, q - c * kDmSlots);
            p = q;
        }
    };

    __syncthreads();  // run table, LoRA terms and zeroed accumulators
    if (nrun > 0) {
        static_assert(kDmRing == 4, "the ring below is unrolled for four stages");
        DmStage<FG> S0, S1, S2, S3;
        load_stage(0, S0);
        load_stage(1, S1);
        load_stage(2, S2);
        for (int u = 0; u < nrun; u += kDmRing) {
            load_stage(u + 3, S3);
            run(u, S0);
            if (u + 1 >= nrun) break;
            load_stage(u + 4, S0);
            run(u + 1, S1);
            if (u + 2 >= nrun) break;
            load_stage(u + 5, S1);
            run(u + 2, S2);
            if (u + 3 >= nrun) break;
            load_stage(u + 6, S2);
            run(u + 3, S3);
        }
    }
    __syncthreads();
    for (int i = tid; i < B * kDownRows; i += kThreads) {
        const int t = i / kDownRows, rr = i % kDownRows, orow = row0 + rr;
        if (orow >= d) continue;
        float v = s_acc[i];
        if (lora) {
            const uint16_t *brow = a.lb[2] + (int64_t)l * (a.lb_ls[2] / 2) + (int64_t)orow * a.r;
            float dl = 0.0f;
            for (int j = 0; j < a.r; ++j) dl += h2f(brow[j]) * s_lora[t * a.r + j];
            v += a.lscale * dl;
        }
        a.y[((int64_t)l * B + t) * d + orow] = v;
    }
}

// ---------------------------------------------------------------------------
// Batch-1 flat kernels. The rows of all experts of all layers form one list
// (layer, expert u, row), u = 0..K-1 the routed experts of the token and u = K
// the shared expert; each wavefront takes kFlatRows consecutive rows, which
// never straddle an expert (kFlatRows divides d_ff) so x and the expert's
// buffer descriptors are set once per wave. The grid is one round of resident
// waves: no tail of half-empty rounds, no per-block imbalance.
// ---------------------------------------------------------------------------
constexpr int kFlatRows = 32;  // rows per wavefront
constexpr int kFlatBatch = 4;  // rows per pipeline stage (loads issued together)

// Resolve expert u of layer l (batch 1): its slot (shared expert: slot 0 of
// the shared stack), or false for an invalid / non-resident id.
E0_DEV bool resolve_b1(const DecodeArgs &a, int l, int u, int &slot, bool flag) {
    if (u == a.K) {
        slot = 0;
        return true;
    }
    const int e = a.idx[(int64_t)l * a.K + u];
    if (e < 0 || e >= a.E) {
        if (flag) set_err(a.err, E0_DEV_BAD_ID);
        return false;
    }
    slot = a.slot_of[(int64_t)l * a.E + e];
    if (slot < 0 || slot >= a.S) {
        if (flag) set_err(a.err, E0_DEV_NOT_RESIDENT);
        return false;
    }
    return true;
}

// Part i of expert u's stack, by value (selecting a pointer between two
// kernel-argument structs would put the arguments in private memory).
E0_DEV Part part_of(const DecodeArgs &a, int u, int i) { return u == a.K ? a.sh.p[i] : a.pool.p[i]; }

template <int NP>
__global__ __launch_bounds__(kThreads) void decode_gateup_flat_kernel(DecodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int U = a.K + (a.has_shared ? 1 : 0);
    const int64_t r0 = ((int64_t)blockIdx.x * kWaves + wave_id()) * kFlatRows;
    if (r0 >= (int64_t)a.L * U * a.f) return;
    const int l = (int)(r0 / ((int64_t)U * a.f));
    const int u = (int)((r0 / a.f) % U);
    const int row0 = (int)(r0 % a.f);
    int slot;
    if (!resolve_b1(a, l, u, slot, row0 == 0 && lane == 0)) return;
    const int d = a.d, ngrp = d / kGroup;

    // x of this layer: 32 inputs per lane per pass, as (x_j, x_{j+4}) pairs.
    uint32_t xp[NP][4][4];
    float xs[NP];
#pragma unroll
    for (int np = 0; np < NP; ++np) {
        float sum = 0.0f;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(a.x + (int64_t)l * d + (np * 64 + lane) * 32 + wd * 8);
            x_pairs(v, xp[np][wd]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f16x2 hv = as_h2(v[j]);
                sum += (float)hv[0] + (float)hv[1];
            }
        }
        xs[np] = sum;
    }
    rsrc_t qr[2], sr[2], br[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        qr[m] = make_rsrc(part_at(part_of(a, u, 3 * m + 0), l, slot), (uint32_t)a.f * d / 2);
        sr[m] = make_rsrc(part_at(part_of(a, u, 3 * m + 1), l, slot), (uint32_t)a.f * ngrp * 2);
        br[m] = make_rsrc(part_at(part_of(a, u, 3 * m + 2), l, slot), (uint32_t)a.f * ngrp * 2);
    }
    float *hout = hrow(a, l, u);
    const bool lora = u == a.K && a.r > 0;
    const NibbleConsts nk = nibble_consts();

    // Two-stage software pipeline over batches of kFlatBatch rows: the loads
    // of batch b+1 are in flight while batch b is computed. The memory
    // clobbers keep the compiler from hoisting later batches' loads.
    struct Batch {
        u32x4 q[kFlatBatch][2][NP];
        uint32_t sb[kFlatBatch][2][NP];  // fp16 scale | fp16 bias << 16
    };
    auto load = [&](int b0, Batch &B) {
#pragma unroll
        for (int rr = 0; rr < kFlatBatch; ++rr) {
            const uint32_t row = (uint32_t)(row0 + b0 + rr);
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int np = 0; np < NP; ++np) {
                    const uint32_t col = (uint32_t)(np * 64 + lane);
                    B.q[rr][m][np] = ld128_once(qr[m], row * (d / 2) + col * 16);
                    const uint32_t so = sb_index(row, col / 2, (uint32_t)ngrp) * 2;
                    B.sb[rr][m][np] = (uint32_t)ld16(sr[m], so) | ((uint32_t)ld16(br[m], so) << 16);
                }
            }
        }
    };
    auto compute = [&](int b0, const Batch &B) {
        float acc[2 * kFlatBatch];
#pragma unroll
        for (int rr = 0; rr < kFlatBatch; ++rr) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                float v = 0.0f;
#pragma unroll
                for (int np = 0; np < NP; ++np) {
                    float dacc = 0.0f;
#pragma unroll
                    for (int wd = 0; wd < 4; ++wd) dacc = dot_word(B.q[rr][m][np][wd], xp[np][wd], dacc, nk);
                    const f16x2 sbv = as_h2(B.sb[rr][m][np]);
                    const float sc = (float)sbv[0], bi = (float)sbv[1];
                    v += sc * dacc + (bi - 16.0f * sc) * xs[np];
                }
                acc[m * kFlatBatch + rr] = v;
            }
        }
        // 2*kFlatBatch values over 64 lanes; gate values in lanes 0..31, the
        // matching up value in lane ^ 32.
        group_reduce_scatter<2 * kFlatBatch, kWave>(acc);
        constexpr int DUP = kWave / (2 * kFlatBatch);
        const int vi = lane / DUP, m = vi / kFlatBatch, rr = vi % kFlatBatch;
        const int row = row0 + b0 + rr;
        float val = acc[0];
        if (lora) {
            const uint16_t *brow = a.lb[m] + (int64_t)l * (a.lb_ls[m] / 2) + (int64_t)row * a.r;
            const float *av = a.lora_a + ((int64_t)l * 3 + m) * a.r;
            float dl = 0.0f;
            for (int i = 0; i < a.r; ++i) dl += h2f(brow[i]) * av[i];
            val += a.lscale * dl;
        }
        const float other = __shfl_xor(val, 32);
        if (m == 0 && lane % DUP == 0) hout[row] = silu(val) * other;
    };

    Batch B0, B1;
    load(0, B0);
#pragma unroll
    for (int b0 = 0; b0 < kFlatRows; b0 += 2 * kFlatBatch) {
        if (b0 + kFlatBatch < kFlatRows) load(b0 + kFlatBatch, B1);
        __asm__ __volatile__("" ::: "memory");
        compute(b0, B0);
        __asm__ __volatile__("" ::: "memory");
        if (b0 + 2 * kFlatBatch < kFlatRows) load(b0 + 2 * kFlatBatch, B0);
        __asm__ __volatile__("" ::: "memory");
        if (b0 + kFlatBatch < kFlatRows) compute(b0 + kFlatBatch, B1);
        __asm__ __volatile__("" ::: "memory");
    }
}

template <int LPR>
__global__ __launch_bounds__(kThreads) void decode_down_flat_kernel(DecodeArgs a) {
    constexpr int RPI = kWave / LPR;        // rows per wave instruction
    constexpr int IT = kFlatRows / RPI;     // instructions per wave
    __shared__ float s_lora[kMaxR];
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int gl = lane % LPR, grp = lane / LPR;
    const int f = a.f, d = a.d, fgrp = f / kGroup;
    // A block covers kWaves * kFlatRows rows of one layer (d is a multiple of 128).
    const int64_t rb0 = (int64_t)blockIdx.x * kWaves * kFlatRows;
    if (rb0 >= (int64_t)a.L * d) return;
    const int l = (int)(rb0 / d);
    const int row0 = (int)(rb0 % d) + wv * kFlatRows;
    const bool lora = a.has_shared && a.r > 0;
    if (lora) {
        // a_d = A_down h_shared for this layer, once per block.
        const float *hs = hrow(a, l, a.K);
        for (int i = wv; i < a.r; i += kWaves) {
            const uint16_t *arow = a.la[2] + (int64_t)l * (a.la_ls[2] / 2) + (int64_t)i * f;
            float acc = 0.0f;
            for (int c = lane; c < f; c += kWave) acc += h2f(arow[c]) * hs[c];
            acc = wave_sum(acc);
            if (lane == 0) s_lora[i] = acc;
        }
        __syncthreads();
    }
    const int col0 = gl * 32, g = col0 / kGroup;
    float acc[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) acc[it] = 0.0f;
    const int U = a.K + (a.has_shared ? 1 : 0);
    for (int u = 0; u < U; ++u) {
        int slot;
        if (!resolve_b1(a, l, u, slot, false)) continue;
        const float wk = u < a.K ? a.w[(int64_t)l * a.K + u] : 1.0f;
        const rsrc_t qb = make_rsrc(part_at(part_of(a, u, 6), l, slot), (uint32_t)d * f / 2);
        const rsrc_t sb = make_rsrc(part_at(part_of(a, u, 7), l, slot), (uint32_t)d * fgrp * 2);
        const rsrc_t bb = make_rsrc(part_at(part_of(a, u, 8), l, slot), (uint32_t)d * fgrp * 2);
        u32x4 qv[IT];
        float sv[IT], bv[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const uint32_t row = (uint32_t)(row0 + it * RPI + grp);
            qv[it] = ld128_once(qb, row * (f / 2) + gl * 16);
            sv[it] = h2f(ld16(sb, sb_index(row, (uint32_t)g, (uint32_t)fgrp) * 2));
            bv[it] = h2f(ld16(bb, sb_index(row, (uint32_t)g, (uint32_t)fgrp) * 2));
        }
        const float *hp = hrow(a, l, u) + col0;
        float h[32];
        float hsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(hp + 4 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h[4 * i + j] = v[j];
                hsum += v[j];
            }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) acc[it] += wk * down_dot(qv[it], sv[it], bv[it], h, hsum);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        float v = group_sum(acc[it], LPR);
        const int row = row0 + it * RPI + grp;
        if (lora) {
            const uint16_t *brow = a.lb[2] + (int64_t)l * (a.lb_ls[2] / 2) + (int64_t)row * a.r;
            float dl = 0.0f;
            for (int i = 0; i < a.r; ++i) dl += h2f(brow[i]) * s_lora[i];
            v += a.lscale * dl;
        }
        if (gl == 0) a.y[(int64_t)l * d + row] = v;
    }
}


// ---------------------------------------------------------------------------
// Batch-1 single-launch decode. The work of a call is one list of items, one
// workgroup each, in blockIdx order:
//   lora items     (l)         A_gate x and A_up x of the shared expert's LoRA
//   gate/up items  (l, u, cg)  gate and up rows of 64 hidden units of unit u
//                              (routed expert k = u < K, shared expert u = K):
//                              h = silu(gate x) * up x, published per 16 units
//   down items     (l, rb)     a block of output rows of layer l:
//                              y = sum over units in k order of w_u down_u h_u
// Consumers (down items; shared gate/up items with LoRA) wait for the flags
// of their producers, which precede them in blockIdx order, and a layer's
// down items are placed about one machine's worth of items after its gate/up
// items, so the waits are short; a down item issues its weight loads before
// it waits. One launch streams every weight byte once, with the down
// projections of early layers overlapping the gate/up rows of later ones.
// ---------------------------------------------------------------------------
constexpr int kHalfBlk = 16;     // hidden units per h half block (one flag each)
constexpr int kFuseThreads = 256;
constexpr int kFuseWaves = kFuseThreads / kWave;
constexpr int kBlk = 36;  // dwords per h block: 16 hi pairs, 16 lo pairs, the sum of each half (+ pad)
constexpr int kBlkSum = 32;
constexpr int kChainSplit = 2;  // wavefronts per h half block in chained gate/up items
constexpr int kChainD = 2048;   // d_model of chained calls (one 32-input slice per lane)

constexpr int kLoraJobs = 2 * kFuseWaves;          // dot products per lora item (two per wavefront)
constexpr int kMaxLoraParts = 2 * kMaxR / kLoraJobs;  // lora items (and flags) per layer at most

E0_DEV uint64_t *gu_flags(const DecodeArgs &a, int l) {
    return a.flags + (int64_t)a.L * kMaxLoraParts + (int64_t)l * a.units * a.nch;
}

// h block of (layer l, unit u, 32-column group g): the down input h[32g ..
// 32g + 32) in the form the down dot product takes (see dot_word_m2).
E0_DEV uint32_t *hblk(const DecodeArgs &a, int l, int u, int g) {
    return a.hblk + (((int64_t)l * a.units + u) * (a.f / 32) + g) * kBlk;
}

// Partial sums of the shared expert's LoRA A_down h of layer l: [nch][r], entry
// (hb, i) = sum over the 16 hidden units of half block hb of A_down[i][unit] h[unit],
// published by that half block's gate/up wavefront (in the layer's h rows of the
// workspace, which this path does not otherwise use: nch * r <= (K + 1) * d_ff).
E0_DEV float *lpart(const DecodeArgs &a, int l) { return hrow(a, l, 0); }

// sum over i < r of b[i] * v[i], b fp16 and v fp32, both in LDS; 16-byte steps
// when r is a multiple of 8 (b and v 16-byte aligned), else one at a time.
E0_DEV float lds_dot_r(const uint16_t *b, const float *v, int r) {
    float acc = 0.0f;
    if ((r & 7) == 0) {
        for (int i = 0; i < r; i += 8) {
            const u32x4 bv = *reinterpret_cast<const u32x4 *>(b + i);
            const f32x4 v0 = *reinterpret_cast<const f32x4 *>(v + i);
            const f32x4 v1 = *reinterpret_cast<const f32x4 *>(v + i + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f16x2 b2 = as_h2(bv[q]);
                const float x0 = q < 2 ? v0[2 * q] : v1[2 * q - 4];
                const float x1 = q < 2 ? v0[2 * q + 1] : v1[2 * q - 3];
                acc += (float)b2[0] * x0 + (float)b2[1] * x1;
            }
        }
    } else {
        for (int i = 0; i < r; ++i) acc += h2f(b[i]) * v[i];
    }
    return acc;
}

// Lora item `part` of layer l: dot products part * kLoraJobs + {w, w + 4} of
// the layer's 2r (A_gate x, then A_up x), wavefront w; every load of both is
// issued before either is summed. The single-launch path runs at d_model 2048.
E0_DEV void fused_lora_item(const DecodeArgs &a, int l, int part) {
    constexpr int kC = 2048 / 512;  // 16-byte chunks per lane of a 2048-long row
    const int lane = threadIdx.x & 63, wv = wave_id();
    const uint16_t *xt = a.x + (int64_t)l * a.d;
    u32x4 xv[kC], av[2][kC];
    bool on[2];
    int p[2], i[2];
#pragma unroll
    for (int c = 0; c < kC; ++c) xv[c] = *reinterpret_cast<const u32x4 *>(xt + c * 512 + lane * 8);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int job = part * kLoraJobs + wv + q * kFuseWaves;
        on[q] = job < 2 * a.r;
        p[q] = on[q] ? job / a.r : 0;
        i[q] = on[q] ? job % a.r : 0;
        const uint16_t *arow = a.la[p[q]] + (int64_t)l * (a.la_ls[p[q]] / 2) + (int64_t)i[q] * a.d;
#pragma unroll
        for (int c = 0; c < kC; ++c) av[q][c] = *reinterpret_cast<const u32x4 *>(arow + c * 512 + lane * 8);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < kC; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_fdot2(as_h2(av[q][c][j]), as_h2(xv[c][j]), acc, false);
        acc = wave_sum(acc);
        if (on[q] && lane == 0) coherent_store(a.lora_a + ((int64_t)l * 3 + p[q]) * a.r + i[q], acc);
    }
    signal_ready(a.flags + (int64_t)l * kMaxLoraParts + part, a.epoch);
}

// Chained decode: the fp16 input slice of this lane (inputs 32 lane .. +31)
// of layer l, x = fp16(r / sqrt(mean(r^2) + eps) * g), r the residual after
// layer l - 1 (the call's input for layer 0). Waits (whole workgroup) for the
// down items of layer l - 1, which publish the residual.
E0_DEV void chain_input(const DecodeArgs &a, int l, u32x4 (&xr)[4], float *s_r) {
    const int lane = threadIdx.x & 63;
    const int d = a.d;
    u32x4 gv[4];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd)
        gv[wd] = *reinterpret_cast<const u32x4 *>(a.norm_w + (int64_t)l * d + lane * 32 + wd * 8);
    float rv[32];
    if (l == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(a.r_in + lane * 32 + 4 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) rv[4 * i + j] = v[j];
        }
    } else {
        if (!wait_ready(a.dflags + (int64_t)(l - 1) * a.n_dn, a.n_dn, a.epoch) && threadIdx.x == 0)
            set_err(a.err, E0_DEV_SYNC_TIMEOUT);
        // The residual is read once per workgroup (device-coherent loads, 32
        // bytes per thread) and shared through LDS: every wavefront of every
        // item reading all of it made a queue at the same lines.
        constexpr int kPer = kChainD / 2 / kFuseThreads;
        const uint64_t *src = reinterpret_cast<const uint64_t *>(a.r_out + (int64_t)(l - 1) * d);
        uint64_t t[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) t[i] = coherent_load(src + threadIdx.x + i * kFuseThreads);
#pragma unroll
        for (int i = 0; i < kPer; ++i) reinterpret_cast<uint64_t *>(s_r)[threadIdx.x + i * kFuseThreads] = t[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(s_r + lane * 32 + 4 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) rv[4 * i + j] = v[j];
        }
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) ss += rv[i] * rv[i];
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)d + a.norm_eps);
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f16x2 g2 = as_h2(gv[wd][j]);
            const f16 x0 = (f16)(rv[8 * wd + 2 * j] * inv * (float)g2[0]);
            const f16 x1 = (f16)(rv[8 * wd + 2 * j + 1] * inv * (float)g2[1]);
            xr[wd][j] = (uint32_t)__builtin_bit_cast(uint16_t, x0) | ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16);
        }
    }
}

// Slot of routed expert k of layer l (batch 1), or -1 with the reason in
// `bits` (E0_DEV_BAD_ID / E0_DEV_NOT_RESIDENT). The result is wave-uniform.
E0_DEV int routed_slot(const DecodeArgs &a, int l, int k, int &bits) {
    const int e = cload(a.idx, (int64_t)l * a.K + k);
    const int slot = cload(a.slot_of, (int64_t)l * a.E + min(max(e, 0), a.E - 1));
    bits = (e < 0 || e >= a.E) ? E0_DEV_BAD_ID : (slot < 0 || slot >= a.S) ? E0_DEV_NOT_RESIDENT : 0;
    return __builtin_amdgcn_readfirstlane(bits ? -1 : slot);
}

// Gate/up rows of unit u (SHARED: the shared expert, else routed expert u).
// Item cg covers hidden units 64cg .. 64cg + 64; wavefront w owns half hf =
// w % 2 of h block c = 2cg + w / 2, i.e. the gate and up rows of 16 hidden
// units, streamed in 4 batches of 4 units with the loads of the next batch in
// flight while one is computed. It publishes its half block with its own
// flag, so the wavefronts of an item never wait on each other. Chained items
// cover 32 hidden units: wavefronts 2j and 2j + 1 take 8 units each of half
// block 2cg + j (both batches requested before the wait), meet in LDS, and
// the first publishes the half block.
template <int NP, bool SHARED, bool CHAIN = false>
E0_DEV void fused_gateup_item(const DecodeArgs &a, int l, int u, int cg, float *s_small, float *s_r = nullptr,
                              uint16_t *s_lb = nullptr) {
    // Chained items: kChainSplit wavefronts share a half block (the wait for
    // the previous layer puts every batch on the critical path, so each
    // wavefront computes fewer of them).
    constexpr int kWph = CHAIN ? kChainSplit : 1;         // wavefronts per half block
    constexpr int kUnitsW = kHalfBlk / kWph;              // hidden units per wavefront
    constexpr int NBT = kUnitsW / kFlatBatch;             // batches per wavefront
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int hb = cg * (kFuseWaves / kWph) + wv / kWph;  // half block of the unit
    const int sub = wv % kWph;
    const int c = hb / 2, hf = hb % 2;
    const int d = a.d, ngrp = d / kGroup;
    const int row0 = c * 32 + hf * 16 + sub * kUnitsW;
    float *s_av = s_small;                                 // [2r] LoRA A x
    float *s_hv = s_small + 2 * kMaxR + (wv / kWph) * 16;  // the half block's 16 h values
    // Prologue: the kernel arguments in one batch, the slot, the weight loads
    // of the first two batches, then the loads of x (in-order load counters:
    // x issued earlier would put its latency in front of the weight loads).
    const Part *parts = SHARED ? a.sh.p : a.pool.p;
    const char *base[6];
    int64_t sstride[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        base[i] = parts[i].ptr + (int64_t)l * parts[i].layer_stride;
        sstride[i] = parts[i].slot_stride;
    }
    __asm__ __volatile__("" ::"s"(base[0]), "s"(base[1]), "s"(base[2]), "s"(base[3]),
                         "s"(base[4]), "s"(base[5]), "s"(sstride[0]), "s"(sstride[1]), "s"(sstride[2]),
                         "s"(sstride[3]), "s"(sstride[4]), "s"(sstride[5]));
    int bits = 0;
    const int slot = SHARED ? 0 : routed_slot(a, l, u, bits);
    if (bits && cg == 0 && threadIdx.x == 0) set_err(a.err, bits);
    const bool lora = SHARED && a.r > 0;
    // LoRA rows of this wavefront's 16 hidden units (shared expert): B_gate and
    // B_up rows in LDS, and A_down's 16 columns of them in registers (lane i < r
    // holds row i) for the partial A_down h this half block publishes.
    uint16_t *s_lbw = s_lb ? s_lb + wv * 2 * kHalfBlk * kMaxR : nullptr;
    u32x4 adn[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    if (slot >= 0) {
        rsrc_t qr[2], sr[2], br[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            qr[m] = make_rsrc(base[3 * m] + slot * sstride[3 * m], (uint32_t)a.f * d / 2);
            sr[m] = make_rsrc(base[3 * m + 1] + slot * sstride[3 * m + 1], (uint32_t)a.f * ngrp * 2);
            br[m] = make_rsrc(base[3 * m + 2] + slot * sstride[3 * m + 2], (uint32_t)a.f * ngrp * 2);
        }
        // One batch: rows r0 .. r0 + 3 of gate and up. Scales and biases are
        // stored in 8-row tiles, so the lane's 4 rows of one group are 8
        // contiguous bytes, and the lanes of a load cover whole tiles.
        struct Stage {
            u32x4 q[kFlatBatch][2][NP];
            uint32_t sc[2][NP][2], bi[2][NP][2];
        };
        auto load = [&](int bt, Stage &S) {
            const uint32_t r0 = (uint32_t)(row0 + bt * kFlatBatch);
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int np = 0; np < NP; ++np) {
                    const uint32_t col = (uint32_t)(np * 64 + lane);
#pragma unroll
                    for (int rr = 0; rr < kFlatBatch; ++rr) S.q[rr][m][np] = ld128_once(qr[m], (r0 + rr) * (d / 2) + col * 16);
                    const uint32_t so = sb_index(r0, col / 2, (uint32_t)ngrp) * 2;  // 4 rows inside one 8-row tile
                    const auto sv = __builtin_amdgcn_raw_buffer_load_b64(sr[m], (int)so, 0, 0);
                    const auto bv = __builtin_amdgcn_raw_buffer_load_b64(br[m], (int)so, 0, 0);
                    S.sc[m][np][0] = sv[0];
                    S.sc[m][np][1] = sv[1];
                    S.bi[m][np][0] = bv[0];
                    S.bi[m][np][1] = bv[1];
                }
            }
        };
        Stage A, B;
        load(0, A);
        load(1, B);
        if (lora) {
            // After the first weight loads: the LoRA rows, then the wait for
            // this layer's A x (its lora item) by the whole workgroup.
            constexpr int kLbMax = 2 * kHalfBlk * kMaxR / kWave;
            const int nlb = 2 * kHalfBlk * a.r;
            uint16_t lbv[kLbMax];
#pragma unroll
            for (int j = 0; j < kLbMax; ++j) {
                const int i = lane + j * kWave;
                const int m = i / (kHalfBlk * a.r), rem = i % (kHalfBlk * a.r);
                lbv[j] = i < nlb ? a.lb[m][(int64_t)l * (a.lb_ls[m] / 2) + (int64_t)row0 * a.r + rem] : (uint16_t)0;
            }
            if (lane < a.r) {
                const u32x4 *ap = reinterpret_cast<const u32x4 *>(a.la[2] + (int64_t)l * (a.la_ls[2] / 2) +
                                                                  (int64_t)lane * a.f + row0);
                adn[0] = ap[0];
                adn[1] = ap[1];
            }
#pragma unroll
            for (int j = 0; j < kLbMax; ++j)
                if (lane + j * kWave < nlb) s_lbw[lane + j * kWave] = lbv[j];
            if (!wait_ready(a.flags + (int64_t)l * kMaxLoraParts, a.lora_parts, a.epoch) && threadIdx.x == 0)
                set_err(a.err, E0_DEV_SYNC_TIMEOUT);
            if (threadIdx.x < 2 * a.r) s_av[threadIdx.x] = coherent_load(a.lora_a + (int64_t)l * 3 * a.r + threadIdx.x);
            __syncthreads();
        }
        u32x4 xr[NP][4];
        if constexpr (CHAIN) {
            // Chained: every batch's weights are requested before the wait for
            // the previous layer, so none of them is on the critical path.
            static_assert(NP == 1 && !SHARED && NBT == 2, "chained items: d_model 2048, routed experts");
            chain_input(a, l, xr[0], s_r);
        } else {
#pragma unroll
            for (int np = 0; np < NP; ++np)
#pragma unroll
                for (int wd = 0; wd < 4; ++wd)
                    xr[np][wd] = *reinterpret_cast<const u32x4 *>(a.x + (int64_t)l * d + (np * 64 + lane) * 32 + wd * 8);
        }
        uint32_t xp[NP][4][4];
        float xs[NP];
#pragma unroll
        for (int np = 0; np < NP; ++np) {
            xs[np] = 0.0f;
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) x_pairs_m(xr[np][wd], xp[np][wd], xs[np]);
        }
        auto compute = [&](int bt, const Stage &S) {
            float acc[2 * kFlatBatch];
#pragma unroll
            for (int rr = 0; rr < kFlatBatch; ++rr) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    float v = 0.0f;
#pragma unroll
                    for (int np = 0; np < NP; ++np) {
                        float dacc = 0.0f;
#pragma unroll
                        for (int wd = 0; wd < 4; ++wd) dacc = dot_word_m(S.q[rr][m][np][wd], xp[np][wd], dacc);
                        const float sc = (float)as_h2(S.sc[m][np][rr / 2])[rr % 2];
                        const float bi = (float)as_h2(S.bi[m][np][rr / 2])[rr % 2];
                        v += (sc * kDenormScale) * dacc + bi * xs[np];
                    }
                    acc[m * kFlatBatch + rr] = v;
                }
            }
            // 2*kFlatBatch values over 64 lanes: gate values in lanes 0..31,
            // the matching up value in lane ^ 32.
            group_reduce_scatter<2 * kFlatBatch, kWave>(acc);
            constexpr int DUP = kWave / (2 * kFlatBatch);
            const int vi = lane / DUP, m = vi / kFlatBatch, rr = vi % kFlatBatch;
            const int row = row0 + bt * kFlatBatch + rr;
            float val = acc[0];
            if (lora) val += a.lscale * lds_dot_r(s_lbw + (m * kHalfBlk + (row - row0)) * a.r, s_av + m * a.r, a.r);
            const float other = __shfl_xor(val, 32);
            if (m == 0 && lane % DUP == 0) s_hv[sub * kUnitsW + bt * kFlatBatch + rr] = silu(val) * other;
        };
        if constexpr (CHAIN) {
            compute(0, A);
            compute(1, B);
        } else {
            // Two-stage pipeline; the empty asm statements keep the compiler from
            // hoisting later batches' loads (register pressure) or sinking them.
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) {
                __asm__ __volatile__("" ::: "memory");
                if (bt & 1) {
                    compute(bt, B);
                    __asm__ __volatile__("" ::: "memory");
                    if (bt + 2 < NBT) load(bt + 2, B);
                } else {
                    compute(bt, A);
                    __asm__ __volatile__("" ::: "memory");
                    if (bt + 2 < NBT) load(bt + 2, A);
                }
            }
        }
    } else if (lane < kUnitsW) {
        s_hv[sub * kUnitsW + lane] = 0.0f;
    }
    if constexpr (CHAIN) {
        // The wavefronts of a half block meet in LDS; the first one publishes.
        __syncthreads();
        if (sub) return;
    } else {
        wave_lds_sync();
    }
    // This wavefront's half of the h block: hi/lo fp16 pairs of h with the
    // odd pairs scaled by 1/16 (the form dot_word_m2 takes), and the half's sum.
    if (lora && lane < a.r) {
        // This half block's share of A_down h (its 16 hidden units, in order).
        float p = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f16x2 a2 = as_h2(adn[j][q]);
                p += (float)a2[0] * s_hv[8 * j + 2 * q] + (float)a2[1] * s_hv[8 * j + 2 * q + 1];
            }
        coherent_store(lpart(a, l) + (int64_t)(2 * c + hf) * a.r + lane, p);
    }
    {
        const int t = lane & 15;
        const float v = s_hv[t];
        const int tb = hf * 16 + t;  // element of the block
        const int p = tb % 8, j = p % 4;
        const float hv = (j & 1) ? v * 0.0625f : v;
        const f16 hi = (f16)hv;
        const f16 lo = (f16)(hv - (float)hi);
        // pair dword (t/8)*4 + j, half p/4: gather the two halves of each dword
        const uint32_t hbits = __builtin_bit_cast(uint16_t, hi), lbits = __builtin_bit_cast(uint16_t, lo);
        const uint32_t hpart = __shfl_xor((int)hbits, 4), lpart = __shfl_xor((int)lbits, 4);
        float se = (j & 1) ? 0.0f : v, so = (j & 1) ? v : 0.0f;
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) {
            se += __shfl_xor(se, o);
            so += __shfl_xor(so, o);
        }
        uint32_t *blk = hblk(a, l, u, c);
        if (lane < 16 && p < 4) {
            const int dw = (tb / 8) * 4 + j;
            __hip_atomic_store(blk + dw, hbits | (hpart << 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(blk + 16 + dw, lbits | (lpart << 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == 0) coherent_store(reinterpret_cast<float *>(blk + kBlkSum + 2 * hf), se + so);
    }
    // This wavefront's stores complete, then its flag.
    __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0)
        __hip_atomic_store(gu_flags(a, l) + (int64_t)u * a.nch + 2 * c + hf, a.epoch, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Down rows: LPR lanes per row (d_ff = 32 * LPR), KM routed units at most
// plus the shared expert, RW output rows per wavefront (kFuseWaves * RW per item).
template <int LPR, int KM, int RW, bool CHAIN = false>
E0_DEV void fused_down_item(const DecodeArgs &a, int l, int rb, uint32_t *s_hb, float *s_part, float *s_lora,
                            uint16_t *s_lbd) {
    constexpr int RPI = kWave / LPR;  // rows per load instruction
    constexpr int IT = RW / RPI;      // load instructions per unit
    static_assert(IT >= 1, "RW >= rows per load instruction");
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int gl = lane % LPR, grp = lane / LPR;
    const int f = a.f, d = a.d, fgrp = f / kGroup;
    const int K = a.K;
    const int row0 = rb * (kFuseWaves * RW) + wv * RW;

    // 1. Slots of every routed unit, then every weight load, before the wait.
    //    The id, weight and slot-table reads are unconditional (indices
    //    clamped into range, invalid results masked afterwards), so they go
    //    out as two batches of scalar loads rather than one at a time.
    int e[KM], slot[KM];
    float wk[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        const int kk = k < K ? k : K - 1;
        e[k] = cload(a.idx, (int64_t)l * K + kk);
        wk[k] = k < K ? cload(a.w, (int64_t)l * K + kk) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        const bool ok = k < K && e[k] >= 0 && e[k] < a.E;
        const int sl = cload(a.slot_of, (int64_t)l * a.E + min(max(e[k], 0), a.E - 1));
        slot[k] = __builtin_amdgcn_readfirstlane((ok && sl >= 0 && sl < a.S) ? sl : -1);
    }
    // Loads are issued without branches (a branch around a load makes the
    // compiler wait for it at the join): a unit that does not exist or has
    // no valid slot reads through a zero-size buffer descriptor, which returns
    // zeros without touching memory, and contributes nothing. Lane group grp
    // owns IT consecutive rows inside one 8-row tile, so its scales (and biases) are
    // 2 * IT contiguous bytes.
    static_assert(IT == 2 || IT == 4 || IT == 8, "scale loads of 4, 8 or 16 bytes");
    u32x4 q[KM + 1][IT];
    uint32_t sv[KM + 1][IT / 2], bv[KM + 1][IT / 2];
    auto load_halves = [&](const rsrc_t &r, uint32_t off, uint32_t (&o)[IT / 2]) {
        if constexpr (IT == 2) {
            o[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
        } else if constexpr (IT == 4) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
            o[0] = v[0];
            o[1] = v[1];
        } else {
            const u32x4 v = ld128_once(r, off);
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = v[j];
        }
    };
    const int rows0 = row0 + grp * IT;  // this lane group's first row
    auto load_unit = [&](int u, const Part &pq, const Part &ps, const Part &pb, int sl, bool on) {
        const int s0 = on ? sl : 0;
        const rsrc_t qb = make_rsrc(part_at(pq, l, s0), on ? (uint32_t)d * f / 2 : 0u);
        const rsrc_t sb = make_rsrc(part_at(ps, l, s0), on ? (uint32_t)d * fgrp * 2 : 0u);
        const rsrc_t bb = make_rsrc(part_at(pb, l, s0), on ? (uint32_t)d * fgrp * 2 : 0u);
#pragma unroll
        for (int it = 0; it < IT; ++it) q[u][it] = ld128_once(qb, (uint32_t)(rows0 + it) * (f / 2) + gl * 16);
        const uint32_t so = sb_index((uint32_t)rows0, (uint32_t)(gl / 2), (uint32_t)fgrp) * 2;  // IT rows in one tile
        load_halves(sb, so, sv[u]);
        load_halves(bb, so, bv[u]);
    };
#pragma unroll
    for (int k = 0; k < KM; ++k) load_unit(k, a.pool.p[6], a.pool.p[7], a.pool.p[8], slot[k], slot[k] >= 0);
    load_unit(KM, a.sh.p[6], a.sh.p[7], a.sh.p[8], 0, a.has_shared != 0);
    // The shared expert's LoRA: B_down rows of this item's output rows, to LDS
    // before the wait.
    const bool lora = a.has_shared && a.r > 0;
    if (lora) {
        const int item_rows = kFuseWaves * RW, row_base = rb * item_rows;
        const int n = item_rows * a.r;
        const uint16_t *src = a.lb[2] + (int64_t)l * (a.lb_ls[2] / 2) + (int64_t)row_base * a.r;
        constexpr int kMaxLb = (kFuseWaves * RW * kMaxR + kFuseThreads - 1) / kFuseThreads;
        uint16_t t[kMaxLb];
#pragma unroll
        for (int j = 0; j < kMaxLb; ++j) {
            const int i = threadIdx.x + j * kFuseThreads;
            t[j] = i < n ? src[i] : (uint16_t)0;
        }
#pragma unroll
        for (int j = 0; j < kMaxLb; ++j) {
            const int i = threadIdx.x + j * kFuseThreads;
            if (i < n) s_lbd[i] = t[j];
        }
    }

    // 2. Wait for the layer's gate/up items, then stage its h blocks (and the
    //    shared expert's fp32 h for the LoRA term).
    if (!wait_ready(gu_flags(a, l), a.units * a.nch, a.epoch) && threadIdx.x == 0) set_err(a.err, E0_DEV_SYNC_TIMEOUT);
    const int U = a.units;
    {
        // All staging loads in flight at once, then the LDS writes.
        constexpr int kMaxStage = ((KM + 1) * LPR * (kBlk / 2) + kFuseThreads - 1) / kFuseThreads;
        const int n = U * LPR * (kBlk / 2);
        const uint64_t *src = reinterpret_cast<const uint64_t *>(hblk(a, l, 0, 0));
        uint64_t tmp[kMaxStage];
#pragma unroll
        for (int j = 0; j < kMaxStage; ++j) {
            const int i = threadIdx.x + j * kFuseThreads;
            tmp[j] = i < n ? coherent_load(src + i) : 0;
        }
#pragma unroll
        for (int j = 0; j < kMaxStage; ++j) {
            const int i = threadIdx.x + j * kFuseThreads;
            if (i < n) reinterpret_cast<uint64_t *>(s_hb)[i] = tmp[j];
        }
    }
    if (lora) {
        // The partial A_down h of every half block of the shared expert.
        const int n = a.nch * a.r;
        const float *src = lpart(a, l);
        for (int i = threadIdx.x; i < n; i += kFuseThreads) s_part[i] = coherent_load(src + i);
    }
    // Chained: the residual rows this lane group adds to, requested with the
    // staging loads (layer l - 1 finished before any gate/up item of l ran).
    float rprev[IT];
    if constexpr (CHAIN) {
#pragma unroll
        for (int it = 0; it < IT; ++it)
            rprev[it] = l == 0 ? a.r_in[rows0 + it] : coherent_load(a.r_out + (int64_t)(l - 1) * d + rows0 + it);
    }
    __syncthreads();
    if (lora) {
        // A_down h_shared: the half blocks' partials summed in order.
        if (threadIdx.x < a.r) {
            float acc = 0.0f;
            for (int hb = 0; hb < a.nch; ++hb) acc += s_part[hb * a.r + threadIdx.x];
            s_lora[threadIdx.x] = acc;
        }
        __syncthreads();
    }
    // 3. y rows: routed units in k order, then the shared expert (weight 1).
    float acc[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) acc[it] = 0.0f;
    auto add_unit = [&](int u, int hu, float wk) {
        uint32_t hh[16], hlo[16];
        const uint32_t *blk = s_hb + (hu * LPR + gl) * kBlk;
        const u32x4 *b4 = reinterpret_cast<const u32x4 *>(blk);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 v = b4[i], w2 = b4[4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hh[4 * i + j] = v[j];
                hlo[4 * i + j] = w2[j];
            }
        }
        const float hsum = __builtin_bit_cast(float, blk[kBlkSum]) + __builtin_bit_cast(float, blk[kBlkSum + 2]);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            float dacc = 0.0f;
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) dacc = dot_word_m2(q[u][it][wd], hh + 4 * wd, hlo + 4 * wd, dacc);
            const float sc = (float)as_h2(sv[u][it / 2])[it % 2], bi = (float)as_h2(bv[u][it / 2])[it % 2];
            acc[it] += wk * ((sc * kDenormScale) * dacc + bi * hsum);
        }
    };
#pragma unroll
    for (int k = 0; k < KM; ++k)
        if (slot[k] >= 0) add_unit(k, k, wk[k]);
    if (a.has_shared) add_unit(KM, K, 1.0f);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        float v = group_sum(acc[it], LPR);
        const int row = rows0 + it;
        if (lora) v += a.lscale * lds_dot_r(s_lbd + (row - rb * (kFuseWaves * RW)) * a.r, s_lora, a.r);
        if (gl == 0) {
            a.y[(int64_t)l * d + row] = v;
            if constexpr (CHAIN) coherent_store(a.r_out + (int64_t)l * d + row, rprev[it] + v);
        }
    }
    if constexpr (CHAIN) signal_ready(a.dflags + (int64_t)l * a.n_dn + rb, a.epoch);
}

template <int NP, int LPR, int KM, int RW, bool CHAIN = false>
__global__ __launch_bounds__(kFuseThreads) void decode_fused_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t s_hb[(KM + 1) * LPR * kBlk];
    __shared__ float s_part[2 * LPR * kMaxR];  // LoRA partials: d_ff / 16 half blocks x r
    __shared__ __attribute__((aligned(16))) float s_small[2 * kMaxR + kFuseWaves * 16];
    __shared__ __attribute__((aligned(16))) uint16_t s_lb[CHAIN ? 2 : kFuseWaves * (RW > 2 * kHalfBlk ? RW : 2 * kHalfBlk) * kMaxR];
    __shared__ __attribute__((aligned(16))) float s_rr[CHAIN ? kChainD : 4];  // chained: the layer's input residual
    // Item order: the lora items, then steps s = 0 .. L + lag - 1, step s
    // holding the gate/up items of layer s (s < L) followed by the down items
    // of layer s - lag (s >= lag). Every down item comes after all gate/up
    // items of its layer, and by the time it is dispatched they have had
    // about a machine's worth of other items to finish in.
    int item = blockIdx.x;
    if (item < a.n_lora) {
        fused_lora_item(a, item / a.lora_parts, item % a.lora_parts);
        return;
    }
    item -= a.n_lora;
    const int n1 = a.n_gu, n2 = a.n_dn, lag = a.lag, L = a.L;
    int l, r, gu;
    if (item < lag * n1) {
        gu = 1;
        l = item / n1;
        r = item % n1;
    } else if ((item -= lag * n1) < (L - lag) * (n1 + n2)) {
        const int st = item / (n1 + n2);
        r = item % (n1 + n2);
        gu = r < n1;
        l = gu ? lag + st : st;
        if (!gu) r -= n1;
    } else {
        item -= (L - lag) * (n1 + n2);
        gu = 0;
        l = L - lag + item / n2;
        r = item % n2;
    }
    if (gu) {
        const int per_u = a.nch / (CHAIN ? kFuseWaves / kChainSplit : kFuseWaves);  // items per unit
        const int u = r / per_u, cg = r % per_u;
        if constexpr (CHAIN)
            fused_gateup_item<NP, false, true>(a, l, u, cg, s_small, s_rr);
        else if (u < a.K)
            fused_gateup_item<NP, false>(a, l, u, cg, s_small);
        else
            fused_gateup_item<NP, true>(a, l, u, cg, s_small, nullptr, s_lb);
    } else {
        fused_down_item<LPR, KM, RW, CHAIN>(a, l, r, s_hb, s_part, s_small, s_lb);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// Supported d_model: 256 .. 2048 powers of two, or multiples of 2048 up to 8192.
int d_lpr(int d, int &np) {
    if (d >= 256 && d <= 2048 && pow2(d)) {
        np = 1;
        return d / 32;
    }
    if (d > 2048 && d % 2048 == 0 && d <= 8192) {
        np = d / 2048;
        return 64;
    }
    return 0;
}

// Supported d_ff: 128 .. 2048 powers of two.
int f_lpr(int f) { return (f >= 128 && f <= 2048 && pow2(f)) ? f / 32 : 0; }

struct Layout {
    size_t ucnt, uexp, uslot, uoff, pairs, pslot, pwt, hbuf, lora, flags, hblk, dflags, total;
};

// Output rows per wavefront of a down item of the single-launch kernel: at
// least two load instructions per unit, so its scales are one 4/8/16-byte load.
int fused_rows_per_wave(int K, int lpr_f) { return (K <= 4 || lpr_f == 8) ? 16 : 8; }

// Chained calls: each down item waits for its layer, so its compute is on the
// critical path; with d_ff 512 a wavefront takes 8 output rows (twice the
// items per layer, half the work after the wait).
int chain_rows_per_wave(int K, int lpr_f) { return lpr_f == 16 ? 8 : fused_rows_per_wave(K, lpr_f); }

// n_dn: down items per layer of a chained call (their ready flags), else 0.
Layout decode_layout(int L, int B, int K, int E, int f, int r, int n_dn = 0) {
    Layout o;
    const int umax = B == 1 ? K : (E < B * K ? E : B * K);
    size_t off = 0;
    o.ucnt = off;
    off = e0_align(off + sizeof(int32_t) * L);
    o.uexp = off;
    off = e0_align(off + sizeof(int32_t) * (size_t)L * umax);
    o.uslot = off;
    off = e0_align(off + sizeof(int32_t) * (size_t)L * umax);
    o.uoff = off;
    off = e0_align(off + sizeof(int32_t) * (size_t)L * (umax + 1));
    o.pairs = off;
    off = e0_align(off + sizeof(int32_t) * (size_t)L * B * K);
    o.pslot = off;
    off = e0_align(off + sizeof(int32_t) * (size_t)L * B * K);
    o.pwt = off;
    off = e0_align(off + sizeof(float) * (size_t)L * B * K);
    o.hbuf = off;
    off = e0_align(off + sizeof(float) * (size_t)L * (B * K + B) * f);
    o.lora = off;
    off = e0_align(off + sizeof(float) * (size_t)L * B * 3 * (r > 0 ? r : 1));
    o.flags = off;
    off = e0_align(off + (B == 1 ? sizeof(uint64_t) * (size_t)L * (kMaxLoraParts + (K + 1) * (size_t)(f / kHalfBlk)) : 0));
    o.hblk = off;
    off = e0_align(off + (B == 1 ? sizeof(uint32_t) * (size_t)L * (K + 1) * (size_t)(f / 32) * kBlk : 0));
    o.dflags = off;
    off = e0_align(off + sizeof(uint64_t) * (size_t)L * n_dn);
    o.total = off;
    return o;
}

template <int LPR, int NP, int TC, int RB, int G>
void launch_gateup(const DecodeArgs &a, dim3 grid, hipStream_t st) {
    hipLaunchKernelGGL((decode_gateup_kernel<LPR, NP, TC, RB, G>), grid, dim3(kThreads), 0, st, a);
}

template <int TC, int RB, int G>
bool dispatch_gateup(int lpr, int np, const DecodeArgs &a, dim3 grid, hipStream_t st) {
    switch (lpr * 8 + np) {
        case 8 * 8 + 1: launch_gateup<8, 1, TC, RB, G>(a, grid, st); return true;
        case 16 * 8 + 1: launch_gateup<16, 1, TC, RB, G>(a, grid, st); return true;
        case 32 * 8 + 1: launch_gateup<32, 1, TC, RB, G>(a, grid, st); return true;
        case 64 * 8 + 1: launch_gateup<64, 1, TC, RB, G>(a, grid, st); return true;
        case 64 * 8 + 2: launch_gateup<64, 2, TC, RB, G>(a, grid, st); return true;
        case 64 * 8 + 3: launch_gateup<64, 3, TC, RB, G>(a, grid, st); return true;
        case 64 * 8 + 4: launch_gateup<64, 4, TC, RB, G>(a, grid, st); return true;
        default: return false;
    }
}

template <int TC, int RB>
int gateup_rows_per_block(int lpr) {
    return (kWave / lpr) * RB * kWaves;
}

bool dispatch_down(int lpr, const DecodeArgs &a, dim3 grid, hipStream_t st) {
    switch (lpr) {
        case 4: hipLaunchKernelGGL(decode_down_kernel<4>, grid, dim3(kThreads), 0, st, a); return true;
        case 8: hipLaunchKernelGGL(decode_down_kernel<8>, grid, dim3(kThreads), 0, st, a); return true;
        case 16: hipLaunchKernelGGL(decode_down_kernel<16>, grid, dim3(kThreads), 0, st, a); return true;
        case 32: hipLaunchKernelGGL(decode_down_kernel<32>, grid, dim3(kThreads), 0, st, a); return true;
        case 64: hipLaunchKernelGGL(decode_down_kernel<64>, grid, dim3(kThreads), 0, st, a); return true;
        default: return false;
    }
}

void launch_fused(const DecodeArgs &a, int lpr_f, bool small, dim3 grid, hipStream_t st) {
    if (a.chain) {
        switch (lpr_f) {
            case 8:
                if (small) hipLaunchKernelGGL((decode_fused_kernel<1, 8, 4, 16, true>), grid, dim3(kFuseThreads), 0, st, a);
                else hipLaunchKernelGGL((decode_fused_kernel<1, 8, 8, 16, true>), grid, dim3(kFuseThreads), 0, st, a);
                break;
            case 16:
                if (small) hipLaunchKernelGGL((decode_fused_kernel<1, 16, 4, 8, true>), grid, dim3(kFuseThreads), 0, st, a);
                else hipLaunchKernelGGL((decode_fused_kernel<1, 16, 8, 8, true>), grid, dim3(kFuseThreads), 0, st, a);
                break;
            default:
                hipLaunchKernelGGL((decode_fused_kernel<1, 32, 4, 16, true>), grid, dim3(kFuseThreads), 0, st, a);
                break;
        }
        return;
    }
    switch (lpr_f) {
        case 8:
            if (small) hipLaunchKernelGGL((decode_fused_kernel<1, 8, 4, 16>), grid, dim3(kFuseThreads), 0, st, a);
            else hipLaunchKernelGGL((decode_fused_kernel<1, 8, 8, 16>), grid, dim3(kFuseThreads), 0, st, a);
            break;
        case 16:
            if (small) hipLaunchKernelGGL((decode_fused_kernel<1, 16, 4, 16>), grid, dim3(kFuseThreads), 0, st, a);
            else hipLaunchKernelGGL((decode_fused_kernel<1, 16, 8, 8>), grid, dim3(kFuseThreads), 0, st, a);
            break;
        default:
            hipLaunchKernelGGL((decode_fused_kernel<1, 32, 4, 16>), grid, dim3(kFuseThreads), 0, st, a);
            break;
    }
}

// Shapes the single-launch batch-1 kernel takes: d_model 2048 and the listed
// d_ff / top-K combinations.
bool fused_shape_ok(int d, int f, int K) {
    int np = 0;
    const int lpr_d = d_lpr(d, np), lpr_f = f_lpr(f);
    return lpr_d == 64 && np == 1 && (lpr_f == 8 || lpr_f == 16 || (lpr_f == 32 && K <= 4)) && K <= 8 &&
           f % (kHalfBlk * kFuseWaves) == 0;
}

bool stack_ok(const e0_stack *s, int first, int last) {
    for (int i = first; i <= last; ++i) {
        const e0_part &p = s->part[i];
        if (!p.ptr) return false;
        if ((reinterpret_cast<uintptr_t>(p.ptr) | (uintptr_t)p.slot_stride | (uintptr_t)p.layer_stride) & 15)
            return false;
    }
    return true;
}

}  // namespace

size_t e0_decode_workspace_bytes(const e0_moe_dims *dims, int32_t L, int32_t B, int32_t r) {
    if (!dims || L < 0 || B < 1) return 0;
    return decode_layout(L, B, dims->top_k, dims->n_experts, dims->d_ff, r).total;
}

extern "C" e0_status e0_moe_staged_decode(const e0_moe_dims *dims, int32_t L, int32_t B, const uint16_t *x,
                                          const int32_t *idx, const float *w, const int32_t *slot_of, int32_t S,
                                          const e0_stack *pool, const e0_shared *shared, float *y, void *ws,
                                          size_t ws_bytes, int32_t *dev_err, void *stream) {
    e0_clear_stale_error();
    E0_REQUIRE(dims && pool, E0_ERR_INVALID_ARG);
    const int d = dims->d_model, f = dims->d_ff, E = dims->n_experts, K = dims->top_k;
    E0_REQUIRE(L >= 0 && B >= 1 && S >= 1 && E >= 1 && K >= 1, E0_ERR_INVALID_ARG);
    E0_REQUIRE(d % 64 == 0 && f % 64 == 0, E0_ERR_UNSUPPORTED_SHAPE);
    int np = 0;
    const int lpr_d = d_lpr(d, np), lpr_f = f_lpr(f);
    E0_REQUIRE(lpr_d && lpr_f, E0_ERR_UNSUPPORTED_SHAPE);
    E0_REQUIRE(K <= kMaxK && K <= E && E <= kMaxE, E0_ERR_UNSUPPORTED_SHAPE);
    E0_REQUIRE(B <= kMaxB, E0_ERR_CAPACITY);
    E0_REQUIRE(x && idx && w && slot_of && y && dev_err, E0_ERR_INVALID_ARG);
    E0_REQUIRE(stack_ok(pool, 0, 8), E0_ERR_INVALID_ARG);
    E0_REQUIRE((reinterpret_cast<uintptr_t>(x) & 15) == 0, E0_ERR_INVALID_ARG);
    int r = 0;
    if (shared) {
        E0_REQUIRE(stack_ok(&shared->w, 0, 8), E0_ERR_INVALID_ARG);
        E0_REQUIRE(shared->d_ff == f, E0_ERR_UNSUPPORTED_SHAPE);
        r = shared->lora_rank;
        E0_REQUIRE(r >= 0 && r <= kMaxR, E0_ERR_UNSUPPORTED_SHAPE);
        if (r > 0) {
            for (int p = 0; p < 3; ++p) {
                E0_REQUIRE(shared->lora_a[p] && shared->lora_b[p], E0_ERR_INVALID_ARG);
                E0_REQUIRE(((reinterpret_cast<uintptr_t>(shared->lora_a[p]) | (uintptr_t)shared->lora_a_layer_stride[p]) & 15) == 0,
                           E0_ERR_INVALID_ARG);
                E0_REQUIRE((shared->lora_b_layer_stride[p] & 1) == 0, E0_ERR_INVALID_ARG);
            }
        }
    }
    const Layout lay = decode_layout(L, B, K, E, f, r);
    E0_REQUIRE(ws && ws_bytes >= lay.total && (reinterpret_cast<uintptr_t>(ws) & 255) == 0, E0_ERR_CAPACITY);
    if (L == 0) return E0_OK;

    DecodeArgs a{};
    a.L = L;
    a.B = B;
    a.K = K;
    a.E = E;
    a.S = S;
    a.d = d;
    a.f = f;
    a.x = x;
    a.idx = idx;
    a.w = w;
    a.slot_of = slot_of;
    a.pool = to_stack(*pool);
    a.has_shared = shared != nullptr;
    if (shared) {
        a.sh = to_stack(shared->w);
        a.r = r;
        a.lscale = shared->lora_scale;
        for (int p = 0; p < 3; ++p) {
            a.la[p] = shared->lora_a[p];
            a.la_ls[p] = shared->lora_a_layer_stride[p];
            a.lb[p] = shared->lora_b[p];
            a.lb_ls[p] = shared->lora_b_layer_stride[p];
        }
    }
    a.y = y;
    a.err = dev_err;
    a.has_plan = B > 1;
    a.umax = B == 1 ? K : (E < B * K ? E : B * K);
    char *wsb = static_cast<char *>(ws);
    a.ucnt = reinterpret_cast<int32_t *>(wsb + lay.ucnt);
    a.uexp = reinterpret_cast<int32_t *>(wsb + lay.uexp);
    a.uslot = reinterpret_cast<int32_t *>(wsb + lay.uslot);
    a.uoff = reinterpret_cast<int32_t *>(wsb + lay.uoff);
    a.pairs = reinterpret_cast<int32_t *>(wsb + lay.pairs);
    a.pslot = reinterpret_cast<int32_t *>(wsb + lay.pslot);
    a.pwt = reinterpret_cast<float *>(wsb + lay.pwt);
    a.hbuf = reinterpret_cast<float *>(wsb + lay.hbuf);
    a.lora_a = reinterpret_cast<float *>(wsb + lay.lora);
    a.flags = reinterpret_cast<uint64_t *>(wsb + lay.flags);
    a.hblk = reinterpret_cast<uint32_t *>(wsb + lay.hblk);

    hipStream_t st = static_cast<hipStream_t>(stream);
    e0_status s;
    const int U = K + (a.has_shared ? 1 : 0);
    if (B == 1 && lpr_d == 64 && np == 1 && (lpr_f == 8 || lpr_f == 16 || (lpr_f == 32 && K <= 4)) && K <= 8 &&
        f % (kHalfBlk * kFuseWaves) == 0) {
        // Batch 1, d_model 2048: the single-launch kernel.
        a.epoch = e0_next_epoch();
        a.units = U;
        a.nch = f / kHalfBlk;
        a.lora_parts = (2 * r + kLoraJobs - 1) / kLoraJobs;
        a.n_lora = (a.has_shared && r > 0) ? L * a.lora_parts : 0;
        const bool small = K <= 4;
        const int rw = fused_rows_per_wave(K, lpr_f);
        const int64_t n_gu = (int64_t)U * (a.nch / kFuseWaves), n_dn = d / (kFuseWaves * rw);  // per layer
        E0_REQUIRE(a.n_lora + L * (n_gu + n_dn) <= (int64_t)INT32_MAX, E0_ERR_CAPACITY);
        a.n_gu = (int)n_gu;
        a.n_dn = (int)n_dn;
        // Lag of the down items: about two machines' worth of resident
        // workgroups (three per compute unit each) between a layer's gate/up
        // items and its down items, so that a down item rarely finds its
        // producers still running (measured: lags of 17 to 40 layers at the
        // 35B shape are within 1 us of each other; 17 leaves down items
        // waiting at the start).
        static int cus = 0;
        if (!cus && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess) cus = 256;
        const int64_t lag = (6 * (int64_t)cus + n_gu + n_dn - 1) / (n_gu + n_dn) + 1;
        a.lag = (int)(lag < L ? lag : L);
        const dim3 grid((unsigned)(a.n_lora + L * (n_gu + n_dn)));
        launch_fused(a, lpr_f, small, grid, st);
        return e0_launch_status();
    }
    if (a.has_plan) {
        hipLaunchKernelGGL(decode_prep_kernel, dim3(L), dim3(kThreads), 0, st, a);
        if ((s = e0_launch_status())) return s;
    }
    if (a.has_shared && r > 0) {
        const int64_t jobs = (int64_t)L * B * 2 * r;
        hipLaunchKernelGGL(decode_lora_kernel, dim3((unsigned)((jobs + kWaves - 1) / kWaves)), dim3(kThreads), 0, st, a);
        if ((s = e0_launch_status())) return s;
    }
    if (B == 1 && lpr_d == 64) {
        // Batch 1 at d_model = 2048 * NP: the flat one-round kernels.
        const int64_t gu_waves = ((int64_t)L * U * f) / kFlatRows;
        const int64_t dn_waves = ((int64_t)L * d) / kFlatRows;
        E0_REQUIRE(gu_waves <= (int64_t)INT32_MAX && dn_waves <= (int64_t)INT32_MAX, E0_ERR_CAPACITY);
        const dim3 gu_grid((unsigned)((gu_waves + kWaves - 1) / kWaves)), dn_grid((unsigned)((dn_waves + kWaves - 1) / kWaves));
        switch (np) {
            case 1: hipLaunchKernelGGL(decode_gateup_flat_kernel<1>, gu_grid, dim3(kThreads), 0, st, a); break;
            case 2: hipLaunchKernelGGL(decode_gateup_flat_kernel<2>, gu_grid, dim3(kThreads), 0, st, a); break;
            case 3: hipLaunchKernelGGL(decode_gateup_flat_kernel<3>, gu_grid, dim3(kThreads), 0, st, a); break;
            default: hipLaunchKernelGGL(decode_gateup_flat_kernel<4>, gu_grid, dim3(kThreads), 0, st, a); break;
        }
        if ((s = e0_launch_status())) return s;
        switch (lpr_f) {
            case 4: hipLaunchKernelGGL(decode_down_flat_kernel<4>, dn_grid, dim3(kThreads), 0, st, a); break;
            case 8: hipLaunchKernelGGL(decode_down_flat_kernel<8>, dn_grid, dim3(kThreads), 0, st, a); break;
            case 16: hipLaunchKernelGGL(decode_down_flat_kernel<16>, dn_grid, dim3(kThreads), 0, st, a); break;
            case 32: hipLaunchKernelGGL(decode_down_flat_kernel<32>, dn_grid, dim3(kThreads), 0, st, a); break;
            default: hipLaunchKernelGGL(decode_down_flat_kernel<64>, dn_grid, dim3(kThreads), 0, st, a); break;
        }
        return e0_launch_status();
    }
    const int ublocks = a.umax + (a.has_shared ? 1 : 0);
    if (B == 1) {
        constexpr int TC = 1, RB = 16;
        const int rpb = gateup_rows_per_block<TC, RB>(lpr_d);
        dim3 grid(L, ublocks, (f + rpb - 1) / rpb);
        const bool ok = dispatch_gateup<TC, RB, 1>(lpr_d, np, a, grid, st);
        E0_REQUIRE(ok, E0_ERR_UNSUPPORTED_SHAPE);
    } else {
        // Each block streams kGuGroups groups of rows of one expert.
        constexpr int TC = 4, RB = 4;
        const int rpb = gateup_rows_per_block<TC, RB>(lpr_d) * kGuGroups;
        dim3 grid(L, ublocks, (f + rpb - 1) / rpb);
        const bool ok = dispatch_gateup<TC, RB, kGuGroups>(lpr_d, np, a, grid, st);
        E0_REQUIRE(ok, E0_ERR_UNSUPPORTED_SHAPE);
    }
    if ((s = e0_launch_status())) return s;
    if (B > 1) {
        // Batches at d_ff = 128, 256 or 512: the matrix-core down kernel.
        const dim3 grid(L, (d + kDownRows - 1) / kDownRows);
        const size_t lds = dm_lds_bytes(B, r, f / kGroup, a.umax);
        bool mf = lds <= kDmMaxLds;
        switch (mf ? f / kGroup : 0) {
            case 2: hipLaunchKernelGGL(decode_down_mfma_kernel<2>, grid, dim3(kThreads), lds, st, a); break;
            case 4: hipLaunchKernelGGL(decode_down_mfma_kernel<4>, grid, dim3(kThreads), lds, st, a); break;
            case 8: hipLaunchKernelGGL(decode_down_mfma_kernel<8>, grid, dim3(kThreads), lds, st, a); break;
            default: mf = false;
        }
        if (mf) return e0_launch_status();
    }
    E0_REQUIRE(dispatch_down(lpr_f, a, dim3(L, (d + kDownRows - 1) / kDownRows), st), E0_ERR_UNSUPPORTED_SHAPE);
    return e0_launch_status();
}

size_t e0_chain_workspace_bytes(const e0_moe_dims *dims, int32_t L) {
    if (!dims || L < 0 || !fused_shape_ok(dims->d_model, dims->d_ff, dims->top_k)) return 0;
    const int n_dn = dims->d_model / (kFuseWaves * chain_rows_per_wave(dims->top_k, f_lpr(dims->d_ff)));
    return decode_layout(L, 1, dims->top_k, dims->n_experts, dims->d_ff, 0, n_dn).total;
}

extern "C" e0_status e0_moe_chained_decode(const e0_moe_dims *dims, int32_t L, const float *r_in, const uint16_t *norm_w,
                                           float eps, const int32_t *idx, const float *w, const int32_t *slot_of,
                                           int32_t S, const e0_stack *pool, float *y, float *r_out, void *ws,
                                           size_t ws_bytes, int32_t *dev_err, void *stream) {
    e0_clear_stale_error();
    E0_REQUIRE(dims && pool, E0_ERR_INVALID_ARG);
    const int d = dims->d_model, f = dims->d_ff, E = dims->n_experts, K = dims->top_k;
    E0_REQUIRE(L >= 0 && S >= 1 && E >= 1 && K >= 1 && K <= E && E <= kMaxE, E0_ERR_INVALID_ARG);
    E0_REQUIRE(fused_shape_ok(d, f, K), E0_ERR_UNSUPPORTED_SHAPE);
    E0_REQUIRE(isfinite(eps) && eps >= 0.0f, E0_ERR_INVALID_ARG);
    E0_REQUIRE(r_in && norm_w && idx && w && slot_of && y && r_out && dev_err, E0_ERR_INVALID_ARG);
    E0_REQUIRE(((reinterpret_cast<uintptr_t>(r_in) | reinterpret_cast<uintptr_t>(norm_w) |
                 reinterpret_cast<uintptr_t>(r_out)) & 15) == 0, E0_ERR_INVALID_ARG);
    E0_REQUIRE(stack_ok(pool, 0, 8), E0_ERR_INVALID_ARG);
    const int lpr_f = f_lpr(f);
    const int rw = chain_rows_per_wave(K, lpr_f);
    const int64_t n_gu = (int64_t)K * (f / kHalfBlk / (kFuseWaves / kChainSplit)), n_dn = d / (kFuseWaves * rw);
    const Layout lay = decode_layout(L, 1, K, E, f, 0, (int)n_dn);
    E0_REQUIRE(ws && ws_bytes >= lay.total && (reinterpret_cast<uintptr_t>(ws) & 255) == 0, E0_ERR_CAPACITY);
    E0_REQUIRE((int64_t)L * (n_gu + n_dn) <= (int64_t)INT32_MAX, E0_ERR_CAPACITY);
    if (L == 0) return E0_OK;

    DecodeArgs a{};
    a.L = L;
    a.B = 1;
    a.K = K;
    a.E = E;
    a.S = S;
    a.d = d;
    a.f = f;
    a.idx = idx;
    a.w = w;
    a.slot_of = slot_of;
    a.pool = to_stack(*pool);
    a.y = y;
    a.err = dev_err;
    a.umax = K;
    char *wsb = static_cast<char *>(ws);
    a.hbuf = reinterpret_cast<float *>(wsb + lay.hbuf);
    a.lora_a = reinterpret_cast<float *>(wsb + lay.lora);
    a.flags = reinterpret_cast<uint64_t *>(wsb + lay.flags);
    a.hblk = reinterpret_cast<uint32_t *>(wsb + lay.hblk);
    a.epoch = e0_next_epoch();
    a.units = K;
    a.nch = f / kHalfBlk;
    a.n_lora = 0;
    a.lora_parts = 0;
    a.n_gu = (int)n_gu;
    a.n_dn = (int)n_dn;
    // Layer l's down items follow its gate/up items directly; the gate/up
    // items of layer l + 1 follow them and wait for them, so every wait is on
    // items dispatched earlier.
    a.lag = 0;
    a.chain = 1;
    a.r_in = r_in;
    a.r_out = r_out;
    a.norm_w = norm_w;
    a.norm_eps = eps;
    a.dflags = reinterpret_cast<uint64_t *>(wsb + lay.dflags);
    launch_fused(a, lpr_f, K <= 4, dim3((unsigned)(L * (n_gu + n_dn))), static_cast<hipStream_t>(stream));
    return e0_launch_status();
}
