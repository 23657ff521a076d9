/*
 * Sanitizer driver for the CPU oracle (TEST INFRASTRUCTURE ONLY): calls every
 * function of oracle.h on small, fixed inputs so that an AddressSanitizer /
 * UndefinedBehaviorSanitizer build of oracle.c reports any out-of-bounds
 * access, use of uninitialised heap, signed overflow or similar on the paths
 * the tests use. Built and run by oracle/build.py (build_sanitized) from a
 * CPU test; prints "sanitize ok" and exits 0 when nothing was reported.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

enum { D = 128, F = 64, E = 16, K = 4, T = 5, S = 8, L = 3, R = 4, HID = 64 };

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return (uint32_t)st;
}
/* fp16 bit pattern of a small value in [-2, 2) with 10 random mantissa bits. */
static uint16_t rnd_half(void) { return orc_to_half(((double)(next32() % 4096) - 2048.0) / 1024.0); }

static orc_mat make_mat(int rows, int cols) {
    orc_mat m;
    uint32_t *q = malloc(sizeof(uint32_t) * (size_t)rows * cols / 8);
    uint16_t *s = malloc(sizeof(uint16_t) * (size_t)rows * cols / 64);
    uint16_t *b = malloc(sizeof(uint16_t) * (size_t)rows * cols / 64);
    for (int i = 0; i < rows * cols / 8; ++i) q[i] = next32();
    for (int i = 0; i < rows * cols / 64; ++i) {
        s[i] = orc_to_half(0.005 + 0.015 * (next32() % 1000) / 1000.0);
        b[i] = orc_to_half(-8.0 * orc_half(s[i]));
    }
    m.q = q;
    m.s = s;
    m.b = b;
    return m;
}
static orc_expert make_expert(int d, int f) {
    orc_expert e = {make_mat(f, d), make_mat(f, d), make_mat(d, f)};
    return e;
}
static uint16_t *halves(size_t n) {
    uint16_t *v = malloc(sizeof(uint16_t) * n);
    for (size_t i = 0; i < n; ++i) v[i] = rnd_half();
    return v;
}

int main(void) {
    orc_expert ex[E];
    for (int e = 0; e < E; ++e) ex[e] = make_expert(D, F);
    uint16_t *x = halves((size_t)T * D);
    uint16_t *wr = halves((size_t)E * D);
    float lg[T * E];
    int32_t idx[T * K];
    double w[T * K], y[T * D], y2[T * D], y3[T * D], dq[F * D];
    int32_t perm[T * K];

    orc_dequant(&ex[0].gate, F, D, dq);
    orc_router_logits(x, wr, T, E, D, lg);
    orc_softmax_topk(lg, T, E, K, idx, w);
    (void)orc_softmax_topk_margin(lg, T, E, K);
    if (orc_sigmoid_group(lg, T, E, K, 4, 2, 2.5, 1e-20, idx, w)) return 2;
    (void)orc_sigmoid_group_margin(lg, T, E, K, 4, 2);
    orc_softmax_topk(lg, T, E, K, idx, w);
    orc_expert_ffn(&ex[1], D, F, x, y);
    if (orc_moe_exact(ex, E, D, F, T, K, x, idx, w, y)) return 3;
    if (orc_moe_sorted(ex, E, D, F, T, K, x, idx, w, y2, perm)) return 4;

    /* slot rule over two steps, then the staged ordering through the pool */
    int32_t slot_of[E], expert_of[S], cs[E], ce[E], nc = 0;
    for (int e = 0; e < E; ++e) slot_of[e] = -1;
    for (int s = 0; s < S; ++s) expert_of[s] = -1;
    if (orc_slot_update(E, S, idx, K, NULL, 0, slot_of, expert_of, cs, ce, &nc)) return 5;
    if (orc_slot_update(E, S, idx + K, K, idx, K, slot_of, expert_of, cs, ce, &nc)) return 6;
    orc_expert pool[S];
    for (int s = 0; s < S; ++s) pool[s] = ex[expert_of[s] >= 0 ? expert_of[s] : 0];
    (void)orc_moe_staged(pool, S, slot_of, E, D, F, 2, K, x, idx, w, y3);

    /* prerouter head and its feature */
    orc_head hd = {halves((size_t)HID * (D + 2 * E)), halves(HID), halves((size_t)E * HID), halves(E),
                   halves((size_t)E * D)};
    double feat[D + 2 * E], o[E];
    orc_head_feature(x, D, E, idx, idx + K, K, feat);
    orc_head_logits(&hd, D, E, HID, x, idx, NULL, K, o);
    orc_head_logits(&hd, D, E, HID, x, idx, idx + K, K, o);

    /* shared expert with unmerged LoRA */
    orc_lora lo[3] = {{halves((size_t)R * D), halves((size_t)F * R)},
                      {halves((size_t)R * D), halves((size_t)F * R)},
                      {halves((size_t)R * F), halves((size_t)D * R)}};
    orc_shared_lora(&ex[2], lo, R, 2.0, D, F, x, y);
    orc_shared_lora(&ex[2], NULL, R, 2.0, D, F, x, y);

    /* threaded staged decode and the chained decode over L layers */
    orc_expert pools[L * S];
    int32_t so[L * E], lidx[L * K];
    double lw[L * K], ly[L * D], lr[L * D], r0[D];
    uint16_t *lx = halves((size_t)L * D);
    uint16_t *g = halves((size_t)L * D);
    for (int l = 0; l < L; ++l) {
        for (int e = 0; e < E; ++e) so[l * E + e] = -1;
        for (int k = 0; k < K; ++k) {
            lidx[l * K + k] = (3 * l + 5 * k) % E;
            lw[l * K + k] = 0.25;
            so[l * E + lidx[l * K + k]] = k;
            pools[l * S + k] = ex[lidx[l * K + k]];
        }
        for (int s = K; s < S; ++s) pools[l * S + s] = ex[0];
    }
    for (int i = 0; i < D; ++i) r0[i] = orc_half(rnd_half());
    if (orc_decode_layers(pools, S, so, L, E, D, F, 1, K, lx, lidx, lw, ly, 3)) return 7;
    if (orc_chain_decode(pools, S, so, L, E, D, F, K, r0, g, 1e-6, lidx, lw, ly, lr)) return 8;
    printf("sanitize ok\n");
    return 0;
}
