// A LoRA delta merged into an int4 group-64 matrix and requantised: the
// alternative to serving the recovery LoRA unmerged that the pages measure
// (jaehun.me review, the paragraph on not merging, citing the report's
// section 3.3 and its retention measure 1 - |U - M| / |U - B|; xyznot.com FAQ
// on why the recovery LoRA stays unmerged). The requantisation is the plain
// min/max affine form of the stacks' format (scale = range / 15, bias = the
// group's least value, codes rounded half to even); every fp32 operation is
// rounded to nearest on its own, so the codes do not depend on contraction.
//
// One thread per (row, 64-column group); a workgroup covers one 8-row tile
// and 32 groups, so its scale and bias stores are 512 contiguous bytes each.
#include "e0_internal.h"

#include <cmath>

namespace {

constexpr int kMergeThreads = 256;
constexpr int kGroupsPerBlock = kMergeThreads / 8;
constexpr int kMaxRank = 64;

// Single fp32 operations rounded to nearest; fp-contract is off here, so no
// multiply and add pair is fused (the library is built with contraction on).
E0_DEV float add_rn(float x, float y) {
#pragma clang fp contract(off)
    return x + y;
}
E0_DEV float mul_rn(float x, float y) {
#pragma clang fp contract(off)
    return x * y;
}
E0_DEV float div_rn(float x, float y) { return x / y; }  // IEEE division (correctly rounded by default)

__global__ __launch_bounds__(kMergeThreads) void lora_merge_kernel(int rows, int cols, const uint32_t *q,
                                                                  const uint16_t *s, const uint16_t *b,
                                                                  const uint16_t *lb, const uint16_t *la, int r,
                                                                  float alpha, uint32_t *q_out, uint16_t *s_out,
                                                                  uint16_t *b_out) {
    const int ngrp = cols / kGroup;
    const int tile = blockIdx.y;
    const int row = tile * 8 + (threadIdx.x & 7);
    const int g = blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 3);
    if (g >= ngrp || row >= rows) return;
    const int64_t sb = ((int64_t)tile * ngrp + g) * 8 + (threadIdx.x & 7);  // 8-row tile layout
    const float sc = (float)__builtin_bit_cast(f16, s[sb]);
    const float bi = (float)__builtin_bit_cast(f16, b[sb]);
    const u32x4 *qw = reinterpret_cast<const u32x4 *>(q + (int64_t)row * (cols / 8) + g * 8);
    const u32x4 qa = qw[0], qb = qw[1];
    const uint32_t words[8] = {qa[0], qa[1], qa[2], qa[3], qb[0], qb[1], qb[2], qb[3]};
    // t for the 64 columns, k outermost (each column's sum in k order).
    float w[kGroup];
#pragma unroll
    for (int c = 0; c < kGroup; ++c) w[c] = 0.0f;
    for (int k = 0; k < r; ++k) {
        const float bk = (float)__builtin_bit_cast(f16, lb[(int64_t)row * r + k]);
        const u32x4 *arow = reinterpret_cast<const u32x4 *>(la + (int64_t)k * cols + g * kGroup);
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {  // 8 columns: one 16-byte load of A
            const u32x4 av = arow[ch];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t aw = av[j];
                const f16x2 a2 = as_h2(aw);
                w[ch * 8 + 2 * j] = add_rn(w[ch * 8 + 2 * j], mul_rn(bk, (float)a2[0]));
                w[ch * 8 + 2 * j + 1] = add_rn(w[ch * 8 + 2 * j + 1], mul_rn(bk, (float)a2[1]));
            }
        }
    }
    // w' = (s q + b) + alpha t.
#pragma unroll
    for (int c = 0; c < kGroup; ++c) {
        const float code = (float)((words[c / 8] >> (4 * (c % 8))) & 15u);
        const float dq = add_rn(mul_rn(sc, code), bi);
        w[c] = add_rn(dq, mul_rn(alpha, w[c]));
    }
    float lo = w[0], hi = w[0];
#pragma unroll
    for (int c = 1; c < kGroup; ++c) {
        lo = w[c] < lo ? w[c] : lo;
        hi = w[c] > hi ? w[c] : hi;
    }
    const f16 s16 = (f16)div_rn(add_rn(hi, -lo), 15.0f);
    const f16 b16 = (f16)lo;
    const float s2 = (float)s16, b2 = (float)b16;
    uint32_t out[8];
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float v = 0.0f;
            if (s2 != 0.0f) {
                v = __builtin_rintf(div_rn(add_rn(w[ch * 8 + j], -b2), s2));
                v = v < 0.0f ? 0.0f : v > 15.0f ? 15.0f : v;
            }
            word |= (uint32_t)v << (4 * j);
        }
        out[ch] = word;
    }
    u32x4 *qo = reinterpret_cast<u32x4 *>(q_out + (int64_t)row * (cols / 8) + g * 8);
    qo[0] = u32x4{out[0], out[1], out[2], out[3]};
    qo[1] = u32x4{out[4], out[5], out[6], out[7]};
    s_out[sb] = __builtin_bit_cast(uint16_t, s16);
    b_out[sb] = __builtin_bit_cast(uint16_t, b16);
}

bool overlaps(const void *p, size_t np, const void *q, size_t nq) {
    const char *a = static_cast<const char *>(p), *b = static_cast<const char *>(q);
    return a < b + nq && b < a + np;
}

}  // namespace

extern "C" e0_status e0_lora_merge_requant(int32_t rows, int32_t cols, const uint32_t *q, const uint16_t *s,
                                           const uint16_t *b, const uint16_t *lora_b, const uint16_t *lora_a,
                                           int32_t r, float alpha_over_r, uint32_t *q_out, uint16_t *s_out,
                                           uint16_t *b_out, void *stream) {
    e0_clear_stale_error();
    E0_REQUIRE(q && s && b && lora_b && lora_a && q_out && s_out && b_out, E0_ERR_INVALID_ARG);
    E0_REQUIRE(rows > 0 && cols > 0 && rows % 8 == 0 && cols % kGroup == 0, E0_ERR_UNSUPPORTED_SHAPE);
    E0_REQUIRE((int64_t)rows * cols < ((int64_t)1 << 31), E0_ERR_UNSUPPORTED_SHAPE);
    E0_REQUIRE(r >= 1 && r <= kMaxRank, E0_ERR_UNSUPPORTED_SHAPE);
    E0_REQUIRE(std::isfinite(alpha_over_r), E0_ERR_INVALID_ARG);
    const void *ptrs[8] = {q, s, b, lora_b, lora_a, q_out, s_out, b_out};
    for (const void *p : ptrs) E0_REQUIRE((reinterpret_cast<uintptr_t>(p) & 15) == 0, E0_ERR_INVALID_ARG);
    const size_t nq = (size_t)rows * cols / 2, ns = (size_t)rows * (cols / kGroup) * 2;
    const void *ins[5] = {q, s, b, lora_b, lora_a};
    const size_t nin[5] = {nq, ns, ns, (size_t)rows * r * 2, (size_t)r * cols * 2};
    const void *outs[3] = {q_out, s_out, b_out};
    const size_t nout[3] = {nq, ns, ns};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 5; ++i) E0_REQUIRE(!overlaps(outs[o], nout[o], ins[i], nin[i]), E0_ERR_INVALID_ARG);
        for (int p = o + 1; p < 3; ++p) E0_REQUIRE(!overlaps(outs[o], nout[o], outs[p], nout[p]), E0_ERR_INVALID_ARG);
    }
    const dim3 grid((unsigned)((cols / kGroup + kGroupsPerBlock - 1) / kGroupsPerBlock), (unsigned)(rows / 8));
    hipLaunchKernelGGL(lora_merge_kernel, grid, dim3(kMergeThreads), 0, static_cast<hipStream_t>(stream), rows, cols,
                       q, s, b, lora_b, lora_a, r, alpha_over_r, q_out, s_out, b_out);
    return e0_launch_status();
}
