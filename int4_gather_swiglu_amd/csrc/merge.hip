// A LoRA delta merged into an int4 group-64 matrix and requantised: the
// alternative to serving the recovery LoRA unmerged that the pages measure
// (jaehun.me review, the paragraph on not merging, citing the report's
// section 3.3 and its retention measure 1 - |U - M| / |U - B|; xyznot.com FAQ
// on why the recovery LoRA stays unmerged). The requantisation is the plain
// min/max affine form of the stacks' format (scale = range / 15, bias = the
// group's least value, codes rounded half to even); every fp32 operation is
// rounded to nearest on its own, so the codes do not depend on contraction.
//
// Eight lanes per (row, 64-column group), one code word each; the group's
// least and largest value meet by lane shuffles. A workgroup covers one 8-row
// tile and 4 groups; its slice of A and its rows of B are staged in LDS
// first. A 512 x 2048 matrix is 2048 wavefronts.
#include "e0_internal.h"

#include <cmath>

namespace {

constexpr int kMergeThreads = 256;
constexpr int kGroupsPerBlock = kMergeThreads / 64;  // 8 rows x 4 groups x 8 lanes
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

// Eight consecutive lanes share one (row, group); lane j of them owns columns
// 8j .. 8j + 7 of the group (its code word j).
__global__ __launch_bounds__(kMergeThreads) void lora_merge_kernel(int rows, int cols, const uint32_t *q,
                                                                  const uint16_t *s, const uint16_t *b,
                                                                  const uint16_t *lb, const uint16_t *la, int r,
                                                                  float alpha, uint32_t *q_out, uint16_t *s_out,
                                                                  uint16_t *b_out) {
    const int ngrp = cols / kGroup;
    const int tile = blockIdx.y;
    const int sub = threadIdx.x & 7, pair = threadIdx.x >> 3;
    const int rl = pair & 7, gl = pair >> 3;
    const int row = tile * 8 + rl;
    const int g0 = blockIdx.x * kGroupsPerBlock, g = g0 + gl;
    // The workgroup's slice of A (r rows x its groups) and the 8 rows of B go
    // to LDS once, all loads in flight together.
    extern __shared__ __attribute__((aligned(16))) uint16_t s_ab[];
    constexpr int kUnits = kGroupsPerBlock * kGroup / 8;  // 16-byte units per row of the slice
    uint16_t *s_a = s_ab;                                 // [r][kGroupsPerBlock * 64]
    uint16_t *s_b = s_ab + r * kUnits * 8;                // [8][r]
    for (int i = threadIdx.x; i < r * kUnits; i += kMergeThreads) {
        const int k = i / kUnits, u = i % kUnits;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (g0 + u / 8 < ngrp) v = *reinterpret_cast<const u32x4 *>(la + (int64_t)k * cols + g0 * kGroup + u * 8);
        *reinterpret_cast<u32x4 *>(s_a + (k * kUnits + u) * 8) = v;
    }
    for (int i = threadIdx.x; i < 8 * r; i += kMergeThreads) s_b[i] = lb[(int64_t)(tile * 8 + i / r) * r + i % r];
    __syncthreads();
    const bool on = g < ngrp;  // lanes past the last group compute on zeros and store nothing
    const int64_t sb = ((int64_t)tile * ngrp + (on ? g : 0)) * 8 + rl;  // 8-row tile layout
    const float sc = (float)__builtin_bit_cast(f16, s[sb]);
    const float bi = (float)__builtin_bit_cast(f16, b[sb]);
    const uint32_t word = q[(int64_t)row * (cols / 8) + (on ? g : 0) * 8 + sub];

    // t for this lane's 8 columns, k outermost (each column's sum in k order).
    float w[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) w[c] = 0.0f;
    for (int k = 0; k < r; ++k) {
        const float bk = (float)__builtin_bit_cast(f16, s_b[rl * r + k]);
        const u32x4 av = *reinterpret_cast<const u32x4 *>(s_a + (k * kUnits + gl * 8 + sub) * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t aw = av[j];
            const f16x2 a2 = as_h2(aw);
            w[2 * j] = add_rn(w[2 * j], mul_rn(bk, (float)a2[0]));
            w[2 * j + 1] = add_rn(w[2 * j + 1], mul_rn(bk, (float)a2[1]));
        }
    }
    // w' = (s q + b) + alpha t; the group's least and largest over its 8 lanes.
    float lo, hi;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float code = (float)((word >> (4 * c)) & 15u);
        const float dq = add_rn(mul_rn(sc, code), bi);
        w[c] = add_rn(dq, mul_rn(alpha, w[c]));
        lo = c ? (w[c] < lo ? w[c] : lo) : w[c];
        hi = c ? (w[c] > hi ? w[c] : hi) : w[c];
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
        const float lo2 = __shfl_xor(lo, o), hi2 = __shfl_xor(hi, o);
        lo = lo2 < lo ? lo2 : lo;
        hi = hi2 > hi ? hi2 : hi;
    }
    const f16 s16 = (f16)div_rn(add_rn(hi, -lo), 15.0f);
    const f16 b16 = (f16)lo;
    const float s2 = (float)s16, b2 = (float)b16;
    uint32_t out = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float v = 0.0f;
        if (s2 != 0.0f) {
            v = __builtin_rintf(div_rn(add_rn(w[c], -b2), s2));
            v = v < 0.0f ? 0.0f : v > 15.0f ? 15.0f : v;
        }
        out |= (uint32_t)v << (4 * c);
    }
    if (!on) return;
    q_out[(int64_t)row * (cols / 8) + g * 8 + sub] = out;
    if (sub == 0) {
        s_out[sb] = __builtin_bit_cast(uint16_t, s16);
        b_out[sb] = __builtin_bit_cast(uint16_t, b16);
    }
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
    const size_t lds = ((size_t)r * kGroupsPerBlock * kGroup + 8 * (size_t)r) * 2;  // A slice + B rows
    hipLaunchKernelGGL(lora_merge_kernel, grid, dim3(kMergeThreads), lds, static_cast<hipStream_t>(stream), rows, cols,
                       q, s, b, lora_b, lora_a, r, alpha_over_r, q_out, s_out, b_out);
    return e0_launch_status();
}
