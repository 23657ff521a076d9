// GPU twin of e0inputs/gen.py: fills int4 group-64 expert bundles from
// counter-based SplitMix64 streams, bit for bit equal to the numpy generator.
// Input generation only: no part of the method's arithmetic is here.
//
// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): draw i of the stream with
// key k is fin(k + (i + 1) * GAMMA). Value recipes (each fp32 step rounded to
// nearest-even on its own, as numpy float32 does):
//   codes : two little-endian uint32 words per 64-bit draw
//   scale : fp16(0.005f + 0.015f * u),   u = (draw >> 40) * 2^-24
//   bias  : fp16(-8 * (s * (1 + (0.2f * v - 0.1f)))), v likewise, s the fp16 scale
// Scale/bias draw r*(cols/64) + g belongs to row r, group g; the bundle stores
// scales and biases in tiles of 8 rows ([rows/8][cols/64][8]), so bundle
// element ((r/8)*(cols/64) + g)*8 + r%8 takes that draw.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t fin(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t draw(uint64_t key, uint64_t i) { return fin(key + (i + 1) * kGamma); }
__device__ __forceinline__ float u24(uint64_t d) { return __fmul_rn((float)(uint32_t)(d >> 40), 5.9604644775390625e-08f); }
__device__ __forceinline__ uint16_t f2h(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ __forceinline__ uint16_t scale_at(uint64_t ks, uint64_t g) {
    return f2h(__fadd_rn(0.005f, __fmul_rn(0.015f, u24(draw(ks, g)))));
}
__device__ __forceinline__ uint16_t bias_at(uint64_t ks, uint64_t kb, uint64_t g) {
    const float s = h2f(scale_at(ks, g));
    const float t = __fadd_rn(1.0f, __fsub_rn(__fmul_rn(0.2f, u24(draw(kb, g))), 0.1f));
    return f2h(-8.0f * __fmul_rn(s, t));
}

struct FillArgs {
    char *dst;
    int64_t stride;        // bytes between consecutive experts
    const uint64_t *keys;  // [n][3 matrices][3 parts]
    int64_t part_units[9];
    int64_t part_end[9];
    int64_t rows[3];  // rows of gate, up, down
    int64_t ngrp[3];  // groups per row (cols / 64)
};

__global__ __launch_bounds__(256) void fill_kernel(FillArgs a) {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte unit of the bundle
    const int e = blockIdx.y;
    if (u >= a.part_end[8]) return;
    int j = 0;
    while (u >= a.part_end[j]) ++j;
    const int64_t off = u - (a.part_end[j] - a.part_units[j]);
    const int m = j / 3, kind = j % 3;
    const uint64_t *k = a.keys + (int64_t)e * 9 + m * 3;
    u32x4 v;
    if (kind == 0) {
        const uint64_t d0 = draw(k[0], 2 * off), d1 = draw(k[0], 2 * off + 1);
        v = u32x4{(uint32_t)d0, (uint32_t)(d0 >> 32), (uint32_t)d1, (uint32_t)(d1 >> 32)};
    } else {
        uint16_t h[8];
        for (int i = 0; i < 8; ++i) {
            const int64_t p = 8 * off + i;  // tiled position ((r/8)*ngrp + g)*8 + r%8
            const int64_t r = (p / (8 * a.ngrp[m])) * 8 + p % 8, g = (p / 8) % a.ngrp[m];
            const uint64_t idx = (uint64_t)(r * a.ngrp[m] + g);
            h[i] = kind == 1 ? scale_at(k[1], idx) : bias_at(k[1], k[2], idx);
        }
        v = u32x4{h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16, h[4] | (uint32_t)h[5] << 16,
                  h[6] | (uint32_t)h[7] << 16};
    }
    *reinterpret_cast<u32x4 *>(a.dst + (int64_t)e * a.stride + 16 * u) = v;
}

}  // namespace

// Fill n_experts bundles at dst (stride bytes apart) for d_model d, d_ff f.
// keys: device uint64 [n][9], in bundle part order (gate q,s,b, up q,s,b, down q,s,b).
extern "C" int e0gen_fill_experts(void *dst, int64_t stride, const uint64_t *keys, int n_experts, int d, int f,
                                  void *stream) {
    if (!dst || !keys || n_experts < 0 || d % 64 || f % 64 || d <= 0 || f <= 0) return 1;
    FillArgs a{};
    a.dst = static_cast<char *>(dst);
    a.stride = stride;
    a.keys = keys;
    const int64_t qb = (int64_t)d * f / 2, sb = (int64_t)d * f / 64 * 2;
    int64_t acc = 0;
    for (int j = 0; j < 9; ++j) {
        a.part_units[j] = (j % 3 == 0 ? qb : sb) / 16;
        acc += a.part_units[j];
        a.part_end[j] = acc;
    }
    for (int m = 0; m < 3; ++m) {
        a.rows[m] = m < 2 ? f : d;
        a.ngrp[m] = (m < 2 ? d : f) / 64;
    }
    if (stride < acc * 16 || (stride & 15) || (reinterpret_cast<uintptr_t>(dst) & 15)) return 1;
    (void)hipGetLastError();  // a status left pending by the caller's earlier runtime calls
    if (n_experts == 0) return 0;
    if (n_experts > 65535) return 1;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((acc + 255) / 256), n_experts), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : 1000 + (int)e;  // 1000 + the HIP error code
}
