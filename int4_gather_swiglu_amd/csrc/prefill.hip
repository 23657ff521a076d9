// Sorted whole-layer prefill on gfx950: the (token, k) pairs of a layer are
// sorted by expert, each active expert runs as a grouped GEMM on the matrix
// cores with its int4 group-64 weights dequantised to fp16 in registers, and
// the weighted results are summed back in token order.
//
// Method: the whole-layer path loads all of a layer's experts and runs a
// sorted gather (jaehun.me review, report 3.1; discuss.pytorch.kr paths
// table; prefill never predicts, report 3.2); the math contract is
// down(silu(gate(x)) * up(x)) for every path (report 3.1), combined as
// y_t = sum_k w_tk FFN_{e_tk}(x_t).
//
// Launches (one stream):
//  1. sort     (1 workgroup): counting sort of the T*K pairs by expert (LDS
//               counters, one scan, scatter), the row offset of every
//               expert and the list of 128-row M-tiles.
//  2. gemm1    (tiles x d_ff/128): H = silu(X G^T) * (X U^T) for one M-tile
//               and 128 columns of d_ff, X gathered through the sort; H fp16.
//  3. gemm2    (tiles x d_model/128): Yb[pair] = w_pair * (H D^T).
//  4. combine  : y[t] = sum over k in order of Yb[t*K + k].
//
// MFMA v_mfma_f32_32x32x16_f16. Inside each 64-wide quantisation group the
// reduction index is permuted the same way on both operands (so the sum is
// unchanged): lane half h of MFMA j covers inputs 32h + 8j .. 32h + 8j + 7, in
// the order (0,4,1,5,2,6,3,7). A lane's B fragment for the four MFMAs of a
// group is then one 16-byte load of four code words of its column, and each
// word dequantises as four (q_c, q_{c+4}) pairs: 1024+q by bit placement,
// minus 1024 exactly, then one fp16 fma s*q + b (a single rounding of the
// exact dequantised weight).
#include "e0_internal.h"

#include <math.h>

namespace {

constexpr int kTM = 128;         // rows per M-tile
constexpr int kTN = 128;         // columns per workgroup (4 waves x 32)
constexpr int kGemmThreads = 256;
constexpr int kSortThreads = 1024;
constexpr int kMaxSortE = 1024;
constexpr int kARowPad = 72;     // halves per LDS row of A (64 + 8 padding)

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

struct PrefillArgs {
    int T, K, E, d, f, n;
    const uint16_t *x;
    const int32_t *idx;
    const float *w;
    Stack layer;
    float *y;
    int32_t *err;
    int32_t *off;       // [E + 1] first sorted row of each expert
    int32_t *perm;      // [n] pair index at each sorted row
    int32_t *ntiles;    // [1]
    int32_t *tile_e;    // [max_tiles]
    int32_t *tile_m0;   // [max_tiles]
    uint16_t *H;        // [n][f] fp16
    float *Yb;          // [n][d] weighted down outputs, by pair index
    int max_tiles;
};

// ---------------------------------------------------------------------------
// 1. sort (one workgroup)
// ---------------------------------------------------------------------------
E0_DEV int block_scan_1024(int v, int *lds16, int &total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    if (lane == 63) lds16[wv] = inc;
    __syncthreads();
    int base = 0;
    total = 0;
    for (int i = 0; i < kSortThreads / 64; ++i) {
        const int t = lds16[i];
        if (i < wv) base += t;
        total += t;
    }
    __syncthreads();
    return base + inc - v;
}

__global__ __launch_bounds__(kSortThreads) void prefill_sort_kernel(PrefillArgs a) {
    __shared__ int s_cnt[kMaxSortE];
    __shared__ int s_fill[kMaxSortE];
    __shared__ int s_scan[kSortThreads / 64];
    const int tid = threadIdx.x;
    const int E = a.E, n = a.n;
    for (int e = tid; e < E; e += kSortThreads) s_cnt[e] = s_fill[e] = 0;
    __syncthreads();
    // Counts per expert (LDS atomics; the counts do not depend on their order).
    for (int p = tid; p < n; p += kSortThreads) {
        const int e = a.idx[p];
        if (e >= 0 && e < E)
            atomicAdd(&s_cnt[e], 1);
        else
            set_err(a.err, E0_DEV_BAD_ID);
    }
    __syncthreads();
    // Exclusive scan -> first sorted row of each expert; tiles per expert.
    const int eper = (E + kSortThreads - 1) / kSortThreads;
    int local = 0, nt = 0;
    for (int e = tid * eper; e < (tid + 1) * eper && e < E; ++e) {
        local += s_cnt[e];
        nt += (s_cnt[e] + kTM - 1) / kTM;
    }
    int total, tt;
    int run = block_scan_1024(local, s_scan, total);
    int tb = block_scan_1024(nt, s_scan, tt);
    for (int e = tid * eper; e < (tid + 1) * eper && e < E; ++e) {
        a.off[e] = run;
        s_fill[e] = run;
        for (int m = 0; m < s_cnt[e]; m += kTM, ++tb) {
            a.tile_e[tb] = e;
            a.tile_m0[tb] = run + m;
        }
        run += s_cnt[e];
    }
    if (tid == 0) {
        a.off[E] = total;
        a.ntiles[0] = tt;
    }
    __syncthreads();
    // Scatter. The order of rows inside an expert's block follows the LDS
    // atomics and may differ from run to run; no output depends on it (every
    // GEMM row is computed on its own and results are stored by pair index).
    for (int p = tid; p < n; p += kSortThreads) {
        const int e = a.idx[p];
        if (e >= 0 && e < E) a.perm[atomicAdd(&s_fill[e], 1)] = p;
    }
}

// ---------------------------------------------------------------------------
// 2./3. grouped GEMM
// ---------------------------------------------------------------------------
E0_DEV uint32_t and_or_v(uint32_t x, uint32_t m, uint32_t c) {
    uint32_t r;
    __asm__("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(c));
    return r;
}

// Eight fp16 weights of one code word, in the pair order (q0,q4,q1,q5,...):
// s * q + b with one rounding. s2 / b2 hold (s, s) / (b, b).
E0_DEV h8 dequant_word(uint32_t w, f16x2 s2, f16x2 b2, uint32_t m, uint32_t c) {
    const f16x2 k1024 = f16x2{(f16)1024.0f, (f16)1024.0f};
    h8 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f16x2 t = as_h2(and_or_v(w >> (4 * j), m, c)) - k1024;  // (q_j, q_{j+4}), exact
        const f16x2 v = __builtin_elementwise_fma(t, s2, b2);
        o[2 * j] = v[0];
        o[2 * j + 1] = v[1];
    }
    return o;
}

// (h0..h7) -> (h0,h4,h1,h5,h2,h6,h3,h7)
E0_DEV u32x4 permute8(u32x4 v) {
    u32x4 o;
    o[0] = __builtin_amdgcn_perm(v[2], v[0], 0x05040100u);
    o[1] = __builtin_amdgcn_perm(v[2], v[0], 0x07060302u);
    o[2] = __builtin_amdgcn_perm(v[3], v[1], 0x05040100u);
    o[3] = __builtin_amdgcn_perm(v[3], v[1], 0x07060302u);
    return o;
}

template <bool GATEUP>
__global__ __launch_bounds__(kGemmThreads) void prefill_gemm_kernel(PrefillArgs a) {
    constexpr int NM = GATEUP ? 2 : 1;  // matrices: gate and up, or down
    __shared__ __attribute__((aligned(16))) uint16_t s_a[2][kTM * kARowPad];
    const int Nall = GATEUP ? a.f : a.d;       // output columns
    const int Kdim = GATEUP ? a.d : a.f;       // reduction length
    const int ngroups = Kdim / kGroup;
    const int nN = Nall / kTN;
    const int tile = blockIdx.x / nN, nt = blockIdx.x % nN;
    if (tile >= a.ntiles[0]) return;
    const int e = a.tile_e[tile], m0 = a.tile_m0[tile];
    const int m_end = a.off[e + 1];
    const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
    const int h = lane >> 5;
    const int col = nt * kTN + wv * 32 + (lane & 31);  // this lane's output column

    // A staging: chunk c = tid + 256 i covers row c / 8, 8-half block c % 8.
    const uint16_t *arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid + 256 * i) >> 3;
        int m = m0 + r;
        if (m >= m_end) m = m0;  // padding rows repeat a valid row; never stored
        if (GATEUP)
            arow[i] = a.x + (int64_t)(a.perm[m] / a.K) * a.d;
        else
            arow[i] = a.H + (int64_t)m * a.f;
    }
    const int akb = tid & 7;
    auto stage = [&](int g, int buf) {
        u32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const u32x4 *>(arow[i] + g * kGroup + akb * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid + 256 * i) >> 3;
            *reinterpret_cast<u32x4 *>(&s_a[buf][r * kARowPad + akb * 8]) = permute8(v[i]);
        }
    };

    // B: this lane's column of each matrix.
    rsrc_t qr[NM], sr[NM], br[NM];
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) {
        const int mi = GATEUP ? mt : 2;
        qr[mt] = make_rsrc(part_at(a.layer.p[3 * mi + 0], 0, e), (uint32_t)Nall * Kdim / 2);
        sr[mt] = make_rsrc(part_at(a.layer.p[3 * mi + 1], 0, e), (uint32_t)Nall * ngroups * 2);
        br[mt] = make_rsrc(part_at(a.layer.p[3 * mi + 2], 0, e), (uint32_t)Nall * ngroups * 2);
    }
    uint32_t km, kc;
    __asm__("v_mov_b32 %0, 0x000f000f" : "=v"(km));
    __asm__("v_mov_b32 %0, 0x64006400" : "=v"(kc));

    f16v acc[NM][4];
#pragma unroll
    for (int mt = 0; mt < NM; ++mt)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[mt][mb][v] = 0.0f;

    // Weight fragments of group g: one 16-byte code load and one scale/bias
    // pair per matrix; fetched one group ahead of their use.
    u32x4 qv[NM], qn[NM];
    uint32_t sbv[NM], sbn[NM];
    auto fetch_b = [&](int g, u32x4 (&q)[NM], uint32_t (&sb)[NM]) {
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) {
            q[mt] = ld128(qr[mt], (uint32_t)col * (Kdim / 2) + g * 32 + h * 16);
            const uint32_t so = sb_index((uint32_t)col, (uint32_t)g, (uint32_t)ngroups) * 2;
            sb[mt] = (uint32_t)ld16(sr[mt], so) | ((uint32_t)ld16(br[mt], so) << 16);
        }
    };
    fetch_b(0, qv, sbv);
    stage(0, 0);
    __syncthreads();
    for (int g = 0; g < ngroups; ++g) {
        const int buf = g & 1;
        if (g + 1 < ngroups) {
            fetch_b(g + 1, qn, sbn);
            stage(g + 1, buf ^ 1);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h8 bfrag[NM];
#pragma unroll
            for (int mt = 0; mt < NM; ++mt) {
                const f16x2 sb = as_h2(sbv[mt]);
                bfrag[mt] = dequant_word(qv[mt][j], f16x2{sb[0], sb[0]}, f16x2{sb[1], sb[1]}, km, kc);
            }
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const h8 afrag = *reinterpret_cast<const h8 *>(&s_a[buf][(mb * 32 + (lane & 31)) * kARowPad + (h * 4 + j) * 8]);
#pragma unroll
                for (int mt = 0; mt < NM; ++mt)
                    acc[mt][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afrag, bfrag[mt], acc[mt][mb], 0, 0, 0);
            }
        }
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) {
            qv[mt] = qn[mt];
            sbv[mt] = sbn[mt];
        }
        __syncthreads();
    }

    // Epilogue. C layout: lane, v -> row 8 (v / 4) + 4 h + v % 4, column lane % 32.
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = m0 + mb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            if (m >= m_end) continue;
            if (GATEUP) {
                const float gv = acc[0][mb][v], uv = acc[NM - 1][mb][v];
                const float hv = gv * __builtin_amdgcn_rcpf(1.0f + expf(-gv)) * uv;
                a.H[(int64_t)m * a.f + col] = __builtin_bit_cast(uint16_t, (f16)hv);
            } else {
                const int p = a.perm[m];
                a.Yb[(int64_t)p * a.d + col] = a.w[p] * acc[0][mb][v];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 4. combine: y[t] = sum over k, in order, of Yb[t*K + k] (already weighted).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 4 outputs each
    const int64_t tot = (int64_t)a.T * a.d / 4;
    if (i >= tot) return;
    const int t = (int)(i / (a.d / 4));
    const int c4 = (int)(i % (a.d / 4));
    f32x4 s = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < a.K; ++k) {
        const int e = a.idx[(int64_t)t * a.K + k];
        if (e < 0 || e >= a.E) continue;
        s += *reinterpret_cast<const f32x4 *>(a.Yb + ((int64_t)t * a.K + k) * a.d + 4 * c4);
    }
    *reinterpret_cast<f32x4 *>(a.y + (int64_t)t * a.d + 4 * c4) = s;
}

struct PLayout {
    size_t off, perm, ntiles, tile_e, tile_m0, H, Yb, total;
    int max_tiles;
};

PLayout prefill_layout(int T, int K, int E, int d, int f) {
    PLayout o;
    const int64_t n = (int64_t)T * K;
    o.max_tiles = (int)((n + kTM - 1) / kTM + E);
    size_t p = 0;
    o.off = p;
    p = e0_align(p + sizeof(int32_t) * (E + 1));
    o.perm = p;
    p = e0_align(p + sizeof(int32_t) * (size_t)n);
    o.ntiles = p;
    p = e0_align(p + sizeof(int32_t));
    o.tile_e = p;
    p = e0_align(p + sizeof(int32_t) * o.max_tiles);
    o.tile_m0 = p;
    p = e0_align(p + sizeof(int32_t) * o.max_tiles);
    o.H = p;
    p = e0_align(p + sizeof(uint16_t) * (size_t)n * f);
    o.Yb = p;
    p = e0_align(p + sizeof(float) * (size_t)n * d);
    o.total = p;
    return o;
}

bool stack_ok(const e0_stack *s) {
    for (int i = 0; i < 9; ++i) {
        const e0_part &p = s->part[i];
        if (!p.ptr) return false;
        if ((reinterpret_cast<uintptr_t>(p.ptr) | (uintptr_t)p.slot_stride) & 15) return false;
    }
    return true;
}

}  // namespace

size_t e0_prefill_workspace_bytes(const e0_moe_dims *dims, int32_t T) {
    if (!dims || T < 0) return 0;
    return prefill_layout(T, dims->top_k, dims->n_experts, dims->d_model, dims->d_ff).total;
}

extern "C" e0_status e0_moe_sorted_prefill(const e0_moe_dims *dims, int32_t T, const uint16_t *x, const int32_t *idx,
                                           const float *w, const e0_stack *layer, float *y, void *ws, size_t ws_bytes,
                                           int32_t *dev_err, void *stream) {
    E0_REQUIRE(dims && layer, E0_ERR_INVALID_ARG);
    const int d = dims->d_model, f = dims->d_ff, E = dims->n_experts, K = dims->top_k;
    E0_REQUIRE(T >= 0 && E >= 1 && K >= 1, E0_ERR_INVALID_ARG);
    E0_REQUIRE(d > 0 && f > 0 && d % kTN == 0 && f % kTN == 0, E0_ERR_UNSUPPORTED_SHAPE);
    E0_REQUIRE(K <= E && E <= 1024 && K <= 32, E0_ERR_UNSUPPORTED_SHAPE);
    const int64_t n = (int64_t)T * K;
    E0_REQUIRE(n <= (1 << 24), E0_ERR_CAPACITY);
    E0_REQUIRE(x && idx && w && y && dev_err, E0_ERR_INVALID_ARG);
    E0_REQUIRE(stack_ok(layer), E0_ERR_INVALID_ARG);
    E0_REQUIRE((reinterpret_cast<uintptr_t>(x) & 15) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0,
               E0_ERR_INVALID_ARG);
    const PLayout lay = prefill_layout(T, K, E, d, f);
    E0_REQUIRE(ws && ws_bytes >= lay.total && (reinterpret_cast<uintptr_t>(ws) & 255) == 0, E0_ERR_CAPACITY);
    // Expert byte ranges addressed with 32-bit offsets.
    E0_REQUIRE((int64_t)d * f / 2 < (int64_t)1 << 31, E0_ERR_UNSUPPORTED_SHAPE);
    if (T == 0) return E0_OK;

    char *wsb = static_cast<char *>(ws);
    PrefillArgs a{};
    a.T = T;
    a.K = K;
    a.E = E;
    a.d = d;
    a.f = f;
    a.n = (int)n;
    a.x = x;
    a.idx = idx;
    a.w = w;
    a.layer = to_stack(*layer);
    a.y = y;
    a.err = dev_err;
    a.off = reinterpret_cast<int32_t *>(wsb + lay.off);
    a.perm = reinterpret_cast<int32_t *>(wsb + lay.perm);
    a.ntiles = reinterpret_cast<int32_t *>(wsb + lay.ntiles);
    a.tile_e = reinterpret_cast<int32_t *>(wsb + lay.tile_e);
    a.tile_m0 = reinterpret_cast<int32_t *>(wsb + lay.tile_m0);
    a.H = reinterpret_cast<uint16_t *>(wsb + lay.H);
    a.Yb = reinterpret_cast<float *>(wsb + lay.Yb);
    a.max_tiles = lay.max_tiles;

    hipStream_t st = static_cast<hipStream_t>(stream);
    e0_status s;
    hipLaunchKernelGGL(prefill_sort_kernel, dim3(1), dim3(kSortThreads), 0, st, a);
    if ((s = e0_launch_status())) return s;
    hipLaunchKernelGGL(prefill_gemm_kernel<true>, dim3(lay.max_tiles * (f / kTN)), dim3(kGemmThreads), 0, st, a);
    if ((s = e0_launch_status())) return s;
    hipLaunchKernelGGL(prefill_gemm_kernel<false>, dim3(lay.max_tiles * (d / kTN)), dim3(kGemmThreads), 0, st, a);
    if ((s = e0_launch_status())) return s;
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((unsigned)(((int64_t)T * d / 4 + 255) / 256)), dim3(256), 0, st, a);
    return e0_launch_status();
}
