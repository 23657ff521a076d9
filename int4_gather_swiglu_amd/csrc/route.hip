// Routing on gfx950: the layer's own router GEMV and the routing math
// (softmax-top-K renormalised; sigmoid-group), one wavefront per token.
//
// Routing math: jaehun.me review of arXiv 2609.18063, report Appx. A
// (softmax-top-k: g = softmax(l), inds = top-k(g, K), w = g[inds]/sum g[inds];
// sigmoid-group: sigma = sigmoid(l), top-G groups by the sum of their two
// largest sigma, inds = top-k(sigma, K), w = s * sigma[inds]/(sum + 1e-20));
// 8B tier n=8, G=4, s=2.5, K=8 (report Tab. 1). The same math routes the
// router's own logits and the prerouter's predicted logits (koala.ai.kr
// prerouter section, "prediction-as-routing").
#include "e0_internal.h"

#include <math.h>

namespace {

constexpr int kMaxE = 1024;
constexpr int kRouteWaves = 4;

struct RouteArgs {
    const void *logits;  // [rows][E] fp16 or fp32
    int logits_fp16;
    int rows;            // n_layers * T
    int E;
    int mode, K, n_groups, topk_groups;
    float scale, eps;
    int32_t *idx;        // [rows][K]
    float *w;            // [rows][K]
    float *logits_out;   // [rows][E] or null (not written when it is the input)
};

// Better of (va, ea) and (vb, eb): larger value, ties to the lower id; ids < 0 lose.
E0_DEV void better(float &va, int &ea, float vb, int eb) {
    bool take = (eb >= 0) && (ea < 0 || vb > va || (vb == va && eb < ea));
    if (take) {
        va = vb;
        ea = eb;
    }
}

E0_DEV void wave_argmax(float &v, int &e) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        float ov = __shfl_xor(v, m);
        int oe = __shfl_xor(e, m);
        better(v, e, ov, oe);
    }
}

E0_DEV float sigm(float l) { return 1.0f / (1.0f + expf(-l)); }

// PL = logits per lane (E <= 64 PL): the loops below run over PL entries only.
template <int PL>
__global__ __launch_bounds__(kWave *kRouteWaves) void route_select_kernel(RouteArgs a) {
    __shared__ float lds_l[kRouteWaves][kMaxE];
    __shared__ float lds_gs[kRouteWaves][kWave];
    const int lane = threadIdx.x & 63;
    const int wv = wave_id();
    const int row = blockIdx.x * kRouteWaves + wv;
    if (row >= a.rows) return;
    const int E = a.E, K = a.K;

    float l[PL];
    bool avail[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = lane + kWave * i;
        avail[i] = false;
        l[i] = -INFINITY;
        if (e < E) {
            if (a.logits_fp16)
                l[i] = h2f(static_cast<const uint16_t *>(a.logits)[(int64_t)row * E + e]);
            else
                l[i] = static_cast<const float *>(a.logits)[(int64_t)row * E + e];
            avail[i] = true;
            if (a.logits_out) a.logits_out[(int64_t)row * E + e] = l[i];
        }
    }

    if (a.mode == 1) {
        // Group scores: sum of the two largest sigmoid scores per contiguous group.
        const int per = E / a.n_groups;
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const int e = lane + kWave * i;
            if (e < E) lds_l[wv][e] = l[i];
        }
        wave_lds_sync();
        float gs = -INFINITY;
        int gid = -1;
        if (lane < a.n_groups) {
            float b1 = -INFINITY, b2 = -INFINITY;
            for (int e = lane * per; e < (lane + 1) * per; ++e) {
                float v = lds_l[wv][e];
                if (v > b1) {
                    b2 = b1;
                    b1 = v;
                } else if (v > b2) {
                    b2 = v;
                }
            }
            gs = sigm(b1) + (per > 1 ? sigm(b2) : 0.0f);
            gid = lane;
        }
        // Keep the top-G groups (ties to the lower group id).
        bool kept = false;
        for (int j = 0; j < a.topk_groups; ++j) {
            float v = kept ? -INFINITY : gs;
            int e = kept ? -1 : gid;
            wave_argmax(v, e);
            if (lane == e) kept = true;
        }
        lds_gs[wv][lane] = kept ? 1.0f : 0.0f;
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const int e = lane + kWave * i;
            if (e < E) avail[i] = lds_gs[wv][e / per] != 0.0f;
        }
    }

    // Top-K by logit (monotone in both softmax and sigmoid), descending, ties
    // to the lower id. Lane k keeps the k-th selection.
    int my_e = -1;
    float my_l = -INFINITY;
    for (int k = 0; k < K; ++k) {
        float bv = -INFINITY;
        int be = -1;
#pragma unroll
        for (int i = 0; i < PL; ++i)
            if (avail[i]) better(bv, be, l[i], lane + kWave * i);
        wave_argmax(bv, be);
#pragma unroll
        for (int i = 0; i < PL; ++i)
            if (lane + kWave * i == be) avail[i] = false;
        if (lane == k) {
            my_e = be;
            my_l = bv;
        }
    }

    float wk;
    if (a.mode == 0) {
        const float l0 = __shfl(my_l, 0);
        const float ex = lane < K ? expf(my_l - l0) : 0.0f;
        wk = ex / wave_sum(ex);
    } else {
        const float s = lane < K ? sigm(my_l) : 0.0f;
        wk = a.scale * s / (wave_sum(s) + a.eps);
    }
    if (lane < K) {
        a.idx[(int64_t)row * K + lane] = my_e;
        a.w[(int64_t)row * K + lane] = wk;
    }
}

// Router GEMV: logits[l][t][e] = x[l][t] . wr[l][e], fp32 accumulation. One
// wavefront per (layer, expert row); the row stays in registers while the
// wave walks the layer's tokens.
constexpr int kGemvWaves = 4;
constexpr int kMaxD = 8192;

struct GemvArgs {
    const uint16_t *x;   // [L][T][d]
    const uint16_t *wr;  // [L][E][d]
    float *out;          // [L][T][E]
    int L, T, E, d;
};

__global__ __launch_bounds__(kWave *kGemvWaves) void router_gemv_kernel(GemvArgs a) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * kGemvWaves + wave_id();
    const int l = blockIdx.y;
    if (e >= a.E) return;
    // chunk c covers elements [512c, 512c + 512): 8 halves per lane
    const int chunks = (a.d + 511) / 512;
    const u32x4 *wrow = reinterpret_cast<const u32x4 *>(a.wr + ((int64_t)l * a.E + e) * a.d);
    u32x4 wreg[kMaxD / 512];
#pragma unroll
    for (int c = 0; c < kMaxD / 512; ++c) {
        wreg[c] = u32x4{0u, 0u, 0u, 0u};
        if (c < chunks && c * 512 + lane * 8 < a.d) wreg[c] = wrow[c * kWave + lane];
    }
    for (int t = 0; t < a.T; ++t) {
        const u32x4 *xrow = reinterpret_cast<const u32x4 *>(a.x + ((int64_t)l * a.T + t) * a.d);
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < kMaxD / 512; ++c) {
            if (c < chunks && c * 512 + lane * 8 < a.d) {
                u32x4 xv = xrow[c * kWave + lane];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc = __builtin_amdgcn_fdot2(as_h2(wreg[c][j]),
                                                 as_h2(xv[j]), acc, false);
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) a.out[((int64_t)l * a.T + t) * a.E + e] = acc;
    }
}

}  // namespace

e0_status e0_route_validate(const e0_route_params *p, int32_t E) {
    E0_REQUIRE(p, E0_ERR_INVALID_ARG);
    E0_REQUIRE(p->mode == 0 || p->mode == 1, E0_ERR_INVALID_ARG);
    E0_REQUIRE(E >= 1 && E <= kMaxE, E0_ERR_UNSUPPORTED_SHAPE);
    E0_REQUIRE(p->k >= 1 && p->k <= 32 && p->k <= E, E0_ERR_UNSUPPORTED_SHAPE);
    if (p->mode == 1) {
        E0_REQUIRE(p->n_groups >= 1 && p->n_groups <= kWave && E % p->n_groups == 0, E0_ERR_UNSUPPORTED_SHAPE);
        E0_REQUIRE(p->topk_groups >= 1 && p->topk_groups <= p->n_groups, E0_ERR_UNSUPPORTED_SHAPE);
        E0_REQUIRE(p->k <= p->topk_groups * (E / p->n_groups), E0_ERR_UNSUPPORTED_SHAPE);
        E0_REQUIRE(isfinite(p->scale) && isfinite(p->eps) && p->eps >= 0.0f, E0_ERR_INVALID_ARG);
    }
    return E0_OK;
}

// Enqueue the selection kernel over `rows` logit rows (used by e0_route and e0_prerouter).
e0_status e0_route_select_launch(const e0_route_params *p, int rows, int E, const void *logits, int fp16,
                                 int32_t *idx, float *w, float *logits_out, hipStream_t st) {
    if (rows == 0) return E0_OK;
    RouteArgs a{logits, fp16, rows, E, p->mode, p->k, p->n_groups, p->topk_groups, p->scale, p->eps, idx, w,
                logits_out};
    const int blocks = (rows + kRouteWaves - 1) / kRouteWaves;
    const dim3 g(blocks), b(kWave * kRouteWaves);
    if (E <= kWave)
        hipLaunchKernelGGL(route_select_kernel<1>, g, b, 0, st, a);
    else if (E <= 2 * kWave)
        hipLaunchKernelGGL(route_select_kernel<2>, g, b, 0, st, a);
    else if (E <= 4 * kWave)
        hipLaunchKernelGGL(route_select_kernel<4>, g, b, 0, st, a);
    else if (E <= 8 * kWave)
        hipLaunchKernelGGL(route_select_kernel<8>, g, b, 0, st, a);
    else
        hipLaunchKernelGGL(route_select_kernel<kMaxE / kWave>, g, b, 0, st, a);
    return e0_launch_status();
}

extern "C" e0_status e0_route(const e0_route_params *p, int32_t n_layers, int32_t T, int32_t E, const void *logits,
                              int32_t logits_fp16, const uint16_t *x, const uint16_t *w_router, int32_t d,
                              int32_t *idx, float *w, float *logits_out, void *stream) {
    e0_clear_stale_error();
    e0_status s = e0_route_validate(p, E);
    if (s) return s;
    E0_REQUIRE(n_layers >= 0 && T >= 0, E0_ERR_INVALID_ARG);
    E0_REQUIRE((int64_t)n_layers * T <= (1 << 24), E0_ERR_CAPACITY);
    E0_REQUIRE(idx && w, E0_ERR_INVALID_ARG);
    const int rows = n_layers * T;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!logits) {
        E0_REQUIRE(x && w_router && logits_out, E0_ERR_INVALID_ARG);
        E0_REQUIRE(d >= 64 && d % 64 == 0 && d <= kMaxD, E0_ERR_UNSUPPORTED_SHAPE);
        if (rows == 0) return E0_OK;
        GemvArgs g{x, w_router, logits_out, n_layers, T, E, d};
        hipLaunchKernelGGL(router_gemv_kernel, dim3((E + kGemvWaves - 1) / kGemvWaves, n_layers),
                           dim3(kWave * kGemvWaves), 0, st, g);
        if ((s = e0_launch_status())) return s;
        return e0_route_select_launch(p, rows, E, logits_out, 0, idx, w, nullptr, st);
    }
    return e0_route_select_launch(p, rows, E, logits, logits_fp16 ? 1 : 0, idx, w, logits_out, st);
}
