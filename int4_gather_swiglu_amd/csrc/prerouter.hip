// Prerouter heads on gfx950: every staged layer's head of one decode step in
// one call (three launches), its output routed by the shared routing math.
//
// Method (arXiv 2609.18063 as described on the pages):
//  - head(x) = fc2(erf-gelu(fc1(x))) + l(x), x = [hidden | current-token
//    top-K one-hot | previous-token top-K one-hot], dim = d_model + 2E
//    (xyznot.com head architecture; jaehun.me review, report 3.2;
//    discuss.pytorch.kr prerouter section);
//  - l is a linear residual warm-started from the next layer's router, so it
//    acts on the hidden state (koala.ai.kr prerouter section);
//  - the head owned by layer N at token t predicts layer N+1 at token t+1,
//    and with that one-token lead all staged layers are predicted in one
//    flush per step (koala.ai.kr; jaehun.me report 3.2);
//  - the logits go through the same softmax-top-K / sigmoid-group math and
//    are the routing (prediction-as-routing, koala.ai.kr; xyznot.com).
//
// The one-hot part of fc1 is not a dense GEMV: only the 2K columns whose
// input is 1 are read (a gather), so a head reads its hidden-part columns,
// 2K gathered columns, fc2 and the residual.
#include "e0_internal.h"

#include <math.h>

e0_status e0_route_validate(const e0_route_params *p, int32_t E);
e0_status e0_route_select_launch(const e0_route_params *p, int rows, int E, const void *logits, int fp16,
                                 int32_t *idx, float *w, float *logits_out, hipStream_t st);

namespace {

constexpr int kWaves = 4;
constexpr int kMaxD = 8192;
constexpr int kMaxB = 64;
constexpr int kMaxK = 32;

struct PrerArgs {
    int H, B, d, E, K, hid;
    const uint16_t *h;     // [H][B][d]
    const int32_t *cur;    // [H][B][K]
    const int32_t *prev;   // [H][B][K] or null
    const char *fc1_w;
    int64_t fc1_ws;
    const char *fc1_b;
    int64_t fc1_bs;
    const char *fc2_w;
    int64_t fc2_ws;
    const char *fc2_b;
    int64_t fc2_bs;
    const char *lin_w;
    int64_t lin_ws;
    float *g;      // ws [H][B][hid]
    float *lin;    // ws [H][B][E]
    float *out;    // [H][B][E]
};

E0_DEV float gelu_erf(float a) { return 0.5f * a * (1.0f + erff(a * 0.70710678118654752f)); }

// One wavefront per row of [fc1 (hid rows) ; lin (E rows)] of head j; the
// row's hidden-part columns stay in registers while the wave walks the tokens.
__global__ __launch_bounds__(kWave *kWaves) void prer_fc1_kernel(PrerArgs a) {
    const int lane = threadIdx.x & 63;
    const int j = blockIdx.y;
    const int r = blockIdx.x * kWaves + wave_id();
    if (r >= a.hid + a.E) return;
    const bool is_fc1 = r < a.hid;
    const int din = a.d + 2 * a.E;
    const uint16_t *row =
        is_fc1 ? reinterpret_cast<const uint16_t *>(a.fc1_w + (int64_t)j * a.fc1_ws) + (int64_t)r * din
               : reinterpret_cast<const uint16_t *>(a.lin_w + (int64_t)j * a.lin_ws) + (int64_t)(r - a.hid) * a.d;
    const int chunks = (a.d + 511) / 512;
    u32x4 wreg[kMaxD / 512];
#pragma unroll
    for (int c = 0; c < kMaxD / 512; ++c) {
        wreg[c] = u32x4{0u, 0u, 0u, 0u};
        if (c < chunks && c * 512 + lane * 8 < a.d) wreg[c] = *reinterpret_cast<const u32x4 *>(row + c * 512 + lane * 8);
    }
    const float bias = (is_fc1 && a.fc1_b) ? h2f(reinterpret_cast<const uint16_t *>(a.fc1_b + (int64_t)j * a.fc1_bs)[r]) : 0.0f;
    for (int b = 0; b < a.B; ++b) {
        const uint16_t *hv = a.h + ((int64_t)j * a.B + b) * a.d;
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < kMaxD / 512; ++c) {
            if (c < chunks && c * 512 + lane * 8 < a.d) {
                const u32x4 xv = *reinterpret_cast<const u32x4 *>(hv + c * 512 + lane * 8);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc = __builtin_amdgcn_fdot2(as_h2(wreg[c][q]), as_h2(xv[q]),
                                                 acc, false);
            }
        }
        if (is_fc1) {
            // The 2K one-hot columns: lane i < K takes current id i, lane K + i
            // previous id i; an id repeated in a row counts once.
            const int32_t *ids = nullptr;
            int col_base = 0, i = -1;
            if (lane < a.K) {
                ids = a.cur + ((int64_t)j * a.B + b) * a.K;
                i = lane;
                col_base = a.d;
            } else if (lane < 2 * a.K && a.prev) {
                ids = a.prev + ((int64_t)j * a.B + b) * a.K;
                i = lane - a.K;
                col_base = a.d + a.E;
            }
            if (ids) {
                const int e = ids[i];
                bool first = e >= 0 && e < a.E;
                for (int q = 0; q < i && first; ++q) first = ids[q] != e;
                if (first) acc += h2f(row[col_base + e]);
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) {
            if (is_fc1)
                a.g[((int64_t)j * a.B + b) * a.hid + r] = gelu_erf(acc + bias);
            else
                a.lin[((int64_t)j * a.B + b) * a.E + (r - a.hid)] = acc;
        }
    }
}

// The same rows for d_model <= 2048 with kRowsPerWave rows per wavefront: all
// of a wavefront's weight loads (and the hidden and the routing ids of its
// head) are issued before any is used, so each wavefront keeps 16 KB in
// flight instead of 4 KB.
constexpr int kRowsPerWave = 4;
constexpr int kSmallD = 2048;

__global__ __launch_bounds__(kWave *kWaves) void prer_fc1_rows_kernel(PrerArgs a) {
    constexpr int kC = kSmallD / 512;  // 16-byte chunks per lane of a row
    const int lane = threadIdx.x & 63;
    const int j = blockIdx.y;
    const int r0 = (blockIdx.x * kWaves + wave_id()) * kRowsPerWave;
    const int nrows = a.hid + a.E;
    if (r0 >= nrows) return;
    const int din = a.d + 2 * a.E;
    const int chunks = a.d / 512;
    // Routing id of this lane for token b (lane i < K: current id i, K + i:
    // previous id i, else none); token 0's is requested before the weights,
    // since its one-hot columns depend on it.
    auto lane_id = [&](int b) {
        int e = -1;
        if (lane < a.K) e = a.cur[((int64_t)j * a.B + b) * a.K + lane];
        else if (lane < 2 * a.K && a.prev) e = a.prev[((int64_t)j * a.B + b) * a.K + lane - a.K];
        return e;
    };
    const int id0 = lane_id(0);
    u32x4 w[kRowsPerWave][kC];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
        const int r = min(r0 + i, nrows - 1);
        const bool fc1 = r < a.hid;
        const uint16_t *row = fc1 ? reinterpret_cast<const uint16_t *>(a.fc1_w + (int64_t)j * a.fc1_ws) + (int64_t)r * din
                                  : reinterpret_cast<const uint16_t *>(a.lin_w + (int64_t)j * a.lin_ws) + (int64_t)(r - a.hid) * a.d;
#pragma unroll
        for (int c = 0; c < kC; ++c)
            w[i][c] = c < chunks ? *reinterpret_cast<const u32x4 *>(row + c * 512 + lane * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    for (int b = 0; b < a.B; ++b) {
        const uint16_t *hv = a.h + ((int64_t)j * a.B + b) * a.d;
        u32x4 xv[kC];
#pragma unroll
        for (int c = 0; c < kC; ++c)
            xv[c] = c < chunks ? *reinterpret_cast<const u32x4 *>(hv + c * 512 + lane * 8) : u32x4{0u, 0u, 0u, 0u};
        // This lane's one-hot column of each fc1 row (an id repeated in a
        // row counts once: every lane compares with the earlier lanes of its
        // list, all lanes taking part in every shuffle).
        const int e = b == 0 ? id0 : lane_id(b);
        const int base = lane < a.K ? 0 : a.K;
        bool first = e >= 0 && e < a.E && lane < 2 * a.K;
        for (int q = 0; q < a.K; ++q) {
            const int other = __shfl(e, (base + q) & 63);
            if (q < lane - base && other == e) first = false;
        }
        const int col = a.d + (lane < a.K ? 0 : a.E) + (first ? e : 0);
        float oh[kRowsPerWave];
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            const int r = min(r0 + i, nrows - 1);
            oh[i] = (first && r < a.hid)
                        ? h2f(reinterpret_cast<const uint16_t *>(a.fc1_w + (int64_t)j * a.fc1_ws)[(int64_t)r * din + col])
                        : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            const int r = r0 + i;
            float acc = oh[i];
#pragma unroll
            for (int c = 0; c < kC; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_fdot2(as_h2(w[i][c][q]), as_h2(xv[c][q]), acc, false);
            acc = wave_sum(acc);
            if (lane == 0 && r < nrows) {
                if (r < a.hid) {
                    const float bias = a.fc1_b ? h2f(reinterpret_cast<const uint16_t *>(a.fc1_b + (int64_t)j * a.fc1_bs)[r]) : 0.0f;
                    a.g[((int64_t)j * a.B + b) * a.hid + r] = gelu_erf(acc + bias);
                } else {
                    a.lin[((int64_t)j * a.B + b) * a.E + (r - a.hid)] = acc;
                }
            }
        }
    }
}

// o[j][b][e] = fc2[e] . g[j][b] + fc2_b[e] + lin[j][b][e]; one wavefront per row.
__global__ __launch_bounds__(kWave *kWaves) void prer_fc2_kernel(PrerArgs a) {
    const int lane = threadIdx.x & 63;
    const int j = blockIdx.y;
    const int e = blockIdx.x * kWaves + wave_id();
    if (e >= a.E) return;
    const uint16_t *row = reinterpret_cast<const uint16_t *>(a.fc2_w + (int64_t)j * a.fc2_ws) + (int64_t)e * a.hid;
    const float bias = a.fc2_b ? h2f(reinterpret_cast<const uint16_t *>(a.fc2_b + (int64_t)j * a.fc2_bs)[e]) : 0.0f;
    const int chunks = (a.hid + 511) / 512;
    for (int b = 0; b < a.B; ++b) {
        const float *gv = a.g + ((int64_t)j * a.B + b) * a.hid;
        float acc = 0.0f;
        for (int c = 0; c < chunks; ++c) {
            const int col = c * 512 + lane * 8;
            if (col < a.hid) {
                const u32x4 wv = *reinterpret_cast<const u32x4 *>(row + col);
                const f32x4 g0 = *reinterpret_cast<const f32x4 *>(gv + col);
                const f32x4 g1 = *reinterpret_cast<const f32x4 *>(gv + col + 4);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f16x2 w2 = as_h2(wv[q]);
                    const float x0 = q < 2 ? g0[2 * q] : g1[2 * q - 4];
                    const float x1 = q < 2 ? g0[2 * q + 1] : g1[2 * q - 3];
                    acc += (float)w2[0] * x0 + (float)w2[1] * x1;
                }
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) a.out[((int64_t)j * a.B + b) * a.E + e] = acc + bias + a.lin[((int64_t)j * a.B + b) * a.E + e];
    }
}

struct PrerLayout {
    size_t g, lin, out, total;
};

PrerLayout prer_layout(int H, int B, int E, int hid) {
    PrerLayout o;
    size_t off = 0;
    o.g = off;
    off = e0_align(off + sizeof(float) * (size_t)H * B * hid);
    o.lin = off;
    off = e0_align(off + sizeof(float) * (size_t)H * B * E);
    o.out = off;
    off = e0_align(off + sizeof(float) * (size_t)H * B * E);
    o.total = off;
    return o;
}

bool al16(const void *p, int64_t stride) { return ((reinterpret_cast<uintptr_t>(p) | (uintptr_t)stride) & 15) == 0; }

}  // namespace

size_t e0_prerouter_workspace_bytes(int32_t H, int32_t B, int32_t E, int32_t hid) {
    if (H < 0 || B < 1 || E < 1 || hid < 1) return 0;
    return prer_layout(H, B, E, hid).total;
}

extern "C" e0_status e0_prerouter(const e0_prerouter_heads *heads, int32_t n_heads, int32_t B, int32_t d, int32_t E,
                                  const uint16_t *h, const int32_t *cur_idx, const int32_t *prev_idx,
                                  const e0_route_params *p, int32_t *next_idx, float *next_w, float *logits_out,
                                  void *ws, size_t ws_bytes, void *stream) {
    e0_clear_stale_error();
    e0_status s = e0_route_validate(p, E);
    if (s) return s;
    E0_REQUIRE(heads, E0_ERR_INVALID_ARG);
    E0_REQUIRE(n_heads >= 0 && B >= 1, E0_ERR_INVALID_ARG);
    E0_REQUIRE(B <= kMaxB && p->k <= kMaxK, E0_ERR_CAPACITY);
    E0_REQUIRE(d >= 64 && d % 64 == 0 && d <= kMaxD, E0_ERR_UNSUPPORTED_SHAPE);
    const int hid = heads->hidden;
    E0_REQUIRE(hid >= 64 && hid % 64 == 0 && hid <= 2048, E0_ERR_UNSUPPORTED_SHAPE);
    E0_REQUIRE(h && cur_idx && next_idx && next_w, E0_ERR_INVALID_ARG);
    E0_REQUIRE(heads->fc1_w && heads->fc2_w && heads->lin_w, E0_ERR_INVALID_ARG);
    E0_REQUIRE((reinterpret_cast<uintptr_t>(h) & 15) == 0, E0_ERR_INVALID_ARG);
    // fc1 rows are d + 2E fp16 long: 16-byte aligned rows need (d + 2E) % 8 == 0.
    E0_REQUIRE((d + 2 * E) % 8 == 0, E0_ERR_UNSUPPORTED_SHAPE);
    E0_REQUIRE(al16(heads->fc1_w, heads->fc1_w_stride) && al16(heads->fc2_w, heads->fc2_w_stride) &&
                   al16(heads->lin_w, heads->lin_w_stride),
               E0_ERR_INVALID_ARG);
    E0_REQUIRE((heads->fc1_b_stride & 1) == 0 && (heads->fc2_b_stride & 1) == 0, E0_ERR_INVALID_ARG);
    const PrerLayout lay = prer_layout(n_heads, B, E, hid);
    E0_REQUIRE(ws && ws_bytes >= lay.total && (reinterpret_cast<uintptr_t>(ws) & 255) == 0, E0_ERR_CAPACITY);
    if (n_heads == 0) return E0_OK;

    char *wsb = static_cast<char *>(ws);
    PrerArgs a{};
    a.H = n_heads;
    a.B = B;
    a.d = d;
    a.E = E;
    a.K = p->k;
    a.hid = hid;
    a.h = h;
    a.cur = cur_idx;
    a.prev = prev_idx;
    a.fc1_w = reinterpret_cast<const char *>(heads->fc1_w);
    a.fc1_ws = heads->fc1_w_stride;
    a.fc1_b = reinterpret_cast<const char *>(heads->fc1_b);
    a.fc1_bs = heads->fc1_b_stride;
    a.fc2_w = reinterpret_cast<const char *>(heads->fc2_w);
    a.fc2_ws = heads->fc2_w_stride;
    a.fc2_b = reinterpret_cast<const char *>(heads->fc2_b);
    a.fc2_bs = heads->fc2_b_stride;
    a.lin_w = reinterpret_cast<const char *>(heads->lin_w);
    a.lin_ws = heads->lin_w_stride;
    a.g = reinterpret_cast<float *>(wsb + lay.g);
    a.lin = reinterpret_cast<float *>(wsb + lay.lin);
    a.out = logits_out ? logits_out : reinterpret_cast<float *>(wsb + lay.out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (d <= kSmallD) {
        const int per_block = kWaves * kRowsPerWave;
        hipLaunchKernelGGL(prer_fc1_rows_kernel, dim3((hid + E + per_block - 1) / per_block, n_heads), dim3(kWave * kWaves),
                           0, st, a);
    } else {
        hipLaunchKernelGGL(prer_fc1_kernel, dim3((hid + E + kWaves - 1) / kWaves, n_heads), dim3(kWave * kWaves), 0, st, a);
    }
    if ((s = e0_launch_status())) return s;
    hipLaunchKernelGGL(prer_fc2_kernel, dim3((E + kWaves - 1) / kWaves, n_heads), dim3(kWave * kWaves), 0, st, a);
    if ((s = e0_launch_status())) return s;
    return e0_route_select_launch(p, n_heads * B, E, a.out, 0, next_idx, next_w, nullptr, st);
}
