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
//               counters, one scan, scatter of the pair index and its routing
//               weight), the row offset of every expert and the list of
//               128-row M-tiles.
//  2. gemm1    (tiles x d_ff/128): H = silu(X G^T) * (X U^T) for one M-tile
//               and 128 columns of d_ff, X gathered through the sort; H fp16.
//  3. gemm2    (tiles x d_model/256): Yb[pair] = w_pair * (H D^T).
//  4. combine  : y[t] = sum over k in order of Yb[t*K + k].
// The last M-tile of an expert runs only the 32-row MFMA blocks that hold
// rows; an expert with at most 16 rows (the popularity tail) runs its own path.
// Tiles are dealt to the eight XCDs, heaviest first.
//
// MFMA v_mfma_f32_32x32x16_f16 on fp16 operands. A rows go from global memory
// straight into LDS; B fragments are code words dequantised in registers (one
// fp16 fma per weight, a single rounding of the exact dequantised value).
// Experts of at most 16 rows: v_mfma_f32_16x16x32_f16 with the code words as
// exact fp16 denormals, the group scale applied to the products in fp32 and
// the bias as a product of the rows' group sums with the biases.
#include "e0_internal.h"

#include <math.h>

#include <type_traits>

namespace {

constexpr int kTM = 128;         // rows per M-tile
constexpr int kGemmThreads = 256;
constexpr int kSortThreads = 1024;
constexpr int kMaxSortE = 1024;
constexpr int kSortBatch = 8;    // pairs per thread whose loads are issued together
constexpr int kStepK = 128;      // reduction inputs per pipeline step (two groups)
constexpr int kARow = kStepK;    // halves per LDS row of A (XOR-swizzled chunks, no padding)

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
    float *wsort;       // [n] routing weight of the pair at each sorted row
    int32_t *ntiles;    // [2]: all tiles, tiles of the heaviest class
    int32_t *tile_e;    // [max_tiles]
    int32_t *tile_m0;   // [max_tiles]
    uint16_t *H;        // [n][f] fp16
    float *Yb;          // [n][d] weighted down outputs, by pair index
    int max_tiles;
};

// ---------------------------------------------------------------------------
// 1. sort (one workgroup)
// ---------------------------------------------------------------------------
// Exclusive scan of four ints per thread over the workgroup, all four in one
// pass (one pair of barriers).
E0_DEV void block_scan4_1024(const int (&v)[4], int (&ex)[4], int (&total)[4], int (*lds)[4]) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int inc[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t = __shfl_up(inc[k], o);
            if (lane >= o) inc[k] += t;
        }
    }
    if (lane == 63)
#pragma unroll
        for (int k = 0; k < 4; ++k) lds[wv][k] = inc[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int base = 0, tot = 0;
        for (int i = 0; i < kSortThreads / 64; ++i) {
            const int t = lds[i][k];
            if (i < wv) base += t;
            tot += t;
        }
        ex[k] = base + inc[k] - v[k];
        total[k] = tot;
    }
    __syncthreads();
}

// Cost class of an M-tile holding r rows: the GEMM runs 4, 2 or 1 blocks of
// 32 rows for it.
E0_DEV int tile_class(int r) { return r > 64 ? 0 : r > 32 ? 1 : 2; }

// One workgroup. Every global store comes after the last barrier: a barrier
// also waits for the workgroup's outstanding stores, so stores issued before
// one would be waited for there.
__global__ __launch_bounds__(kSortThreads) void prefill_sort_kernel(PrefillArgs a) {
    __shared__ int s_cnt[kMaxSortE];
    __shared__ int s_fill[kMaxSortE];
    __shared__ int s_scan[kSortThreads / 64][4];
    const int tid = threadIdx.x;
    const int E = a.E, n = a.n;
    // The ids and weights of the first batch of pairs are loaded first and
    // stay in registers; each later batch is loaded whole before its atomics,
    // so the global loads overlap instead of waiting one by one.
    int ids0[kSortBatch];
    float wts0[kSortBatch];
#pragma unroll
    for (int i = 0; i < kSortBatch; ++i) {
        const int p = i * kSortThreads + tid;
        ids0[i] = p < n ? a.idx[p] : -1;
        wts0[i] = p < n ? a.w[p] : 0.0f;
    }
    for (int e = tid; e < E; e += kSortThreads) s_cnt[e] = 0;
    __syncthreads();
    // Counts per expert (LDS atomics; the counts do not depend on their order).
    int bad = 0;
    for (int base = 0; base < n; base += kSortThreads * kSortBatch) {
        int ids[kSortBatch];
#pragma unroll
        for (int i = 0; i < kSortBatch; ++i) {
            const int p = base + i * kSortThreads + tid;
            ids[i] = base == 0 ? ids0[i] : p < n ? a.idx[p] : 0;
        }
#pragma unroll
        for (int i = 0; i < kSortBatch; ++i) {
            if (base + i * kSortThreads + tid >= n) continue;
            const int e = ids[i];
            if (e >= 0 && e < E)
                atomicAdd(&s_cnt[e], 1);
            else
                bad = 1;
        }
    }
    __syncthreads();
    // Exclusive scans: first sorted row of each expert, and the position of
    // each of its M-tiles in the tile list. The list holds the tiles by cost
    // class (128-row tiles and tails above 64 rows, then tails of 33..64
    // rows, then tails of at most 32), each class in expert order.
    const int eper = (E + kSortThreads - 1) / kSortThreads;
    int cnt4[4] = {0, 0, 0, 0};  // rows, tiles of class 0, 1, 2
    for (int e = tid * eper; e < (tid + 1) * eper && e < E; ++e) {
        const int c = s_cnt[e];
        cnt4[0] += c;
        cnt4[1] += c / kTM;
        if (c % kTM) ++cnt4[1 + tile_class(c % kTM)];
    }
    int ex[4], tot[4];
    block_scan4_1024(cnt4, ex, tot, s_scan);
    int run = ex[0];
    for (int e = tid * eper; e < (tid + 1) * eper && e < E; ++e) {
        s_fill[e] = run;
        run += s_cnt[e];
    }
    __syncthreads();
    // Scatter. The order of rows inside an expert's block follows the LDS
    // atomics and may differ from run to run; no output depends on it (every
    // GEMM row is computed on its own, with the same arithmetic in whichever
    // of its expert's tiles it falls, and results are stored by pair index).
    for (int base = 0; base < n; base += kSortThreads * kSortBatch) {
        int ids[kSortBatch];
        float wts[kSortBatch];
#pragma unroll
        for (int i = 0; i < kSortBatch; ++i) {
            const int p = base + i * kSortThreads + tid;
            ids[i] = base == 0 ? ids0[i] : p < n ? a.idx[p] : -1;
            wts[i] = base == 0 ? wts0[i] : p < n ? a.w[p] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kSortBatch; ++i) {
            const int e = ids[i];
            if (e >= 0 && e < E) {
                const int row = atomicAdd(&s_fill[e], 1);
                a.perm[row] = base + i * kSortThreads + tid;
                a.wsort[row] = wts[i];
            }
        }
    }
    // Expert offsets and the tile list.
    int pos[3] = {ex[1], tot[1] + ex[2], tot[1] + tot[2] + ex[3]};
    run = ex[0];
    for (int e = tid * eper; e < (tid + 1) * eper && e < E; ++e) {
        const int c = s_cnt[e];
        a.off[e] = run;
        int m = 0;
        for (; m + kTM <= c; m += kTM, ++pos[0]) {
            a.tile_e[pos[0]] = e;
            a.tile_m0[pos[0]] = run + m;
        }
        if (m < c) {
            const int k = tile_class(c - m);
            const int q = k == 0 ? pos[0]++ : k == 1 ? pos[1]++ : pos[2]++;
            a.tile_e[q] = e;
            a.tile_m0[q] = run + m;
        }
        run += c;
    }
    if (bad) set_err(a.err, E0_DEV_BAD_ID);
    if (tid == 0) {
        a.off[E] = tot[0];
        a.ntiles[0] = tot[1] + tot[2] + tot[3];
        a.ntiles[1] = tot[1];  // tiles of the heaviest class (the first ones of the list)
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

// One 128-row M-tile (rows m0 .. of expert e) times 32 * NB * 4 output
// columns, of which the first NMB 32-row blocks are computed. GATEUP: the two
// B operands of a wave are the gate and the up column of one d_ff index, and
// the epilogue stores H = silu(gate) * up. Down (NB 1 or 2): the B operands
// are NB adjacent 32-column blocks of d_model, and the epilogue stores the
// weighted row w_pair * (H D^T).
//
// Pipeline step = 128 inputs = two quantisation groups. Lane half h owns
// group 2s + h of step s whole: its eight code words (32 contiguous bytes of
// its column) and one scale/bias pair; MFMA j takes word j of each half, so
// its 16-wide reduction slice is inputs 8j..8j+7 of both groups.
//
// A rows go from global memory straight into LDS (global_load_lds_dwordx4:
// lane L of a wave's load lands at the wave's LDS base + 16 L), so a load
// covers four rows of 16 chunks; a lane fetches chunk c' ^ (row % 16) for LDS
// slot c', which makes the fragment reads (32 rows, one chunk) conflict-free.
// The rows and weights of step s + 1 are requested before the MFMAs of step
// s and waited for after them. Inside a step, word j + 1 is dequantised and
// its A fragments read in slices between the MFMAs of word j.
template <int NB, bool GATEUP, int NMB>
E0_DEV void prefill_tile(const PrefillArgs &a, uint16_t (*s_a)[kTM * kARow], int e, int m0, int m_end, int nt) {
    constexpr int kCols = 4 * 32 * (GATEUP ? 1 : NB);  // output columns per workgroup
    constexpr int kMf = NMB * NB;                      // MFMAs per code word
    constexpr int kPairs = 4 * NB;                     // weight pairs per code word set
    const int Nall = GATEUP ? a.f : a.d;
    const int Kdim = GATEUP ? a.d : a.f;
    const int ngroups = Kdim / kGroup;
    const int nsteps = Kdim / kStepK;
    const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
    const int h = lane >> 5;

    // A staging: wave wv loads rows 32 wv .. 32 wv + 31 (only waves below NMB),
    // load i covering rows 32 wv + 4 i + lane / 16.
    const int lrow = lane >> 4, lslot = lane & 15;
    const uint16_t *abase = GATEUP ? a.x : a.H;
    const int64_t alen = GATEUP ? a.d : a.f;
    int arow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int m = m0 + wv * 32 + 4 * i + lrow;
        if (m >= m_end) m = m0;  // padding rows repeat a valid row; never stored
        arow[i] = GATEUP ? a.perm[m] / a.K : m;
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)&s_a[0][0];
    auto load_a = [&](int st, int buf) {
        if (wv >= NMB) return;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = wv * 32 + 4 * i + lrow;
            const int c = lslot ^ (r & 15);
            const uint16_t *src = abase + arow[i] * alen + st * kStepK + c * 8;
            const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(buf * kTM * kARow + (wv * 32 + 4 * i) * kStepK) * 2);
            // m0 holds the wave's LDS destination (lane L lands at m0 + 16 L);
            // the {m0} operand makes the compiler set it and know it is used.
            asm volatile("global_load_lds_dwordx4 %1, off" ::"{m0}"(dst), "v"(src) : "memory");
        }
    };

    // Down: pair index and weight of row tid (tid < 128), loaded now and
    // parked in LDS after the main loop for the epilogue.
    int my_p = 0;
    float my_w = 0.0f;
    if (!GATEUP && tid < kTM && m0 + tid < m_end) {
        my_p = a.perm[m0 + tid];
        my_w = a.wsort[m0 + tid];
    }

    // B operands: part base of each and this lane's column.
    rsrc_t qr[NB], sr[NB], br[NB];
    uint32_t colb[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        const int mi = GATEUP ? n : 2;
        qr[n] = make_rsrc(part_at(a.layer.p[3 * mi + 0], 0, e), (uint32_t)Nall * Kdim / 2);
        sr[n] = make_rsrc(part_at(a.layer.p[3 * mi + 1], 0, e), (uint32_t)Nall * ngroups * 2);
        br[n] = make_rsrc(part_at(a.layer.p[3 * mi + 2], 0, e), (uint32_t)Nall * ngroups * 2);
        colb[n] = GATEUP ? nt * kCols + wv * 32 + (lane & 31) : nt * kCols + wv * 32 * NB + n * 32 + (lane & 31);
    }
    // Scale and bias stay apart until their use: packing them right after
    // the loads would wait for those loads, and with them for every load
    // issued before.
    struct Bst {
        u32x4 q[NB][2];
        uint32_t s[NB], b[NB];
    };
    auto fetch_b = [&](int st, Bst &b) {
        const int g = 2 * st + h;
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const uint32_t qo = colb[n] * (uint32_t)(Kdim / 2) + g * 32;
            b.q[n][0] = ld128(qr[n], qo);
            b.q[n][1] = ld128(qr[n], qo + 16);
            const uint32_t so = sb_index(colb[n], (uint32_t)g, (uint32_t)ngroups) * 2;
            b.s[n] = ld16(sr[n], so);
            b.b[n] = ld16(br[n], so);
        }
    };
    uint32_t km, kc;
    __asm__("v_mov_b32 %0, 0x00f0000f" : "=v"(km));
    __asm__("v_mov_b32 %0, 0x64006400" : "=v"(kc));

    f16v acc[NB][NMB];
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[n][mb][v] = 0.0f;

    // Fragment of rows mb*32 .. +31, chunk h*8 + j (inputs h*64 + 8j ..).
    auto afrag = [&](int buf, int mb, int j) {
        const int r = mb * 32 + (lane & 31);
        const int c = (h * 8 + j) ^ (r & 15);
        return *reinterpret_cast<const h8 *>(&s_a[buf][r * kStepK + c * 8]);
    };
    // Pairs p0 .. p0 + N - 1 of code word j, dequantised stage by stage (all
    // byte placements, then all masks, then both fmas of every pair), so the N
    // dependency chains overlap instead of running one after another.
    auto dq_pairs = [&](const Bst &b, int j, int p0, auto &dst, auto cnt) {
        constexpr int N = decltype(cnt)::value;
        uint32_t t[N];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int p = p0 + i;
            t[i] = __builtin_amdgcn_perm(b.q[p >> 2][j >> 2][j & 3], b.q[p >> 2][j >> 2][j & 3],
                                         0x0c000c00u | (uint32_t)(p & 3) << 16 | (uint32_t)(p & 3));
        }
#pragma unroll
        for (int i = 0; i < N; ++i) t[i] = and_or_v(t[i], km, kc);
        const f16x2 kmul = f16x2{(f16)1.0f, (f16)0.0625f};
        const f16x2 kadd = f16x2{(f16)-1024.0f, (f16)-64.0f};
        f16x2 q[N];
#pragma unroll
        for (int i = 0; i < N; ++i) q[i] = __builtin_elementwise_fma(as_h2(t[i]), kmul, kadd);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int p = p0 + i, n = p >> 2;
            const f16 sv = __builtin_bit_cast(f16, (uint16_t)b.s[n]), bv = __builtin_bit_cast(f16, (uint16_t)b.b[n]);
            const f16x2 v = __builtin_elementwise_fma(q[i], f16x2{sv, sv}, f16x2{bv, bv});
            dst[n][2 * (p & 3)] = v[0];
            dst[n][2 * (p & 3) + 1] = v[1];
        }
    };
    // MFMAs in windows of two; each window also dequantises its share of the
    // next code word (kPairs / (kMf / 2) pairs) and reads the next A
    // fragments, with a scheduling barrier between windows.
    constexpr int kWin = kMf >= 2 ? 2 : 1;
    constexpr int kPpw = kPairs / (kMf / kWin);
    auto compute = [&](int buf, const Bst &b) {
        h8 bcur[NB], af[NMB];
        dq_pairs(b, 0, 0, bcur, std::integral_constant<int, kPairs>{});
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) af[mb] = afrag(buf, mb, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            h8 bnx[NB], afn[NMB];
#pragma unroll
            for (int w0 = 0; w0 < kMf; w0 += kWin) {
#pragma unroll
                for (int k = w0; k < w0 + kWin; ++k) {
                    const int mb = k / NB, n = k % NB;
                    acc[n][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mb], bcur[n], acc[n][mb], 0, 0, 0);
                }
                if (j < 7) {
                    dq_pairs(b, j + 1, (w0 / kWin) * kPpw, bnx, std::integral_constant<int, kPpw>{});
#pragma unroll
                    for (int k = w0; k < w0 + kWin; ++k)
                        if (k % NB == 0) afn[k / NB] = afrag(buf, k / NB, j + 1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (j < 7) {
#pragma unroll
                for (int n = 0; n < NB; ++n) bcur[n] = bnx[n];
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) af[mb] = afn[mb];
            }
        }
    };

    // Step st: request the rows (into LDS buffer (st + 1) & 1) and weights of
    // step st + 1, run the MFMAs of step st from buffer st & 1, then wait for
    // all of them before the barrier.
    Bst cur, next;
    fetch_b(0, cur);
    load_a(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const bool more = st + 1 < nsteps;
        if (more) {
            load_a(st + 1, (st + 1) & 1);
            fetch_b(st + 1, next);
        }
        compute(st & 1, cur);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (more) cur = next;
        __syncthreads();
    }

    // Epilogue. C layout: lane, v -> row 8 (v / 4) + 4 h + v % 4, column lane % 32.
    int *s_p = reinterpret_cast<int *>(&s_a[0][0]);
    float *s_w = reinterpret_cast<float *>(&s_a[0][0]) + kTM;
    if (!GATEUP) {
        if (tid < kTM) {
            s_p[tid] = my_p;
            s_w[tid] = my_w;
        }
        __syncthreads();
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = m0 + mb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            if (m >= m_end) continue;
            if (GATEUP) {
                const float gv = acc[0][mb][v], uv = acc[1][mb][v];
                const float hv = gv * __builtin_amdgcn_rcpf(1.0f + expf(-gv)) * uv;
                a.H[(int64_t)m * a.f + colb[0]] = __builtin_bit_cast(uint16_t, (f16)hv);
            } else {
                const int r = m - m0;
                const int p = s_p[r];
                const float wp = s_w[r];
#pragma unroll
                for (int n = 0; n < NB; ++n) a.Yb[(int64_t)p * a.d + colb[n]] = wp * acc[n][mb][v];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Experts with at most 16 rows (one tile): most active experts of a layer
// receive only a few of its pairs (the popularity tail), and a 32-row block
// would compute padding while every weight of the tile is still dequantised.
// Only whole experts take this path: the sort orders an expert's rows by its
// LDS atomics, so which rows fall in the tail tile of a larger expert can
// change from run to run, and a row must get the same arithmetic whichever
// tile holds it (every output is then the same from run to run). Here the
// matrix cores take v_mfma_f32_16x16x32_f16 with the code words themselves
// as the B operand, fp16 denormals q 2^-24 (exact), so no weight is
// dequantised: the two MFMAs of quantisation group g give P_g = 2^-24
// sum_k q_k x_k for 16 rows x 16 columns, and the group adds s_g 2^24 P_g
// (one fma per output). The bias part, sum_g b_g sum_{k in g} x_k, is itself
// a product over the groups: the rows' group sums X (fp32, as fp16 hi + lo)
// against the fp16 biases, two MFMAs per 32 groups after the main loop.
// Every product is exact in fp32; the dequantised weight s q + b is never
// rounded to fp16 (the 128-row tiles round it once).
//
// Lane (n = lane % 16, kq = lane / 16): A row n, B column n (the wavefront's
// output column 16 cb + n), over inputs 32 (kq & 1) + 8 (kq >> 1) + 16 s .. + 7
// of group g for the slices s = 0, 1; C rows 4 kq .. 4 kq + 3 of column n.
// A code word (8 codes, the lowest nibble first) becomes (q0, q4, 16 q1,
// 16 q5, q2, q6, 16 q3, 16 q7) x 2^-24 by one shift and four masks; the rows
// are staged in LDS in the same order, the positions of 16 q scaled by 1/16
// (exact for |x| >= 2^-10; below that the fp16 quotient is subnormal and keeps
// fewer bits). Each lane loads 16 bytes of its column per 128-input step (64
// contiguous bytes per column: group 2 st in lanes 0-31, 2 st + 1 in lanes
// 32-63); two lane swaps leave registers that each hold one group.
constexpr int kSmallRowPad = 136;     // halves per staged row: 16 chunks + one (rows start on other banks)
constexpr int kSmallMaxGroups = 256;  // group sums kept in LDS (reduction length up to 16384)

typedef float f4v __attribute__((ext_vector_type(4)));

// (x_j, x_{j+4}) pairs of 8 consecutive fp16 values in the MFMA order above,
// the pairs that meet 16 q scaled by 1/16.
E0_DEV u32x4 small_a_chunk(u32x4 x) {
    const f16x2 k16 = f16x2{(f16)0.0625f, (f16)0.0625f};
    u32x4 o;
    o[0] = __builtin_amdgcn_perm(x[2], x[0], 0x05040100u);
    o[1] = __builtin_bit_cast(uint32_t, as_h2(__builtin_amdgcn_perm(x[2], x[0], 0x07060302u)) * k16);
    o[2] = __builtin_amdgcn_perm(x[3], x[1], 0x05040100u);
    o[3] = __builtin_bit_cast(uint32_t, as_h2(__builtin_amdgcn_perm(x[3], x[1], 0x07060302u)) * k16);
    return o;
}

// A code word as the B operand: (q0, q4, 16 q1, 16 q5, q2, q6, 16 q3, 16 q7) x 2^-24.
E0_DEV h8 small_b_word(uint32_t w) {
    const uint32_t w8 = w >> 8;
    return __builtin_bit_cast(h8, u32x4{w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u});
}

template <int NB, bool GATEUP>
E0_DEV void prefill_small_tile(const PrefillArgs &a, uint16_t (*s_a)[kTM * kARow], int e, int m0, int m_end, int nt) {
    constexpr int kCols = 4 * 32 * (GATEUP ? 1 : NB);
    constexpr int kNcb = GATEUP ? 4 : 2 * NB;  // 16-column blocks per wavefront (gate/up: gate 0-1, up 2-3)
    constexpr int kMats = GATEUP ? 2 : 1;
    constexpr float kDenorm = 16777216.0f;    // 2^24
    const int Kdim = GATEUP ? a.d : a.f;
    const int Nall = GATEUP ? a.f : a.d;
    const int ngroups = Kdim / kGroup;
    const int nsteps = Kdim / kStepK;
    const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
    const int nl = lane & 15, kq = lane >> 4;

    uint16_t *sA = &s_a[0][0];                                      // [2][16][kSmallRowPad]
    float *sX = reinterpret_cast<float *>(sA + 2 * 16 * kSmallRowPad);  // [16][ngroups] group sums

    // Staging: thread tid takes chunk c = tid % 16 (inputs 8 c .. 8 c + 7 of
    // the step) of row r = tid / 16. Rows past the tile load row m0 and stage
    // zeros.
    const int sr_ = tid >> 4, sc_ = tid & 15;
    const bool aok = m0 + sr_ < m_end;
    const int arow = GATEUP ? a.perm[aok ? m0 + sr_ : m0] / a.K : (aok ? m0 + sr_ : m0);
    const uint16_t *asrc = (GATEUP ? a.x : a.H) + (int64_t)arow * Kdim + 8 * sc_;
    const int scc = sc_ & 7, sg = sc_ >> 3;
    const int sslot = ((sg * 4 + ((scc >> 2) | ((scc & 1) << 1))) * 2 + ((scc >> 1) & 1)) * 8;
    auto stage_a = [&](int st, int buf, u32x4 x) {
        if (!aok) x = u32x4{0u, 0u, 0u, 0u};
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f16x2 p = as_h2(x[i]);
            sum += (float)p[0] + (float)p[1];
        }
        // the 8 chunks of one (row, group) are 8 consecutive lanes
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        sum += __shfl_xor(sum, 4);
        if (scc == 0) sX[sr_ * ngroups + 2 * st + sg] = sum;
        *reinterpret_cast<u32x4 *>(sA + (buf * 16 + sr_) * kSmallRowPad + sslot) = small_a_chunk(x);
    };

    rsrc_t qr[kMats], sr[kMats], br[kMats];
#pragma unroll
    for (int mi = 0; mi < kMats; ++mi) {
        const int pm = GATEUP ? mi : 2;
        qr[mi] = make_rsrc(part_at(a.layer.p[3 * pm + 0], 0, e), (uint32_t)Nall * Kdim / 2);
        sr[mi] = make_rsrc(part_at(a.layer.p[3 * pm + 1], 0, e), (uint32_t)Nall * ngroups * 2);
        br[mi] = make_rsrc(part_at(a.layer.p[3 * pm + 2], 0, e), (uint32_t)Nall * ngroups * 2);
    }
    uint32_t col[kNcb];
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb)
        col[cb] = GATEUP ? nt * kCols + wv * 32 + (cb & 1) * 16 + nl : nt * kCols + wv * 32 * NB + cb * 16 + nl;
    auto mat = [](int cb) { return GATEUP ? cb >> 1 : 0; };

    struct Stage {
        u32x4 w[kNcb];
        uint32_t s[kNcb][2];
    };
    auto fetch = [&](int st, Stage &S) {
#pragma unroll
        for (int cb = 0; cb < kNcb; ++cb) {
            S.w[cb] = ld128(qr[mat(cb)], col[cb] * (uint32_t)(Kdim / 2) + st * 64 + kq * 16);
#pragma unroll
            for (int g = 0; g < 2; ++g) S.s[cb][g] = ld16(sr[mat(cb)], sb_index(col[cb], 2 * st + g, ngroups) * 2);
        }
    };

    f4v tot[kNcb];
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb) tot[cb] = f4v{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int buf, const Stage &S) {
        u32x4 W[kNcb];
#pragma unroll
        for (int cb = 0; cb < kNcb; ++cb) {
            const auto r01 = __builtin_amdgcn_permlane32_swap(S.w[cb][0], S.w[cb][1], false, false);
            const auto r23 = __builtin_amdgcn_permlane32_swap(S.w[cb][2], S.w[cb][3], false, false);
            W[cb] = u32x4{r01[0], r01[1], r23[0], r23[1]};  // word 2 s + g: slice s of group g
        }
        const uint16_t *arow_l = sA + (buf * 16 + nl) * kSmallRowPad + kq * 16;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const h8 a0 = *reinterpret_cast<const h8 *>(arow_l + g * 64);
            const h8 a1 = *reinterpret_cast<const h8 *>(arow_l + g * 64 + 8);
#pragma unroll
            for (int cb = 0; cb < kNcb; ++cb) {
                f4v P = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, small_b_word(W[cb][g]), f4v{0.0f, 0.0f, 0.0f, 0.0f},
                                                               0, 0, 0);
                P = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, small_b_word(W[cb][2 + g]), P, 0, 0, 0);
                const float sc = h2f((uint16_t)S.s[cb][g]) * kDenorm;
#pragma unroll
                for (int i = 0; i < 4; ++i) tot[cb][i] = __builtin_fmaf(sc, P[i], tot[cb][i]);
            }
        }
    };

    // Step st: request the rows and weights of step st + 1, compute step st
    // from LDS buffer st & 1, wait, stage the next rows, barrier.
    Stage cur, nxt;
    fetch(0, cur);
    u32x4 av = *reinterpret_cast<const u32x4 *>(asrc);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    stage_a(0, 0, av);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const bool more = st + 1 < nsteps;
        if (more) {
            av = *reinterpret_cast<const u32x4 *>(asrc + (st + 1) * kStepK);
            fetch(st + 1, nxt);
        }
        compute(st & 1, cur);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (more) {
            stage_a(st + 1, (st + 1) & 1, av);
            cur = nxt;
        }
        __syncthreads();
    }

    // Bias part: B' = biases of groups 32 c + 8 kq .. + 7 of the lane's
    // column, A' = the group sums of row n over the same groups (0 past the
    // last group), as fp16 hi + lo.
    for (int c = 0; c * 32 < ngroups; ++c) {
        h8 xh, xl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int g = 32 * c + 8 * kq + j;
            const float v = g < ngroups ? sX[nl * ngroups + g] : 0.0f;
            const f16 h = (f16)v;
            xh[j] = h;
            xl[j] = (f16)(v - (float)h);
        }
#pragma unroll
        for (int cb = 0; cb < kNcb; ++cb) {
            h8 bb;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int g = 32 * c + 8 * kq + j;
                const uint16_t bv = ld16(br[mat(cb)], sb_index(col[cb], (uint32_t)min(g, ngroups - 1), ngroups) * 2);
                bb[j] = g < ngroups ? __builtin_bit_cast(f16, bv) : (f16)0.0f;
            }
            tot[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, bb, tot[cb], 0, 0, 0);
            tot[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl, bb, tot[cb], 0, 0, 0);
        }
    }

    // Epilogue: lane holds rows 4 kq + i of column col[cb].
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + 4 * kq + i;
        if (m >= m_end) continue;
        if (GATEUP) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const float gv = tot[cb][i], uv = tot[cb + 2][i];
                const float hv = gv * __builtin_amdgcn_rcpf(1.0f + expf(-gv)) * uv;
                a.H[(int64_t)m * a.f + col[cb]] = __builtin_bit_cast(uint16_t, (f16)hv);
            }
        } else {
            const int p = a.perm[m];
            const float wp = a.wsort[m];
#pragma unroll
            for (int cb = 0; cb < kNcb; ++cb) a.Yb[(int64_t)p * a.d + col[cb]] = wp * tot[cb][i];
        }
    }
}

template <int NB, bool GATEUP>
__global__ __launch_bounds__(kGemmThreads, 2) void prefill_gemm_kernel(PrefillArgs a) {
    static_assert(!GATEUP || NB == 2, "gate/up runs two B operands per wave");
    constexpr int kCols = 4 * 32 * (GATEUP ? 1 : NB);
    __shared__ __attribute__((aligned(16))) uint16_t s_a[2][kTM * kARow];
    const int nN = (GATEUP ? a.f : a.d) / kCols;
    // The hardware deals block b to XCD b % 8 and dispatches in block order.
    // Work items (tile, column block) of the heaviest class come first: XCD x
    // takes the x-th of eight contiguous ranges of them (about one per CU),
    // then the x-th contiguous range of the lighter ones. Contiguous ranges
    // keep the tiles of one expert, and the column blocks of one tile, on one
    // XCD, so its L2 fetches their weights and rows once; the heavy items are
    // spread over all CUs before any light one starts.
    const int nh = a.ntiles[1] * nN, nl = (a.ntiles[0] - a.ntiles[1]) * nN;
    const int ph = (nh + 7) >> 3, pl = (nl + 7) >> 3;
    const int bi = blockIdx.x >> 3, xcd = blockIdx.x & 7;
    int wi;
    if (bi < ph) {
        wi = xcd * ph + bi;
        if (wi >= nh) return;
    } else {
        const int li = xcd * pl + (bi - ph);
        if (bi - ph >= pl || li >= nl) return;
        wi = nh + li;
    }
    const int tile = wi / nN, nt = wi % nN;
    const int e = a.tile_e[tile], m0 = a.tile_m0[tile];
    const int m_end = a.off[e + 1];
    const int rows = m_end - m0;
    if (rows > 64)
        prefill_tile<NB, GATEUP, 4>(a, s_a, e, m0, m_end, nt);
    else if (rows > 32)
        prefill_tile<NB, GATEUP, 2>(a, s_a, e, m0, m_end, nt);
    else if (rows > 16 || m0 != a.off[e] || (GATEUP ? a.d : a.f) / kGroup > kSmallMaxGroups)
        prefill_tile<NB, GATEUP, 1>(a, s_a, e, m0, m_end, nt);
    else
        prefill_small_tile<NB, GATEUP>(a, s_a, e, m0, m_end, nt);
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
    // Rows are loaded before their ids are checked (every row of Yb is in
    // bounds; a skipped pair's row holds stale bytes and is dropped), so the
    // id loads and the row loads are in flight together.
    f32x4 s = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    int k = 0;
    for (; k + 4 <= a.K; k += 4) {
        int e[4];
        f32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            e[i] = a.idx[(int64_t)t * a.K + k + i];
            v[i] = *reinterpret_cast<const f32x4 *>(a.Yb + ((int64_t)t * a.K + k + i) * a.d + 4 * c4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (e[i] >= 0 && e[i] < a.E) s += v[i];
    }
    for (; k < a.K; ++k) {
        const int e = a.idx[(int64_t)t * a.K + k];
        const f32x4 v = *reinterpret_cast<const f32x4 *>(a.Yb + ((int64_t)t * a.K + k) * a.d + 4 * c4);
        if (e >= 0 && e < a.E) s += v;
    }
    *reinterpret_cast<f32x4 *>(a.y + (int64_t)t * a.d + 4 * c4) = s;
}

struct PLayout {
    size_t off, perm, wsort, ntiles, tile_e, tile_m0, H, Yb, total;
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
    o.wsort = p;
    p = e0_align(p + sizeof(float) * (size_t)n);
    o.ntiles = p;
    p = e0_align(p + sizeof(int32_t) * 2);
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
    e0_clear_stale_error();
    E0_REQUIRE(dims && layer, E0_ERR_INVALID_ARG);
    const int d = dims->d_model, f = dims->d_ff, E = dims->n_experts, K = dims->top_k;
    E0_REQUIRE(T >= 0 && E >= 1 && K >= 1, E0_ERR_INVALID_ARG);
    E0_REQUIRE(d > 0 && f > 0 && d % 128 == 0 && f % 128 == 0, E0_ERR_UNSUPPORTED_SHAPE);
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
    a.wsort = reinterpret_cast<float *>(wsb + lay.wsort);
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
    // Grids cover the largest tile count in whole groups of eight blocks;
    // blocks past the tiles the sort produced exit at once.
    // Blocks for every work item with each of the two classes rounded up to a
    // multiple of eight (blocks past the sort's items exit at once).
    auto grid = [&](int cols) { return dim3((unsigned)((((int64_t)lay.max_tiles * (cols) + 7) / 8 + 1) * 8)); };
    hipLaunchKernelGGL((prefill_gemm_kernel<2, true>), grid(f / 128), dim3(kGemmThreads), 0, st, a);
    if ((s = e0_launch_status())) return s;
    if (d % 256 == 0)
        hipLaunchKernelGGL((prefill_gemm_kernel<2, false>), grid(d / 256), dim3(kGemmThreads), 0, st, a);
    else
        hipLaunchKernelGGL((prefill_gemm_kernel<1, false>), grid(d / 128), dim3(kGemmThreads), 0, st, a);
    if ((s = e0_launch_status())) return s;
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((unsigned)(((int64_t)T * d / 4 + 255) / 256)), dim3(256), 0, st, a);
    return e0_launch_status();
}
