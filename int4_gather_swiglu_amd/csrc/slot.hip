// Slot update on gfx950: fixed double-buffered slots per layer, rewritten in
// place for changed experts only, with the tables kept on the GPU.
//
// Method: "staged" path with fixed double-buffered slots and a slot table,
// incr_stack rewriting only changed slots in place (koala.ai.kr paths table
// and the Appx. B note on incr_stack; jaehun.me review, report 3.1 and
// Appx. B; xyznot.com glossary, "incremental sticky-slot stack").
//
// Rule per layer (deterministic, so slot tables can be compared bit for bit):
// the next set U' and the in-use set U are read from the routing ids; an
// expert of U' already resident stays; the i-th missing expert of U' in
// ascending id takes the i-th lowest slot whose occupant is in neither U'
// nor U (or is empty). This equals assigning missing experts one at a time to
// the lowest such slot, because each assignment only removes its own slot
// from the candidates.
//
// Hot-set variant (e0_slot_update_lru): a pool larger than one step needs,
// kept as a per-layer least-recently-used cache of the store (koala.ai.kr on
// the hot path of resident experts; jaehun.me review, report 3.2 on whole-
// layer residency): every wanted expert, resident or placed, gets the step
// as its slot's last use, and the candidates are taken in ascending (last
// use, slot) order instead of ascending slot, so a miss evicts the expert
// least recently used. The result stays exact: every wanted expert is made
// resident before the decode reads it.
//
// Two launches: plan (one workgroup per layer: sets, compaction, tables, copy
// list) and copy (many workgroups: 16-byte vector copies of the nine parts,
// one linear range per expert when store and pool hold whole bundles). The
// store's bytes are read once, with the nontemporal hint; the pool's bytes
// are written with ordinary stores, which the next decode reads back: with
// nontemporal stores the overlapped decode35b step measured 173 us against
// 157 us with ordinary ones.
#include "e0_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxE = 4096;
constexpr int kMaxS = 4096;
constexpr int kCopyUnits = 2;  // 16-byte units per thread per copy block (8 KB blocks: 2-3% faster beside
                               // the decode than 16 KB ones; 32 KB and larger blocks copy at a fraction)
constexpr int kCopyChunk = kThreads * kCopyUnits * 16;
constexpr int kHostCopyBlocks = 64;  // copy blocks when the store is in host memory

struct SlotArgs {
    int L, BK, E, S;
    const int32_t *next_idx;  // [L][BK]
    const int32_t *cur_idx;   // [L][BK] or null
    int32_t *slot_of;         // [L][E]
    int32_t *expert_of;       // [L][S]
    int32_t *n_copied;        // [L] or null
    int32_t *err;
    int32_t *ncopy;           // ws [L]
    int32_t *copy_slot;       // ws [L][maxc]
    int32_t *copy_exp;        // ws [L][maxc]
    int maxc;
    int32_t *last_use;        // [L][S] last step each slot was wanted (-1 never), or null: lowest-slot rule
    int32_t step;
};

// Exclusive scan of one int per thread over the block.
E0_DEV int block_scan(int v, int *lds, int &total) {
    const int lane = threadIdx.x & 63, wv = wave_id();
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    if (lane == 63) lds[wv] = inc;
    __syncthreads();
    int base = 0;
    total = 0;
    for (int i = 0; i < kThreads / 64; ++i) {
        if (i < wv) base += lds[i];
        total += lds[i];
    }
    __syncthreads();
    return base + inc - v;
}

__global__ __launch_bounds__(kThreads) void slot_plan_kernel(SlotArgs a) {
    __shared__ unsigned char s_want[kMaxE];
    __shared__ unsigned char s_keep[kMaxE];
    __shared__ int s_miss[kMaxS];
    __shared__ int s_free[kMaxS];
    __shared__ int s_order[kMaxS];
    __shared__ int s_scan[kThreads / 64];
    const int l = blockIdx.x, tid = threadIdx.x;
    int32_t *slot_of = a.slot_of + (int64_t)l * a.E;
    int32_t *expert_of = a.expert_of + (int64_t)l * a.S;

    for (int e = tid; e < a.E; e += kThreads) s_want[e] = s_keep[e] = 0;
    __syncthreads();
    for (int p = tid; p < a.BK; p += kThreads) {
        const int e = a.next_idx[(int64_t)l * a.BK + p];
        if (e >= 0 && e < a.E)
            s_want[e] = 1;
        else
            set_err(a.err, E0_DEV_BAD_ID);
        if (a.cur_idx) {
            const int c = a.cur_idx[(int64_t)l * a.BK + p];
            if (c >= 0 && c < a.E) s_keep[c] = 1;
        }
    }
    __syncthreads();

    // Missing experts (ascending id): wanted and without a valid slot.
    const int eper = (a.E + kThreads - 1) / kThreads;
    int nm = 0;
    for (int e = tid * eper; e < (tid + 1) * eper && e < a.E; ++e) {
        const int s = slot_of[e];
        nm += s_want[e] && !(s >= 0 && s < a.S && expert_of[s] == e);
    }
    int mtot;
    int mb = block_scan(nm, s_scan, mtot);
    int32_t *last_use = a.last_use ? a.last_use + (int64_t)l * a.S : nullptr;
    for (int e = tid * eper; e < (tid + 1) * eper && e < a.E; ++e) {
        const int s = slot_of[e];
        const bool resident = s >= 0 && s < a.S && expert_of[s] == e;
        if (s_want[e] && !resident) s_miss[mb++] = e;
        if (s_want[e] && resident && last_use) last_use[s] = a.step;  // a hit (never a candidate below)
    }
    // Free slots (ascending): empty, or holding an expert in neither set.
    const int sper = (a.S + kThreads - 1) / kThreads;
    int nf = 0;
    for (int s = tid * sper; s < (tid + 1) * sper && s < a.S; ++s) {
        const int o = expert_of[s];
        nf += (o < 0 || o >= a.E) || (!s_want[o] && !s_keep[o]);
    }
    int ftot;
    int fb = block_scan(nf, s_scan, ftot);
    for (int s = tid * sper; s < (tid + 1) * sper && s < a.S; ++s) {
        const int o = expert_of[s];
        if ((o < 0 || o >= a.E) || (!s_want[o] && !s_keep[o])) s_free[fb++] = s;
    }
    __syncthreads();
    // Hot set: candidates in ascending (last use, slot) order; each one's
    // rank is the number of candidates before it.
    const int *cand = s_free;
    if (last_use) {
        for (int i = tid; i < ftot; i += kThreads) {
            const int si = s_free[i], ki = last_use[si];
            int rank = 0;
            for (int j = 0; j < ftot; ++j) {
                const int sj = s_free[j], kj = last_use[sj];
                rank += kj < ki || (kj == ki && sj < si);
            }
            s_order[rank] = si;
        }
        __syncthreads();
        cand = s_order;
    }

    const int n = mtot < ftot ? mtot : ftot;
    if (tid == 0 && mtot > ftot) set_err(a.err, E0_DEV_NO_SLOT);
    for (int i = tid; i < n; i += kThreads) {
        const int s = cand[i], e = s_miss[i];
        const int old = expert_of[s];
        if (old >= 0 && old < a.E && slot_of[old] == s) slot_of[old] = -1;
        expert_of[s] = e;
        slot_of[e] = s;
        if (last_use) last_use[s] = a.step;
        a.copy_slot[(int64_t)l * a.maxc + i] = s;
        a.copy_exp[(int64_t)l * a.maxc + i] = e;
    }
    if (tid == 0) {
        a.ncopy[l] = n;
        if (a.n_copied) a.n_copied[l] = n;
    }
}

struct CopyArgs {
    int maxc;
    const int32_t *ncopy;
    const int32_t *copy_slot;
    const int32_t *copy_exp;
    Stack store, pool;
    int64_t part_units[9];  // 16-byte units per part
    int64_t part_end[9];    // cumulative units
    int contiguous;         // store and pool are bundle-contiguous
};

// Chunk z of copy i of layer l (a no-op when layer l has fewer copies).
E0_DEV void copy_chunk(const CopyArgs &a, int l, int i, int64_t z) {
    if (i >= cload(a.ncopy, l)) return;
    const int slot = cload(a.copy_slot, (int64_t)l * a.maxc + i);
    const int e = cload(a.copy_exp, (int64_t)l * a.maxc + i);
    const int64_t u0 = z * (kCopyChunk / 16);
    u32x4 v[kCopyUnits];
    if (a.contiguous) {
        // Store and pool hold whole bundles: one linear range per expert.
        const u32x4 *src = reinterpret_cast<const u32x4 *>(part_at(a.store.p[0], l, e));
        u32x4 *dst = reinterpret_cast<u32x4 *>(const_cast<char *>(part_at(a.pool.p[0], l, slot)));
        const int64_t n = a.part_end[8];
#pragma unroll
        for (int k = 0; k < kCopyUnits; ++k) {
            const int64_t u = u0 + (int64_t)k * kThreads + threadIdx.x;
            if (u < n) v[k] = __builtin_nontemporal_load(src + u);
        }
#pragma unroll
        for (int k = 0; k < kCopyUnits; ++k) {
            const int64_t u = u0 + (int64_t)k * kThreads + threadIdx.x;
            if (u < n) dst[u] = v[k];
        }
        return;
    }
    int64_t dst_off[kCopyUnits];
    int dst_part[kCopyUnits];
#pragma unroll
    for (int k = 0; k < kCopyUnits; ++k) {
        const int64_t u = u0 + (int64_t)k * kThreads + threadIdx.x;
        dst_part[k] = -1;
        if (u >= a.part_end[8]) continue;
        int j = 0;
        while (u >= a.part_end[j]) ++j;
        const int64_t off = u - (a.part_end[j] - a.part_units[j]);
        const u32x4 *src = reinterpret_cast<const u32x4 *>(part_at(a.store.p[j], l, e)) + off;
        v[k] = __builtin_nontemporal_load(src);
        dst_part[k] = j;
        dst_off[k] = off;
    }
#pragma unroll
    for (int k = 0; k < kCopyUnits; ++k) {
        if (dst_part[k] < 0) continue;
        u32x4 *dst = reinterpret_cast<u32x4 *>(const_cast<char *>(part_at(a.pool.p[dst_part[k]], l, slot))) + dst_off[k];
        *dst = v[k];
    }
}

// Store in device memory: one block per (layer, copy, chunk).
__global__ __launch_bounds__(kThreads) void slot_copy_kernel(CopyArgs a) {
    copy_chunk(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Store in host memory: a few blocks walk every (layer, copy, chunk). Reads
// over the host link take microseconds each; one block per chunk would hold
// every CU while it waits and starve the decode that runs beside the
// update, while a few blocks with 16 KB each in flight already keep the link
// busy.
__global__ __launch_bounds__(kThreads) void slot_copy_strided_kernel(CopyArgs a, int L, int64_t chunks) {
    const int64_t items = (int64_t)L * a.maxc * chunks;
    for (int64_t w = blockIdx.x; w < items; w += gridDim.x) {
        const int64_t z = w % chunks, li = w / chunks;
        copy_chunk(a, (int)(li / a.maxc), (int)(li % a.maxc), z);
    }
}

// True when every part of the stack sits at its bundle offset from part 0
// with part 0's strides (bundle-contiguous storage).
bool stack_contiguous(const e0_stack *s, const int64_t (&part_end)[9]) {
    for (int j = 1; j < 9; ++j) {
        const e0_part &p = s->part[j], &p0 = s->part[0];
        if (static_cast<const char *>(p.ptr) != static_cast<const char *>(p0.ptr) + part_end[j - 1] * 16) return false;
        if (p.slot_stride != p0.slot_stride || p.layer_stride != p0.layer_stride) return false;
    }
    return true;
}

bool stack_ok(const e0_stack *s) {
    for (int i = 0; i < 9; ++i) {
        const e0_part &p = s->part[i];
        if (!p.ptr) return false;
        if ((reinterpret_cast<uintptr_t>(p.ptr) | (uintptr_t)p.slot_stride | (uintptr_t)p.layer_stride) & 15)
            return false;
    }
    return true;
}

struct SlotLayout {
    size_t ncopy, cslot, cexp, total;
    int maxc;
};

SlotLayout slot_layout(int L, int BK, int S, int E) {
    SlotLayout o;
    int maxc = BK < S ? BK : S;
    if (maxc > E) maxc = E;
    o.maxc = maxc;
    size_t off = 0;
    o.ncopy = off;
    off = e0_align(off + sizeof(int32_t) * L);
    o.cslot = off;
    off = e0_align(off + sizeof(int32_t) * (size_t)L * maxc);
    o.cexp = off;
    off = e0_align(off + sizeof(int32_t) * (size_t)L * maxc);
    o.total = off;
    return o;
}

// The store may live in device memory or in pinned host memory mapped for
// the device (then the copy pulls the changed experts over the host link).
// Each part's address is resolved to the one the device uses; a part in
// memory the device cannot reach rejects the call before anything is enqueued.
bool resolve_for_device(const e0_stack &in, e0_stack &out, bool &host) {
    out = in;
    host = false;
    for (int i = 0; i < 9; ++i) {
        hipPointerAttribute_t at{};
        if (hipPointerGetAttributes(&at, in.part[i].ptr) != hipSuccess) {
            (void)hipGetLastError();  // leave no error for the next launch check
            return false;
        }
        if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) continue;
        if (at.type != hipMemoryTypeHost || !at.devicePointer) return false;
        out.part[i].ptr = at.devicePointer;
        host = true;
    }
    return true;
}

}  // namespace

size_t e0_slot_workspace_bytes(const e0_moe_dims *dims, int32_t L, int32_t B, int32_t S) {
    if (!dims || L < 0 || B < 1 || S < 1) return 0;
    return slot_layout(L, B * dims->top_k, S, dims->n_experts).total;
}

namespace {

e0_status slot_update_impl(const e0_moe_dims *dims, int32_t L, int32_t B, int32_t S, const int32_t *next_idx,
                           const int32_t *cur_idx, int32_t *slot_of, int32_t *expert_of, int32_t *last_use,
                           int32_t step, const e0_stack *store, const e0_stack *pool, int32_t *n_copied, void *ws,
                           size_t ws_bytes, int32_t *dev_err, void *stream) {
    E0_REQUIRE(dims && store && pool, E0_ERR_INVALID_ARG);
    const int d = dims->d_model, f = dims->d_ff, E = dims->n_experts, K = dims->top_k;
    E0_REQUIRE(L >= 0 && B >= 1 && S >= 1 && K >= 1 && E >= 1, E0_ERR_INVALID_ARG);
    E0_REQUIRE(d > 0 && f > 0 && d % 64 == 0 && f % 64 == 0, E0_ERR_UNSUPPORTED_SHAPE);
    E0_REQUIRE(E <= kMaxE && S <= kMaxS && (int64_t)B * K <= 4096, E0_ERR_CAPACITY);
    E0_REQUIRE(next_idx && slot_of && expert_of && dev_err, E0_ERR_INVALID_ARG);
    E0_REQUIRE(stack_ok(store) && stack_ok(pool), E0_ERR_INVALID_ARG);
    const SlotLayout lay = slot_layout(L, B * K, S, E);
    E0_REQUIRE(ws && ws_bytes >= lay.total && (reinterpret_cast<uintptr_t>(ws) & 255) == 0, E0_ERR_CAPACITY);
    if (L == 0) return E0_OK;
    e0_stack dstore;
    bool host_store = false;
    E0_REQUIRE(resolve_for_device(*store, dstore, host_store), E0_ERR_INVALID_ARG);

    CopyArgs c{};
    const int64_t qb = (int64_t)d * f / 2, sb = (int64_t)d * f / kGroup * 2;
    int64_t acc = 0;
    for (int j = 0; j < 9; ++j) {
        c.part_units[j] = ((j % 3) == 0 ? qb : sb) / 16;
        acc += c.part_units[j];
        c.part_end[j] = acc;
    }
    const int64_t chunks = (acc * 16 + kCopyChunk - 1) / kCopyChunk;
    E0_REQUIRE(chunks <= 65535, E0_ERR_CAPACITY);

    char *wsb = static_cast<char *>(ws);
    SlotArgs a{L, B * K, E, S, next_idx, cur_idx, slot_of, expert_of, n_copied, dev_err,
               reinterpret_cast<int32_t *>(wsb + lay.ncopy), reinterpret_cast<int32_t *>(wsb + lay.cslot),
               reinterpret_cast<int32_t *>(wsb + lay.cexp), lay.maxc, last_use, step};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(slot_plan_kernel, dim3(L), dim3(kThreads), 0, st, a);
    e0_status s = e0_launch_status();
    if (s) return s;
    if (lay.maxc == 0) return E0_OK;
    c.maxc = lay.maxc;
    c.ncopy = a.ncopy;
    c.copy_slot = a.copy_slot;
    c.copy_exp = a.copy_exp;
    c.store = to_stack(dstore);
    c.pool = to_stack(*pool);
    c.contiguous = stack_contiguous(&dstore, c.part_end) && stack_contiguous(pool, c.part_end);
    if (host_store)
        hipLaunchKernelGGL(slot_copy_strided_kernel, dim3(kHostCopyBlocks), dim3(kThreads), 0, st, c, (int)L, chunks);
    else
        hipLaunchKernelGGL(slot_copy_kernel, dim3(L, lay.maxc, (unsigned)chunks), dim3(kThreads), 0, st, c);
    return e0_launch_status();
}

}  // namespace

extern "C" e0_status e0_slot_update(const e0_moe_dims *dims, int32_t L, int32_t B, int32_t S,
                                    const int32_t *next_idx, const int32_t *cur_idx, int32_t *slot_of,
                                    int32_t *expert_of, const e0_stack *store, const e0_stack *pool,
                                    int32_t *n_copied, void *ws, size_t ws_bytes, int32_t *dev_err, void *stream) {
    e0_clear_stale_error();
    return slot_update_impl(dims, L, B, S, next_idx, cur_idx, slot_of, expert_of, nullptr, 0, store, pool, n_copied,
                            ws, ws_bytes, dev_err, stream);
}

extern "C" e0_status e0_slot_update_lru(const e0_moe_dims *dims, int32_t L, int32_t B, int32_t S,
                                        const int32_t *next_idx, const int32_t *cur_idx, int32_t *slot_of,
                                        int32_t *expert_of, int32_t *last_use, int32_t step, const e0_stack *store,
                                        const e0_stack *pool, int32_t *n_copied, void *ws, size_t ws_bytes,
                                        int32_t *dev_err, void *stream) {
    e0_clear_stale_error();
    E0_REQUIRE(last_use && step >= 0, E0_ERR_INVALID_ARG);
    return slot_update_impl(dims, L, B, S, next_idx, cur_idx, slot_of, expert_of, last_use, step, store, pool,
                            n_copied, ws, ws_bytes, dev_err, stream);
}
