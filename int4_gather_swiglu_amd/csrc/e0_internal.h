// Internal helpers shared by the gfx950 kernels of libe0 (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/e0.h"

#define E0_DEV __device__ __forceinline__

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Index of this wavefront in its workgroup, as a wave-uniform (scalar) value:
// derived values stay in SGPRs and buffer descriptors built from them need no
// per-lane waterfall loops.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
constexpr int kGroup = 64;  // quantisation group along the input dimension

// A part of a stacked tensor, as kernels see it.
struct Part {
    const char *ptr;
    int64_t slot_stride;
    int64_t layer_stride;
};

struct Stack {
    Part p[9];  // [3 * matrix + kind]; matrix 0 gate, 1 up, 2 down; kind 0 q, 1 s, 2 b
};

inline Stack to_stack(const e0_stack &s) {
    Stack o;
    for (int i = 0; i < 9; ++i) {
        o.p[i].ptr = static_cast<const char *>(s.part[i].ptr);
        o.p[i].slot_stride = s.part[i].slot_stride;
        o.p[i].layer_stride = s.part[i].layer_stride;
    }
    return o;
}

E0_DEV const char *part_at(const Part &p, int layer, int slot) {
    return p.ptr + (int64_t)layer * p.layer_stride + (int64_t)slot * p.slot_stride;
}

E0_DEV float h2f(uint16_t b) { return (float)__builtin_bit_cast(f16, b); }

// Element index of the scale (or bias) of row r, group g in the bundle's
// 8-row tiles [rows/8][ngrp][8].
E0_DEV uint32_t sb_index(uint32_t r, uint32_t g, uint32_t ngrp) { return ((r >> 3) * ngrp + g) * 8 + (r & 7); }

// Reinterpret a dword as two fp16. Takes the dword by value: applying
// __builtin_bit_cast directly to an element of an ext_vector (v[j]) reads the
// vector's first element whatever j is, so every such cast goes through here.
E0_DEV f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// Raw buffer resources: an SGPR descriptor over `bytes` bytes at `p`, loaded
// with 32-bit per-lane byte offsets (no 64-bit address registers per load).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;
E0_DEV rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcFlags);
}
E0_DEV u32x4 ld128(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0); }
// The same with the nontemporal hint (cache policy bit 1), for code words a
// call reads exactly once (the decode's expert weights): with the slot copy
// running beside the decode, the step takes about 5% less time than with
// the default policy.
constexpr int kPolicyNt = 2;
E0_DEV u32x4 ld128_once(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicyNt);
}
E0_DEV uint16_t ld16(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0); }

// A read through the constant address space: with a wave-uniform index it
// becomes a scalar load (several issued together, one wait), for small tables
// that no kernel writes while the reading kernel runs (routing ids and
// weights, slot tables).
template <class T>
E0_DEV T cload(const T *p, int64_t i) {
    typedef const __attribute__((address_space(4))) T ct;
    return ((ct *)p)[i];
}

E0_DEV float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
E0_DEV float group_sum(float v, int width) {
    for (int m = width >> 1; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// Reduce-scatter of N values held by each of 64 lanes (N a power of two,
// 32 <= N). After the call, lane l holds in v[0 .. N/64) the totals of value
// indices l*(N/64) + j for N >= 64; for N == 32 lane l holds in v[0] the total
// of index l >> 1.
template <int N>
E0_DEV void wave_reduce_scatter(float (&v)[N]) {
    const int lane = threadIdx.x & 63;
    int n = N;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        if (n == 1) {
            v[0] += __shfl_xor(v[0], m);
            continue;
        }
        const bool hi = (lane & m) != 0;
        const int h = n >> 1;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            if (i < h) {
                float keep = hi ? v[i + h] : v[i];
                float send = hi ? v[i] : v[i + h];
                v[i] = keep + __shfl_xor(send, m);
            }
        }
        n = h;
    }
}

// Orders LDS accesses of one wavefront (lanes exchange values through LDS).
E0_DEV void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

E0_DEV void set_err(int32_t *err, int bits) {
    if (err) atomicOr(err, bits);
}

// ---------------------------------------------------------------------------
// Hand-off between workgroups of one launch. A producer workgroup publishes
// values with device-coherent stores, waits until they have completed, and
// then stores the call's epoch into its flag; a consumer workgroup (always at
// a higher blockIdx than its producers, and workgroups are dispatched in
// blockIdx order, so every producer it waits for has started) polls the flags
// with device-coherent loads and then reads the values with device-coherent
// loads. Device-coherent accesses go to the coherence point shared by all
// XCDs, so no cache write-back or invalidate is needed. Flags hold a 64-bit
// epoch unique to each call, so they never need clearing. The wait is bounded
// (kSpinTicks of the 100 MHz wall clock); on expiry it reports failure.
// ---------------------------------------------------------------------------
constexpr uint64_t kSpinTicks = 5000000;  // 50 ms

E0_DEV void coherent_store(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
E0_DEV float coherent_load(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
E0_DEV uint64_t coherent_load(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread of the workgroup calls this after its last coherent store.
E0_DEV void signal_ready(uint64_t *flag, uint64_t epoch) {
    __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread of the workgroup calls this; true when flags[0, n) all hold
// `epoch`, false if the bounded wait expired. Ends with a workgroup barrier.
E0_DEV bool wait_ready(const uint64_t *flags, int n, uint64_t epoch) {
    int ok = 1;
    const uint64_t t0 = wall_clock64();
    for (int i = threadIdx.x; i < n && ok; i += blockDim.x) {
        while (coherent_load(flags + i) != epoch) {
            if (wall_clock64() - t0 > kSpinTicks) {
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    return __syncthreads_and(ok) != 0;
}

// A per-call epoch for the flags above (never 0, distinct for 2^64 calls).
uint64_t e0_next_epoch();

// Status plumbing for host entry points.
#define E0_REQUIRE(cond, code) \
    do {                       \
        if (!(cond)) return (code); \
    } while (0)

// Every entry point starts with this: a status left pending in the calling
// thread by an earlier runtime call (the caller's, not this library's) is
// cleared, so that e0_launch_status reports this call's launches only.
inline void e0_clear_stale_error() { (void)hipGetLastError(); }

inline e0_status e0_launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? E0_OK : E0_ERR_HIP;
}

inline size_t e0_align(size_t x) { return (x + 255) & ~(size_t)255; }
