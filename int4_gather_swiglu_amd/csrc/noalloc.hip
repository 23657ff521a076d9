// e0_moe_staged_decode_noalloc: the staged decode for callers that cannot
// allocate (code under graph capture, tight serving loops, harnesses that
// forbid hipMalloc). Same kernels as e0_moe_staged_decode; the workspace is a
// fixed device array of this library instead of a caller buffer.
//
// The array is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy until the process ends. Host code never uses its name as
// an address: on the first call on a device (that device current) its device
// address is looked up once with hipGetSymbolAddress and kept per device.
// Calls on one GPU share the array and it keeps the last call's contents; the
// decode kernels need none of it zeroed (every value they read is written by
// the same call first, and the batch-1 hand-off flags hold per-call epochs),
// so nothing is cleared. Two calls in flight at once on one GPU race on it.
#include "e0_internal.h"

#include <mutex>

size_t e0_decode_workspace_bytes(const e0_moe_dims *dims, int32_t L, int32_t B, int32_t r);

static constexpr size_t kScratchBytes = size_t(32) << 20;  // E0_NOALLOC_SCRATCH_BYTES in e0.h
static_assert(kScratchBytes == E0_NOALLOC_SCRATCH_BYTES, "e0.h states the scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Device address of the array on the current device (looked up on the first
// call on that device).
e0_status scratch_of_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return E0_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return E0_ERR_CAPACITY;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return E0_ERR_HIP;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return E0_OK;
}

}  // namespace

extern "C" e0_status e0_moe_staged_decode_noalloc(const e0_moe_dims *dims, int32_t L, int32_t B,
                                                  const uint16_t *x, const int32_t *idx, const float *w,
                                                  const int32_t *slot_of, int32_t S, const e0_stack *pool,
                                                  const e0_shared *shared, float *y, int32_t *dev_err,
                                                  void *stream) {
    e0_clear_stale_error();
    E0_REQUIRE(dims && pool, E0_ERR_INVALID_ARG);
    E0_REQUIRE(L >= 0 && B >= 1, E0_ERR_INVALID_ARG);
    const int32_t r = shared ? shared->lora_rank : 0;
    E0_REQUIRE(r >= 0, E0_ERR_UNSUPPORTED_SHAPE);
    // Sizes whose workspace exceeds the array are refused before anything else.
    E0_REQUIRE(e0_decode_workspace_bytes(dims, L, B, r) <= kScratchBytes, E0_ERR_CAPACITY);
    void *ws = nullptr;
    const e0_status s = scratch_of_current_device(&ws);
    if (s) return s;
    return e0_moe_staged_decode(dims, L, B, x, idx, w, slot_of, S, pool, shared, y, ws, kScratchBytes, dev_err,
                                stream);
}
