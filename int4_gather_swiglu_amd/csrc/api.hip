// libe0 entry points that launch nothing: ABI version, status strings and
// workspace sizes of the five calls.
#include "e0_internal.h"

#include <atomic>

size_t e0_decode_workspace_bytes(const e0_moe_dims *dims, int32_t L, int32_t B, int32_t r);
size_t e0_slot_workspace_bytes(const e0_moe_dims *dims, int32_t L, int32_t B, int32_t S);
size_t e0_prerouter_workspace_bytes(int32_t H, int32_t B, int32_t E, int32_t hid);
size_t e0_prefill_workspace_bytes(const e0_moe_dims *dims, int32_t T);
size_t e0_chain_workspace_bytes(const e0_moe_dims *dims, int32_t L);

extern "C" int32_t e0_abi_version(void) { return E0_ABI_VERSION; }

// Epochs of the in-launch hand-off flags: a process-wide call counter passed
// through a 64-bit bijective mixer (Stafford's "Mix13" finaliser), so that a
// flag word left over from other data is unlikely to equal the epoch.
uint64_t e0_next_epoch() {
    static std::atomic<uint64_t> calls{0};
    uint64_t z = calls.fetch_add(1, std::memory_order_relaxed) + 1;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z ? z : 1;
}

extern "C" const char *e0_status_string(e0_status s) {
    switch (s) {
        case E0_OK: return "ok";
        case E0_ERR_INVALID_ARG: return "invalid argument";
        case E0_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case E0_ERR_CAPACITY: return "capacity exceeded (workspace, slots or a size limit)";
        case E0_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

// n = layers / tokens / heads, b = tokens per layer, s = slots (see e0.h).
// For E0_OP_STAGED_DECODE, `s` carries the shared expert's LoRA rank (0 = none).
extern "C" size_t e0_workspace_bytes(int32_t op, const e0_moe_dims *dims, int32_t n, int32_t b, int32_t s) {
    if (!dims) return 0;
    switch (op) {
        case E0_OP_ROUTE: return 0;
        case E0_OP_PREROUTER: return e0_prerouter_workspace_bytes(n, b, dims->n_experts, dims->d_ff);
        case E0_OP_STAGED_DECODE: return e0_decode_workspace_bytes(dims, n, b, s);
        case E0_OP_SORTED_PREFILL: return e0_prefill_workspace_bytes(dims, n);
        case E0_OP_SLOT_UPDATE: return e0_slot_workspace_bytes(dims, n, b, s);
        case E0_OP_CHAINED_DECODE: return e0_chain_workspace_bytes(dims, n);
        default: return 0;
    }
}
