// Sorted whole-layer prefill (grouped GEMM on matrix cores) — being written.
#include "e0_internal.h"

size_t e0_prefill_workspace_bytes(const e0_moe_dims *dims, int32_t T) {
    if (!dims || T < 0) return 0;
    return 256;
}

extern "C" e0_status e0_moe_sorted_prefill(const e0_moe_dims *dims, int32_t T, const uint16_t *x, const int32_t *idx,
                                           const float *w, const e0_stack *layer, float *y, void *ws, size_t ws_bytes,
                                           int32_t *dev_err, void *stream) {
    (void)dims; (void)T; (void)x; (void)idx; (void)w; (void)layer; (void)y; (void)ws; (void)ws_bytes;
    (void)dev_err; (void)stream;
    return E0_ERR_UNSUPPORTED_SHAPE;
}
