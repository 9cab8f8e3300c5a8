// Host-only parts of the C ABI: status strings and workspace sizes.
#include "moe_internal.h"

size_t moe_permute_workspace_bytes(int64_t T, int32_t E);
size_t moe_route_workspace_bytes(int64_t T, int64_t d, int32_t E);
size_t moe_gemm_workspace_bytes(int32_t G);
size_t moe_quant_workspace_bytes(int32_t G);
size_t moe_route_backward_workspace_bytes(int64_t T, int64_t d, int32_t E, int32_t k);
size_t moe_combine_bwd_quant_workspace_bytes(int64_t T, int32_t k, int32_t G);

extern "C" const char* moe_status_str(int32_t status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
        case MOE_ENOTSUP: return "MOE_ENOTSUP: unsupported dtype or option";
        case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace missing or too small";
        case MOE_EHIP: return "MOE_EHIP: HIP launch failed";
        default: return "MOE_UNKNOWN_STATUS";
    }
}

extern "C" size_t moe_workspace_bytes(int32_t op, int64_t T, int64_t d, int32_t E, int32_t k, int32_t G) {
    (void)d;
    switch (op) {
        case MOE_OP_ROUTE: return moe_route_workspace_bytes(T, d, E);
        case MOE_OP_PERMUTE: return moe_permute_workspace_bytes(T, E);
        case MOE_OP_GROUPED_GEMM: return moe_gemm_workspace_bytes(G);
        case MOE_OP_QUANT: return moe_quant_workspace_bytes(G);
        case MOE_OP_ROUTE_BWD: return moe_route_backward_workspace_bytes(T, d, E, k);
        case MOE_OP_COMBINE_BWD_QUANT: return moe_combine_bwd_quant_workspace_bytes(T, k, G);
        default: return 0;
    }
}
