// Internal interface between the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "moe_route.h"

namespace moe_route {

// One routing problem after host-side validation.
struct RouteProblem {
    const void* logits;     // [M, E] f32 or bf16
    route_dtype_t dtype;
    const float* bias;      // [E] or nullptr
    int64_t M;
    int E, K, G, TG;
    route_scoring_t scoring;
    route_group_score_t rule;
    bool renorm;
    float* weights;         // [M, K]
    int32_t* ids;           // [M, K]
    hipStream_t stream;
};

struct FusedProblem {
    const void* hidden;     // [M, H] bf16
    const void* w;          // [H, E] bf16
    int64_t M;
    int H;
    RouteProblem route;     // logits/dtype unused
};

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 64;
constexpr int kMaxGroups = 64;

// Kernel launchers (route_kernels.hip / fused_router.hip).  They assume a
// validated problem with M > 0 and return ROUTE_OK or ROUTE_ELAUNCH.
route_status_t launch_route(const RouteProblem& p);
route_status_t launch_fused_router(const FusedProblem& p);
bool fused_router_supported(const FusedProblem& p);

}  // namespace moe_route
