// Internal interface between the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "moe_route.h"

namespace moe_route {

// A per-expert correction bias of E entries, float32 or bfloat16 (the
// aiter-style call passes it in the logits' dtype).  p == nullptr: no bias.
struct BiasRef {
    const void* p;
    int bf16;  // 0: float32 entries, 1: bfloat16 entries
};

// One routing problem after host-side validation.
struct RouteProblem {
    const void* logits;     // [M, E] f32 or bf16
    route_dtype_t dtype;
    BiasRef bias;           // [E]; bias.p == nullptr: none
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
    float softcap;          // 0: none; else logits -> softcap * tanh(logits / softcap)
    float* workspace;       // fused_router_workspace_bytes(M, H), or nullptr: one kernel
    RouteProblem route;     // logits/dtype unused
};

// Dispatch metadata of a routing result (route_dispatch.hip).
struct DispatchProblem {
    const int32_t* ids;     // [n] expert ids (n = M * K)
    const float* weights;   // [n] or nullptr when sorted_weights is nullptr
    int64_t n;
    int E;
    int32_t* counts;        // [E]
    int32_t* offsets;       // [E + 1]
    int32_t* gather;        // [n]
    int32_t* scatter;       // [n]
    float* sorted_weights;  // [n] or nullptr
    void* workspace;        // dispatch_workspace_bytes(n, E)
    hipStream_t stream;
};

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 64;
constexpr int kMaxGroups = 64;

int device_cu_count();  // compute units of the current device (cached)

// Blocks of `kernel` that fit on one compute unit at `threads` per block (1
// if the query fails).  Callers keep it in a function-local static, whose
// initialisation C++ makes thread-safe.
template <typename F>
int resident_blocks(F kernel, int threads) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess ||
        n <= 0)
        n = 1;
    return n;
}

// Kernel launchers (route_kernels.hip / fused_router.hip).  They assume a
// validated problem with M > 0 and return ROUTE_OK or ROUTE_ELAUNCH.
route_status_t launch_route(const RouteProblem& p);
// One wavefront per row (route_row.hip): 256 experts, sigmoid scoring, K <= 8,
// no groups or 8 groups, up to kRowMaxTokens rows; launch_route sends such
// problems there when their pointers allow 8-byte (bf16) or 16-byte loads.
#ifndef MOE_ROUTE_ROW_MAX_TOKENS
#define MOE_ROUTE_ROW_MAX_TOKENS 2048
#endif
constexpr int64_t kRowMaxTokens = MOE_ROUTE_ROW_MAX_TOKENS;
bool route_row_supported(const RouteProblem& p);
route_status_t launch_route_row(const RouteProblem& p);
route_status_t launch_fused_router(const FusedProblem& p);
bool fused_router_supported(const FusedProblem& p);
bool small_router_supported(const FusedProblem& p);  // E = 8 or 16 (fused_router_small.hip)
route_status_t launch_small_router(const FusedProblem& p);
struct SplitPlan {
    int rows;    // tokens per tile of the partial kernel (32, 64 or 128)
    int splits;  // hidden-dimension splits; 1: the single fused kernel
};
SplitPlan fused_router_split_plan(int64_t M, int H);
size_t fused_router_workspace_bytes(int64_t M, int H);
size_t dispatch_workspace_bytes(int64_t n, int E);
// The static scratch of route_dispatch_metadata_noalloc: its size, and its
// device address on the current device (nullptr if the lookup fails).
size_t dispatch_noalloc_scratch_bytes();
void* dispatch_noalloc_scratch();
route_status_t launch_dispatch(const DispatchProblem& d);
route_status_t launch_fuse_shared(float* w, int32_t* ids, int64_t M, int K,
                                  const int32_t* shared_ids, float rsf, hipStream_t stream);
route_status_t launch_sort_ids(float* w, int32_t* ids, int64_t M, int K, hipStream_t stream);

}  // namespace moe_route
