// C-ABI entry points: host-side argument validation and dispatch.  No HIP call
// is made before the arguments are known to define a routing problem.
#include <stdint.h>

#include "route_internal.h"

using moe_route::FusedProblem;
using moe_route::RouteProblem;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape rules shared by every routing entry point.  The top-K has to fit in
// the kept groups; a top-2 group score needs two experts per group.
route_status_t check_shape(int64_t M, int E, int K, int G, int TG, route_group_score_t rule) {
    if (M < 0 || E < 1 || G < 1 || E % G != 0) return ROUTE_EINVAL;
    if (TG < 1 || TG > G) return ROUTE_EINVAL;
    if (K < 1 || (int64_t)K > (int64_t)TG * (E / G)) return ROUTE_EINVAL;
    if (rule != ROUTE_GROUP_MAX && rule != ROUTE_GROUP_TOP2_SUM) return ROUTE_EINVAL;
    if (G > 1 && rule == ROUTE_GROUP_TOP2_SUM && E / G < 2) return ROUTE_EINVAL;
    if (E > moe_route::kMaxExperts || K > moe_route::kMaxTopK || G > moe_route::kMaxGroups)
        return ROUTE_ENOTSUP;
    return ROUTE_OK;
}

bool known_dtype(route_dtype_t d) { return d == ROUTE_F32 || d == ROUTE_BF16; }

route_status_t check_io(const void* logits, route_dtype_t dtype, moe_route::BiasRef bias,
                        int64_t M, float* w, int32_t* ids) {
    if (!known_dtype(dtype)) return ROUTE_EINVAL;
    if (M == 0) return ROUTE_OK;
    if (!logits || !w || !ids) return ROUTE_EINVAL;
    if (!aligned(logits, dtype == ROUTE_F32 ? 4 : 2) || !aligned(w, 4) || !aligned(ids, 4))
        return ROUTE_EINVAL;
    if (bias.p && !aligned(bias.p, bias.bf16 ? 2 : 4)) return ROUTE_EINVAL;
    return ROUTE_OK;
}

// The bias reference of an entry point; false for an unknown bias dtype.
bool make_bias(const void* bias, route_dtype_t bias_dtype, moe_route::BiasRef& out) {
    out = moe_route::BiasRef{bias, bias_dtype == ROUTE_BF16 ? 1 : 0};
    return known_dtype(bias_dtype);
}

// Checks shared by the dispatch entry points; sets d.n = num_tokens * top_k.
route_status_t check_dispatch(moe_route::DispatchProblem& d, const float* topk_weights,
                              int64_t num_tokens, int32_t top_k) {
    if (num_tokens < 0 || top_k < 1 || d.E < 1) return ROUTE_EINVAL;
    if (d.E > moe_route::kMaxExperts) return ROUTE_ENOTSUP;
    if (num_tokens > (int64_t(1) << 31) / top_k ||
        num_tokens * top_k >= (int64_t(1) << 31)) return ROUTE_ENOTSUP;
    d.n = num_tokens * top_k;
    if (!d.counts || !d.offsets) return ROUTE_EINVAL;
    if (!aligned(d.counts, 4) || !aligned(d.offsets, 4)) return ROUTE_EINVAL;
    if (d.sorted_weights && !topk_weights) return ROUTE_EINVAL;
    if (d.n > 0) {
        if (!d.ids || !d.gather || !d.scatter) return ROUTE_EINVAL;
        if (!aligned(d.ids, 4) || !aligned(d.gather, 4) || !aligned(d.scatter, 4))
            return ROUTE_EINVAL;
        if (d.sorted_weights && (!aligned(d.sorted_weights, 4) || !aligned(topk_weights, 4)))
            return ROUTE_EINVAL;
    }
    return ROUTE_OK;
}

route_status_t route_common(RouteProblem p) {
    route_status_t st = check_shape(p.M, p.E, p.K, p.G, p.TG, p.rule);
    if (st != ROUTE_OK) return st;
    if (p.scoring != ROUTE_SOFTMAX && p.scoring != ROUTE_SIGMOID) return ROUTE_EINVAL;
    st = check_io(p.logits, p.dtype, p.bias, p.M, p.weights, p.ids);
    if (st != ROUTE_OK || p.M == 0) return st;
    return moe_route::launch_route(p);
}

}  // namespace

extern "C" {

route_status_t route_topk_softmax(const void* gating_output, route_dtype_t dtype,
                                  int64_t num_tokens, int32_t num_experts, int32_t top_k,
                                  int32_t renormalize, float* topk_weights, int32_t* topk_ids,
                                  void* stream) {
    RouteProblem p{gating_output, dtype, {nullptr, 0}, num_tokens, num_experts, top_k, 1, 1,
                   ROUTE_SOFTMAX, ROUTE_GROUP_MAX, renormalize != 0, topk_weights, topk_ids,
                   static_cast<hipStream_t>(stream)};
    return route_common(p);
}

route_status_t route_grouped_topk(const void* gating_output, route_dtype_t dtype,
                                  int64_t num_tokens, int32_t num_experts, int32_t top_k,
                                  int32_t num_expert_group, int32_t topk_group,
                                  int32_t renormalize, route_scoring_t scoring_func,
                                  float* topk_weights, int32_t* topk_ids, void* stream) {
    RouteProblem p{gating_output, dtype, {nullptr, 0}, num_tokens, num_experts, top_k,
                   num_expert_group, topk_group, scoring_func, ROUTE_GROUP_MAX,
                   renormalize != 0, topk_weights, topk_ids, static_cast<hipStream_t>(stream)};
    return route_common(p);
}

route_status_t route_biased_grouped_topk(const void* gating_output, route_dtype_t dtype,
                                         const void* correction_bias, route_dtype_t bias_dtype,
                                         int64_t num_tokens, int32_t num_experts, int32_t top_k,
                                         int32_t num_expert_group, int32_t topk_group,
                                         int32_t renormalize, float* topk_weights,
                                         int32_t* topk_ids, void* stream) {
    moe_route::BiasRef bias;
    if (!make_bias(correction_bias, bias_dtype, bias)) return ROUTE_EINVAL;
    RouteProblem p{gating_output, dtype, bias, num_tokens, num_experts, top_k,
                   num_expert_group, topk_group, ROUTE_SIGMOID, ROUTE_GROUP_TOP2_SUM,
                   renormalize != 0, topk_weights, topk_ids, static_cast<hipStream_t>(stream)};
    return route_common(p);
}

size_t route_fused_router_workspace_size(int64_t num_tokens, int32_t hidden_dim,
                                         int32_t num_experts) {
    if (num_tokens <= 0 || hidden_dim < 1 || num_experts != 256 || hidden_dim % 64 != 0)
        return 0;
    return moe_route::fused_router_workspace_bytes(num_tokens, hidden_dim);
}

route_status_t route_fused_router(const void* hidden_states, const void* router_weight,
                                  int64_t num_tokens, int32_t hidden_dim, int32_t num_experts,
                                  route_scoring_t scoring_func, const void* correction_bias,
                                  route_dtype_t bias_dtype, route_group_score_t group_score,
                                  int32_t top_k,
                                  int32_t num_expert_group, int32_t topk_group,
                                  int32_t renormalize, float logit_softcap,
                                  float* topk_weights, int32_t* topk_ids, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    route_status_t st = check_shape(num_tokens, num_experts, top_k, num_expert_group, topk_group,
                                    group_score);
    if (!(logit_softcap == logit_softcap) || logit_softcap - logit_softcap != 0.0f)
        return ROUTE_EINVAL;  // NaN or infinite cap
    if (st != ROUTE_OK) return st;
    if (scoring_func != ROUTE_SOFTMAX && scoring_func != ROUTE_SIGMOID) return ROUTE_EINVAL;
    if (hidden_dim < 1) return ROUTE_EINVAL;
    moe_route::BiasRef bias;
    if (!make_bias(correction_bias, bias_dtype, bias)) return ROUTE_EINVAL;
    st = check_io(hidden_states, ROUTE_BF16, bias, num_tokens, topk_weights, topk_ids);
    if (st != ROUTE_OK) return st;
    if (num_tokens > 0 && (!router_weight || !aligned(router_weight, 2))) return ROUTE_EINVAL;
    if (workspace == nullptr ? workspace_bytes != 0 : !aligned(workspace, 16))
        return ROUTE_EINVAL;
    FusedProblem f{hidden_states, router_weight, num_tokens, hidden_dim, logit_softcap, nullptr,
                   RouteProblem{nullptr, ROUTE_BF16, bias, num_tokens, num_experts,
                                top_k, num_expert_group, topk_group, scoring_func, group_score,
                                renormalize != 0, topk_weights, topk_ids,
                                static_cast<hipStream_t>(stream)}};
    if (!moe_route::fused_router_supported(f)) return ROUTE_ENOTSUP;
    if (workspace != nullptr) {
        // the size this shape asks for (0 for 8 or 16 experts: none is used)
        if (workspace_bytes <
            route_fused_router_workspace_size(num_tokens, hidden_dim, num_experts))
            return ROUTE_EINVAL;
        f.workspace = static_cast<float*>(workspace);
    }
    if (num_tokens == 0) return ROUTE_OK;
    return moe_route::launch_fused_router(f);
}

size_t route_dispatch_workspace_size(int64_t num_tokens, int32_t top_k, int32_t num_experts) {
    if (num_tokens < 0 || top_k < 1 || num_experts < 1 || num_experts > moe_route::kMaxExperts)
        return 0;
    const int64_t n = num_tokens * top_k;
    if (n >= (int64_t(1) << 31)) return 0;
    return moe_route::dispatch_workspace_bytes(n, num_experts);
}

route_status_t route_dispatch_metadata(const int32_t* topk_ids, const float* topk_weights,
                                       int64_t num_tokens, int32_t top_k, int32_t num_experts,
                                       int32_t* expert_counts, int32_t* expert_offsets,
                                       int32_t* gather_idx, int32_t* scatter_idx,
                                       float* sorted_weights, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    moe_route::DispatchProblem d{topk_ids, sorted_weights ? topk_weights : nullptr, 0,
                                 num_experts, expert_counts, expert_offsets, gather_idx,
                                 scatter_idx, sorted_weights, workspace,
                                 static_cast<hipStream_t>(stream)};
    route_status_t st = check_dispatch(d, topk_weights, num_tokens, top_k);
    if (st != ROUTE_OK) return st;
    if (!workspace || !aligned(workspace, 4)) return ROUTE_EINVAL;
    if (workspace_bytes < moe_route::dispatch_workspace_bytes(d.n, num_experts))
        return ROUTE_EINVAL;
    return moe_route::launch_dispatch(d);
}

route_status_t route_dispatch_metadata_noalloc(const int32_t* topk_ids,
                                               const float* topk_weights, int64_t num_tokens,
                                               int32_t top_k, int32_t num_experts,
                                               int32_t* expert_counts, int32_t* expert_offsets,
                                               int32_t* gather_idx, int32_t* scatter_idx,
                                               float* sorted_weights, void* stream) {
    moe_route::DispatchProblem d{topk_ids, sorted_weights ? topk_weights : nullptr, 0,
                                 num_experts, expert_counts, expert_offsets, gather_idx,
                                 scatter_idx, sorted_weights, nullptr,
                                 static_cast<hipStream_t>(stream)};
    route_status_t st = check_dispatch(d, topk_weights, num_tokens, top_k);
    if (st != ROUTE_OK) return st;
    if (moe_route::dispatch_workspace_bytes(d.n, num_experts) >
        moe_route::dispatch_noalloc_scratch_bytes())
        return ROUTE_ETOOBIG;
    d.workspace = moe_route::dispatch_noalloc_scratch();  // no allocation: a static buffer
    if (d.workspace == nullptr) return ROUTE_ELAUNCH;
    return moe_route::launch_dispatch(d);
}

route_status_t route_fuse_shared_expert(float* topk_weights, int32_t* topk_ids,
                                        int64_t num_tokens, int32_t top_k,
                                        const int32_t* shared_expert_ids,
                                        float routed_scaling_factor, void* stream) {
    if (num_tokens < 0 || top_k < 2) return ROUTE_EINVAL;
    if (!(routed_scaling_factor == routed_scaling_factor) ||
        routed_scaling_factor - routed_scaling_factor != 0.0f)  // NaN or infinite
        return ROUTE_EINVAL;
    if (top_k > moe_route::kMaxTopK) return ROUTE_ENOTSUP;
    if (num_tokens == 0) return ROUTE_OK;
    if (!topk_weights || !topk_ids || !shared_expert_ids) return ROUTE_EINVAL;
    if (!aligned(topk_weights, 4) || !aligned(topk_ids, 4) || !aligned(shared_expert_ids, 4))
        return ROUTE_EINVAL;
    return moe_route::launch_fuse_shared(topk_weights, topk_ids, num_tokens, top_k,
                                         shared_expert_ids, routed_scaling_factor,
                                         static_cast<hipStream_t>(stream));
}

route_status_t route_sort_ids(float* topk_weights, int32_t* topk_ids, int64_t num_tokens,
                              int32_t top_k, void* stream) {
    if (num_tokens < 0 || top_k < 1) return ROUTE_EINVAL;
    if (top_k > moe_route::kMaxTopK) return ROUTE_ENOTSUP;
    if (num_tokens == 0) return ROUTE_OK;
    if (!topk_weights || !topk_ids) return ROUTE_EINVAL;
    if (!aligned(topk_weights, 4) || !aligned(topk_ids, 4)) return ROUTE_EINVAL;
    return moe_route::launch_sort_ids(topk_weights, topk_ids, num_tokens, top_k,
                                      static_cast<hipStream_t>(stream));
}

const char* route_status_str(route_status_t status) {
    switch (status) {
        case ROUTE_OK: return "ROUTE_OK";
        case ROUTE_EINVAL: return "ROUTE_EINVAL: invalid argument";
        case ROUTE_ENOTSUP: return "ROUTE_ENOTSUP: shape outside the compiled range";
        case ROUTE_ELAUNCH: return "ROUTE_ELAUNCH: kernel launch failed";
        case ROUTE_ETOOBIG:
            return "ROUTE_ETOOBIG: problem larger than the library's static scratch buffer";
    }
    return "unknown route_status_t";
}

}  // extern "C"
