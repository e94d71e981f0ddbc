/*
 * moe_route.h -- C ABI of the MI355X (gfx950) MoE routing library
 * (libmoe_route.so).
 *
 * Per token row of router logits, the library scores every expert, optionally
 * keeps only the best expert groups, picks the top-K experts among the
 * survivors, and writes fp32 weights and int32 expert ids.  The operations are
 * defined on these pages:
 *
 *   [ROUTING] "[SGLang] MoE routing: token-to-expert assignment algorithms"
 *             (blog.secrett2633.cloud/opensource/sglang/moe-routing)
 *   [AITER]   "[sglang] SGLang MoE routing optimisation: using
 *             aiter.biased_grouped_topk on AMD GPUs" (sglang PR 23611 analysis)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every pointer is a DEVICE pointer owned by the caller.  Tensors are
 *           dense, row-major, with no padding between rows.  Outputs are
 *           preallocated by the caller and filled in place, as the pages' call
 *           sites do ([ROUTING] section 2; [AITER] section "Code analysis").
 * Outputs.  topk_weights: float32 [num_tokens, top_k].
 *           topk_ids:     int32   [num_tokens, top_k], row r lists its K chosen
 *           experts by selection score descending; equal scores go to the lower
 *           expert index first.  weights[r][k] belongs to ids[r][k].
 * Streams.  `stream` is a hipStream_t (NULL = the legacy default stream).  Work
 *           is only enqueued; nothing is synchronised, allocated or freed.
 * Threads.  Entry points are reentrant.  The only state the library keeps is
 *           a cache, filled on first use and safe under concurrent calls, of
 *           each device's compute-unit count and of each kernel's resident
 *           blocks per compute unit.
 * Errors.   Arguments are checked on the host before any HIP call:
 *             ROUTE_EINVAL   the arguments do not define a routing problem
 *                            (null pointer with num_tokens > 0, num_tokens < 0,
 *                            top_k outside [1, topk_group * E / G],
 *                            E % num_expert_group != 0, topk_group outside
 *                            [1, num_expert_group], a top-2 group score with
 *                            groups of one expert, a misaligned pointer, an
 *                            unknown enum value);
 *             ROUTE_ENOTSUP  a valid problem outside the compiled range
 *                            (num_experts > 1024, top_k > 64,
 *                            num_expert_group > 64; fused router limits below);
 *             ROUTE_ELAUNCH  the kernel launch failed (hipGetLastError).
 *           num_tokens == 0 returns ROUTE_OK without touching the GPU.  After an
 *           error the output contents are unspecified.
 * Inputs.   Logits (and bias) are expected finite; results for NaN or infinite
 *           inputs are unspecified.
 * Precision. Scores are computed in fp32 with the GPU's exp2 and reciprocal
 *           instructions.  Expert choices therefore agree with an exact
 *           computation except where two selection scores lie within a few
 *           fp32 rounding units (a few 1e-7) of each other.  With sigmoid
 *           scoring, 256 or 160 experts and top_k <= 8 (the specialised
 *           kernels and the fused router), picks that close are re-ranked
 *           in double precision, so the order of the chosen experts is
 *           exact; only the K-th choice itself, or the last kept group,
 *           can then differ from an exact computation on such a near tie.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ROUTE_OK = 0,
    ROUTE_EINVAL = 1,
    ROUTE_ENOTSUP = 2,
    ROUTE_ELAUNCH = 3,
    ROUTE_ETOOBIG = 4  /* larger than a static scratch buffer (noalloc entry points) */
} route_status_t;

/* Element type of the router logits / hidden states. */
typedef enum {
    ROUTE_F32 = 0,  /* IEEE binary32 */
    ROUTE_BF16 = 1  /* bfloat16: the upper 16 bits of a binary32 */
} route_dtype_t;

/* Scoring function.
 *   ROUTE_SOFTMAX: exp(x_i - max_j x_j) / sum_j exp(x_j - max_j x_j) over all E
 *                  experts of the row ([ROUTING] section 2).
 *   ROUTE_SIGMOID: 1 / (1 + exp(-x_i)) ([ROUTING] section 4; [AITER]). */
typedef enum {
    ROUTE_SOFTMAX = 0,
    ROUTE_SIGMOID = 1
} route_scoring_t;

/* Group score used to rank expert groups (groups are contiguous blocks of
 * E / num_expert_group experts).
 *   ROUTE_GROUP_MAX:      the group's largest selection score
 *                         ([ROUTING] section 3, DeepSeek-V2 style).
 *   ROUTE_GROUP_TOP2_SUM: the sum of the group's two largest selection scores
 *                         ([ROUTING] section 4, DeepSeek-V3 style). */
typedef enum {
    ROUTE_GROUP_MAX = 0,
    ROUTE_GROUP_TOP2_SUM = 1
} route_group_score_t;

/*
 * Softmax top-k ([ROUTING] section 2): softmax over all E experts, the top_k
 * largest probabilities and their ids; with renormalize != 0 the K weights are
 * divided by their sum so they add up to 1.
 *   gating_output  [num_tokens, num_experts] logits of type `dtype`.
 */
route_status_t route_topk_softmax(const void* gating_output, route_dtype_t dtype,
                                  int64_t num_tokens, int32_t num_experts, int32_t top_k,
                                  int32_t renormalize, float* topk_weights, int32_t* topk_ids,
                                  void* stream);

/*
 * Grouped top-k ([ROUTING] section 3): score with `scoring_func`, rank the
 * num_expert_group groups by their largest score (ROUTE_GROUP_MAX), keep the
 * best topk_group groups (ties: lower group index), then take the top_k
 * experts of the kept groups.  Weights are the scores of the chosen experts
 * (for softmax: the probability over all E experts), optionally renormalised.
 * num_expert_group == 1 is plain top-k.
 */
route_status_t route_grouped_topk(const void* gating_output, route_dtype_t dtype,
                                  int64_t num_tokens, int32_t num_experts, int32_t top_k,
                                  int32_t num_expert_group, int32_t topk_group,
                                  int32_t renormalize, route_scoring_t scoring_func,
                                  float* topk_weights, int32_t* topk_ids, void* stream);

/*
 * Biased grouped top-k ([ROUTING] section 4; [AITER] "Code analysis"):
 * s_i = sigmoid(x_i); selection score c_i = s_i + correction_bias[i]; group
 * score = sum of the group's two largest c (ROUTE_GROUP_TOP2_SUM); keep the
 * best topk_group groups; take the top_k experts of the kept groups by c.  The
 * emitted weight is the UNBIASED s of each chosen expert, optionally divided
 * by the sum of the K weights.  num_expert_group == topk_group == 1 is the
 * sigmoid-with-bias top-k the [AITER] page swaps in.
 *   correction_bias  [num_experts] of type bias_dtype, or NULL for all zeros.
 *   bias_dtype       ROUTE_F32, or ROUTE_BF16: the [AITER] call ("Code
 *                    analysis") casts the bias to the logits' dtype before
 *                    passing it; bf16 entries are widened exactly to fp32.
 *                    An unknown value is ROUTE_EINVAL (also with a NULL bias).
 *   With num_expert_group > 1 every group needs at least two experts.
 */
route_status_t route_biased_grouped_topk(const void* gating_output, route_dtype_t dtype,
                                         const void* correction_bias, route_dtype_t bias_dtype,
                                         int64_t num_tokens, int32_t num_experts, int32_t top_k,
                                         int32_t num_expert_group, int32_t topk_group,
                                         int32_t renormalize, float* topk_weights,
                                         int32_t* topk_ids, void* stream);

/*
 * Fused router ([ROUTING] section 5): the router projection
 *   logits[m][e] = sum_h hidden_states[m][h] * router_weight[h][e]
 * with bf16 operands and fp32 accumulation, followed by the routing above
 * (scoring_func, optional correction_bias, group_score rule,
 * num_expert_group / topk_group, top_k, renormalize).
 *   hidden_states  [num_tokens, hidden_dim] bf16
 *   router_weight  [hidden_dim, num_experts] bf16 (expert index contiguous)
 *   correction_bias [num_experts] of type bias_dtype (float32, or bf16 as in
 *                  route_biased_grouped_topk) or NULL (zeros)
 *   logit_softcap  0, or a cap c: every logit l is replaced by c * tanh(l / c)
 *                  before scoring ([ROUTING] section 5, soft-capping); tanh
 *                  is increasing, so the cap changes weights, not choices.
 *                  NaN or infinite caps are ROUTE_EINVAL.
 *   workspace      NULL (workspace_bytes 0), or device scratch of at least
 *                  route_fused_router_workspace_size(num_tokens, hidden_dim,
 *                  num_experts) bytes, 16-byte aligned, owned by the caller.
 *                  With NULL, or when that size is 0, one kernel computes
 *                  the projection and the routing and the logits never reach
 *                  memory.  Otherwise (up to 8192 tokens, 256 experts) the
 *                  hidden dimension is split over more workgroups: their
 *                  fp32 partial logits go to the workspace, which calls
 *                  sharing it must not use at the same time.  The two
 *                  paths add the products in different orders, so their
 *                  logits may differ in the last bits.
 * Compiled range, with hidden_states and router_weight 16-byte aligned:
 *   num_experts == 256: hidden_dim a positive multiple of 64 (MFMA router);
 *   num_experts 8 or 16 ([ROUTING] section 5's small-router case):
 *     hidden_dim a positive multiple of 8, num_expert_group == 1; no
 *     workspace is used (its size is 0; a workspace passed anyway is
 *     ignored).
 * Other valid shapes return ROUTE_ENOTSUP.  A misaligned workspace,
 * workspace_bytes without a workspace, or a workspace smaller than required
 * is ROUTE_EINVAL.
 */
size_t route_fused_router_workspace_size(int64_t num_tokens, int32_t hidden_dim,
                                         int32_t num_experts);
route_status_t route_fused_router(const void* hidden_states, const void* router_weight,
                                  int64_t num_tokens, int32_t hidden_dim, int32_t num_experts,
                                  route_scoring_t scoring_func, const void* correction_bias,
                                  route_dtype_t bias_dtype, route_group_score_t group_score,
                                  int32_t top_k,
                                  int32_t num_expert_group, int32_t topk_group,
                                  int32_t renormalize, float logit_softcap, float* topk_weights,
                                  int32_t* topk_ids, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Dispatch metadata of a routing result ([ROUTING] section "output format":
 * the kernel-oriented output of routing data, gather index and scatter index;
 * the page names them without defining their fields, and the definition
 * below is this library's).  The num_tokens * top_k assignments, numbered
 * a = token * top_k + slot, are put in order of expert id, keeping the order
 * of a among assignments of the same expert (a stable counting sort):
 *   topk_ids       [num_tokens, top_k] int32, e.g. a routing call's output;
 *                  ids outside [0, num_experts) are dropped
 *   topk_weights   [num_tokens, top_k] float32, or NULL when sorted_weights
 *                  is NULL
 *   expert_counts  [num_experts] int32: assignments per expert
 *   expert_offsets [num_experts + 1] int32: start of each expert's run in the
 *                  sorted order (offsets[num_experts] = valid assignments)
 *   gather_idx     [num_tokens * top_k] int32: the assignment at each sorted
 *                  position; -1 past offsets[num_experts]
 *   scatter_idx    [num_tokens * top_k] int32: the sorted position of each
 *                  assignment, -1 for a dropped one
 *   sorted_weights [num_tokens * top_k] float32 or NULL: topk_weights in
 *                  sorted order; 0 past offsets[num_experts]
 *   workspace      device scratch of at least
 *                  route_dispatch_workspace_size(num_tokens, top_k,
 *                  num_experts) bytes, 4-byte aligned, owned by the caller;
 *                  its contents are overwritten (calls that share it must not
 *                  overlap)
 * All arrays are device memory; every int32/float array 4-byte aligned.
 * Errors: ROUTE_EINVAL for num_tokens < 0, top_k < 1, num_experts < 1, a null
 * or misaligned required pointer, sorted_weights without topk_weights, or a
 * workspace smaller than required; ROUTE_ENOTSUP for num_experts > 1024 or
 * num_tokens * top_k >= 2^31.  num_tokens == 0 is valid and still writes
 * zero counts and offsets.
 */
size_t route_dispatch_workspace_size(int64_t num_tokens, int32_t top_k, int32_t num_experts);
route_status_t route_dispatch_metadata(const int32_t* topk_ids, const float* topk_weights,
                                       int64_t num_tokens, int32_t top_k, int32_t num_experts,
                                       int32_t* expert_counts, int32_t* expert_offsets,
                                       int32_t* gather_idx, int32_t* scatter_idx,
                                       float* sorted_weights, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * route_dispatch_metadata without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same outputs, bit for bit, with the
 * scratch taken from a static device buffer of the library instead of a
 * caller workspace.  The entry point allocates nothing and frees nothing.
 *   Limit: route_dispatch_workspace_size(num_tokens, top_k, num_experts)
 *          must not exceed 4 MiB (e.g. up to 8,386,560 assignments at 256
 *          experts, 2,095,104 at 1024); larger problems return
 *          ROUTE_ETOOBIG before any GPU work.
 *   The buffer is one per device, held until the process ends, and shared
 *   by every call on that device: calls on one device whose executions
 *   overlap (different streams without ordering between them) race on it.
 *   Calls on one stream are ordered and safe.  Nothing in the buffer needs
 *   to start at zero: every call overwrites what it reads.
 * Other arguments and errors as route_dispatch_metadata; ROUTE_ELAUNCH also
 * when the buffer's device address cannot be looked up.
 */
route_status_t route_dispatch_metadata_noalloc(const int32_t* topk_ids,
                                               const float* topk_weights, int64_t num_tokens,
                                               int32_t top_k, int32_t num_experts,
                                               int32_t* expert_counts, int32_t* expert_offsets,
                                               int32_t* gather_idx, int32_t* scatter_idx,
                                               float* sorted_weights, void* stream);

/*
 * Shared-expert slot ([ROUTING] section 6), in place on a routing result:
 * row m's last slot gets topk_ids[m][top_k-1] = shared_expert_ids[m] (the
 * page draws this id at random from [E, E + num_shared); the caller supplies
 * the draw).  When routed_scaling_factor != 0 the slot's weight becomes the
 * sum of the row's other top_k - 1 weights divided by it (fp32 sum in slot
 * order, IEEE division); with 0 the weight is left as it is.  Other slots are
 * untouched.
 *   topk_weights [num_tokens, top_k] float32, topk_ids [num_tokens, top_k]
 *   int32, shared_expert_ids [num_tokens] int32; device memory, 4-byte
 *   aligned.
 * Errors: ROUTE_EINVAL for num_tokens < 0, top_k < 2, a NaN or infinite
 * factor, or a null or misaligned pointer (num_tokens > 0); ROUTE_ENOTSUP for
 * top_k > 64.  num_tokens == 0 returns ROUTE_OK without touching the GPU.
 */
route_status_t route_fuse_shared_expert(float* topk_weights, int32_t* topk_ids,
                                        int64_t num_tokens, int32_t top_k,
                                        const int32_t* shared_expert_ids,
                                        float routed_scaling_factor, void* stream);

/*
 * Ascending id order, in place on a routing result: each row's top_k
 * (id, weight) pairs reordered by expert id, lowest first; equal ids keep
 * their slot order.  (Routing emits ids by selection score; some consumers
 * want them by expert, as the decode top-k of "[sglang] MiniMax-M3 ... FP8
 * Attention GEMM", section 1, orders its ids.)
 * Errors: ROUTE_EINVAL for num_tokens < 0, top_k < 1, or a null or
 * misaligned pointer (num_tokens > 0); ROUTE_ENOTSUP for top_k > 64.
 */
route_status_t route_sort_ids(float* topk_weights, int32_t* topk_ids, int64_t num_tokens,
                              int32_t top_k, void* stream);

/* Static, human-readable name of a status code. */
const char* route_status_str(route_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
