"""MI355X-native MoE routing top-k: thin Python binding over libmoe_route.so.

Every function here only marshals arguments (torch tensors -> device
pointers, the current HIP stream) and calls the C-ABI entry point of the same
name declared in ``include/moe_route.h``.  All routing arithmetic runs in the
library's HIP kernels; there is no CPU or PyTorch fallback.  If the library
is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_route.so")

ROUTE_OK, ROUTE_EINVAL, ROUTE_ENOTSUP, ROUTE_ELAUNCH, ROUTE_ETOOBIG = 0, 1, 2, 3, 4
ROUTE_F32, ROUTE_BF16 = 0, 1
ROUTE_SOFTMAX, ROUTE_SIGMOID = 0, 1
ROUTE_GROUP_MAX, ROUTE_GROUP_TOP2_SUM = 0, 1

EXPORTED = (
    "route_topk_softmax",
    "route_grouped_topk",
    "route_biased_grouped_topk",
    "route_fused_router",
    "route_fused_router_workspace_size",
    "route_dispatch_metadata",
    "route_dispatch_workspace_size",
    "route_dispatch_metadata_noalloc",
    "route_fuse_shared_expert",
    "route_sort_ids",
    "route_status_str",
)

_lib = None


class RouteError(RuntimeError):
    """A kernel launch failed (ROUTE_ELAUNCH)."""


def lib() -> ctypes.CDLL:
    """The loaded C library with argument types set (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m moe_expert_routing_amd.build` "
            "(the routing path has no fallback)")
    L = ctypes.CDLL(LIB_PATH)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.route_topk_softmax.argtypes = [p, i32, i64, i32, i32, i32, p, p, p]
    L.route_grouped_topk.argtypes = [p, i32, i64, i32, i32, i32, i32, i32, i32, p, p, p]
    L.route_biased_grouped_topk.argtypes = [p, i32, p, i32, i64, i32, i32, i32, i32, i32, p, p,
                                            p]
    L.route_fused_router.argtypes = [p, p, i64, i32, i32, i32, p, i32, i32, i32, i32, i32, i32,
                                     ctypes.c_float, p, p, p, ctypes.c_size_t, p]
    L.route_fused_router_workspace_size.argtypes = [i64, i32, i32]
    L.route_fused_router_workspace_size.restype = ctypes.c_size_t
    L.route_dispatch_metadata.argtypes = [p, p, i64, i32, i32, p, p, p, p, p, p, ctypes.c_size_t,
                                          p]
    L.route_dispatch_workspace_size.argtypes = [i64, i32, i32]
    L.route_dispatch_metadata_noalloc.argtypes = [p, p, i64, i32, i32, p, p, p, p, p, p]
    L.route_fuse_shared_expert.argtypes = [p, p, i64, i32, p, ctypes.c_float, p]
    L.route_sort_ids.argtypes = [p, p, i64, i32, p]
    L.route_dispatch_workspace_size.restype = ctypes.c_size_t
    for name in EXPORTED[:-1]:
        if not name.endswith("_workspace_size"):
            getattr(L, name).restype = i32
    L.route_status_str.argtypes = [i32]
    L.route_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def status_str(code: int) -> str:
    return lib().route_status_str(code).decode()


def _check(code: int, what: str):
    if code == ROUTE_OK:
        return
    msg = f"{what}: {status_str(code)}"
    if code in (ROUTE_EINVAL, ROUTE_ENOTSUP, ROUTE_ETOOBIG):
        raise ValueError(msg)
    raise RouteError(msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ROUTE_F32
    if t.dtype == torch.bfloat16:
        return ROUTE_BF16
    raise ValueError(f"router logits must be float32 or bfloat16, got {t.dtype}")


def _bias_code(bias, E) -> int:
    """dtype code of a correction bias of shape [E] (float32, or bfloat16 as the
    aiter-style call passes it in the logits' dtype); float32 for None."""
    if bias is None:
        return ROUTE_F32
    if tuple(bias.shape) != (E,):
        raise ValueError(f"correction_bias must have shape [{E}]")
    if bias.dtype == torch.float32:
        return ROUTE_F32
    if bias.dtype == torch.bfloat16:
        return ROUTE_BF16
    raise ValueError(f"correction_bias must be float32 or bfloat16, got {bias.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_device(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _outputs(M, K, device, topk_weights, topk_ids):
    if topk_weights is None:
        topk_weights = torch.empty((M, K), dtype=torch.float32, device=device)
    if topk_ids is None:
        topk_ids = torch.empty((M, K), dtype=torch.int32, device=device)
    if topk_weights.dtype != torch.float32 or topk_ids.dtype != torch.int32:
        raise ValueError("topk_weights must be float32 and topk_ids int32")
    if tuple(topk_weights.shape) != (M, K) or tuple(topk_ids.shape) != (M, K):
        raise ValueError(f"outputs must have shape ({M}, {K})")
    return topk_weights, topk_ids


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _scoring_code(scoring_func) -> int:
    codes = {"softmax": ROUTE_SOFTMAX, "sigmoid": ROUTE_SIGMOID}
    if scoring_func not in codes:
        raise ValueError(f"Invalid scoring function: {scoring_func}")
    return codes[scoring_func]


def route_topk_softmax(gating_output, top_k, renormalize=False, topk_weights=None, topk_ids=None,
                       stream=None):
    """Softmax top-k over [M, E] logits; returns (topk_weights f32, topk_ids i32)."""
    M, E = gating_output.shape
    w, ids = _outputs(M, top_k, gating_output.device, topk_weights, topk_ids)
    _need_device(gating_output, w, ids)
    _check(lib().route_topk_softmax(_ptr(gating_output), _dtype_code(gating_output), M, E, top_k,
                                    int(bool(renormalize)), _ptr(w), _ptr(ids),
                                    _stream(gating_output.device, stream)),
           "route_topk_softmax")
    return w, ids


def route_grouped_topk(gating_output, top_k, num_expert_group, topk_group, renormalize=False,
                       scoring_func="softmax", topk_weights=None, topk_ids=None, stream=None):
    """Grouped top-k with the per-group max as group score."""
    M, E = gating_output.shape
    w, ids = _outputs(M, top_k, gating_output.device, topk_weights, topk_ids)
    _need_device(gating_output, w, ids)
    _check(lib().route_grouped_topk(_ptr(gating_output), _dtype_code(gating_output), M, E, top_k,
                                    num_expert_group, topk_group, int(bool(renormalize)),
                                    _scoring_code(scoring_func), _ptr(w), _ptr(ids),
                                    _stream(gating_output.device, stream)),
           "route_grouped_topk")
    return w, ids


def route_biased_grouped_topk(gating_output, correction_bias, top_k, num_expert_group=1,
                              topk_group=1, renormalize=False, topk_weights=None, topk_ids=None,
                              stream=None):
    """Sigmoid + correction bias, top-2-sum group score; weights are unbiased.
    correction_bias: None, or [E] float32 or bfloat16 (widened exactly)."""
    M, E = gating_output.shape
    w, ids = _outputs(M, top_k, gating_output.device, topk_weights, topk_ids)
    bias_code = _bias_code(correction_bias, E)
    _need_device(gating_output, correction_bias, w, ids)
    _check(lib().route_biased_grouped_topk(_ptr(gating_output), _dtype_code(gating_output),
                                           _ptr(correction_bias), bias_code, M, E, top_k,
                                           num_expert_group,
                                           topk_group, int(bool(renormalize)), _ptr(w), _ptr(ids),
                                           _stream(gating_output.device, stream)),
           "route_biased_grouped_topk")
    return w, ids


def route_fused_router_workspace_size(num_tokens, hidden_dim, num_experts) -> int:
    """Bytes of device workspace the few-token path of route_fused_router uses
    (0: that shape runs as one kernel)."""
    return int(lib().route_fused_router_workspace_size(num_tokens, hidden_dim, num_experts))


def route_fused_router(hidden_states, router_weight, top_k, num_expert_group=1, topk_group=1,
                       renormalize=False, scoring_func="sigmoid", correction_bias=None,
                       group_score="top2sum", topk_weights=None, topk_ids=None, stream=None,
                       logit_softcap=0.0, workspace=None):
    """bf16 router projection [M,H] x [H,E] followed by routing; logit_softcap
    c != 0 replaces each logit l by c * tanh(l / c) before scoring.

    workspace: None allocates the workspace the library asks for (a uint8
    device tensor from torch's caching allocator), False passes none (always
    the single fused kernel), or a uint8 device tensor of at least
    route_fused_router_workspace_size(M, H, E) bytes."""
    M, H = hidden_states.shape
    H2, E = router_weight.shape
    if H2 != H:
        raise ValueError("hidden_states and router_weight disagree on the hidden size")
    if hidden_states.dtype != torch.bfloat16 or router_weight.dtype != torch.bfloat16:
        raise ValueError("fused router operands must be bfloat16")
    rules = {"max": ROUTE_GROUP_MAX, "top2sum": ROUTE_GROUP_TOP2_SUM}
    if group_score not in rules:
        raise ValueError(f"unknown group score {group_score!r}")
    bias_code = _bias_code(correction_bias, E)
    w, ids = _outputs(M, top_k, hidden_states.device, topk_weights, topk_ids)
    ws_ptr, ws_bytes = None, 0
    if workspace is None:
        need = route_fused_router_workspace_size(M, H, E)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=hidden_states.device)
    if workspace is not None and workspace is not False:
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
        _need_device(workspace)
    _need_device(hidden_states, router_weight, correction_bias, w, ids)
    _check(lib().route_fused_router(_ptr(hidden_states), _ptr(router_weight), M, H, E,
                                    _scoring_code(scoring_func), _ptr(correction_bias),
                                    bias_code, rules[group_score], top_k, num_expert_group,
                                    topk_group,
                                    int(bool(renormalize)), float(logit_softcap), _ptr(w),
                                    _ptr(ids), ws_ptr, ws_bytes,
                                    _stream(hidden_states.device, stream)),
           "route_fused_router")
    return w, ids


def route_dispatch_workspace_size(num_tokens, top_k, num_experts) -> int:
    """Bytes of device workspace route_dispatch_metadata needs (0: invalid shape)."""
    return int(lib().route_dispatch_workspace_size(num_tokens, top_k, num_experts))


def route_dispatch_metadata(topk_ids, num_experts, topk_weights=None, workspace=None,
                            stream=None, out=None):
    """Expert-sorted dispatch metadata of a routing result: the assignments
    a = token * top_k + slot in order of expert id (stable), ids outside
    [0, num_experts) dropped.  Returns (expert_counts [E], expert_offsets
    [E+1], gather_idx [M*K], scatter_idx [M*K], sorted_weights [M*K] or None),
    all int32 / float32 tensors on the ids' device.  `workspace` (a uint8
    tensor of at least route_dispatch_workspace_size bytes) is allocated when
    not given; so are the outputs unless `out` holds those five tensors
    (sorted_weights None when topk_weights is None), which are then filled and
    returned."""
    M, K = topk_ids.shape
    dev = topk_ids.device
    if topk_ids.dtype != torch.int32:
        raise ValueError("topk_ids must be int32")
    if topk_weights is not None and (topk_weights.dtype != torch.float32 or
                                     tuple(topk_weights.shape) != (M, K)):
        raise ValueError(f"topk_weights must be float32 of shape ({M}, {K})")
    need = route_dispatch_workspace_size(M, K, num_experts)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    _need_device(topk_ids, topk_weights, workspace)
    if out is None:
        counts = torch.empty(num_experts, dtype=torch.int32, device=dev)
        offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
        gather = torch.empty(M * K, dtype=torch.int32, device=dev)
        scatter = torch.empty(M * K, dtype=torch.int32, device=dev)
        sw = None if topk_weights is None else torch.empty(M * K, dtype=torch.float32, device=dev)
    else:
        counts, offsets, gather, scatter, sw = out
        want = ((counts, torch.int32, (num_experts,)), (offsets, torch.int32, (num_experts + 1,)),
                (gather, torch.int32, (M * K,)), (scatter, torch.int32, (M * K,)))
        for t, dt, shape in want:
            if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous():
                raise ValueError(f"out tensors must be contiguous {dt} of shape {shape}")
        if (sw is None) != (topk_weights is None):
            raise ValueError("out sorted_weights must be given exactly when topk_weights is")
        if sw is not None and (sw.dtype != torch.float32 or tuple(sw.shape) != (M * K,)
                               or not sw.is_contiguous()):
            raise ValueError(f"out sorted_weights must be contiguous float32 of shape ({M * K},)")
        _need_device(topk_ids, counts, offsets, gather, scatter, sw)
    _check(lib().route_dispatch_metadata(_ptr(topk_ids), _ptr(topk_weights), M, K, num_experts,
                                         _ptr(counts), _ptr(offsets), _ptr(gather),
                                         _ptr(scatter), _ptr(sw), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(),
                                         _stream(dev, stream)),
           "route_dispatch_metadata")
    return counts, offsets, gather, scatter, sw


def route_fuse_shared_expert(topk_weights, topk_ids, shared_expert_ids,
                             routed_scaling_factor=None, stream=None):
    """In place: each row's last slot gets its shared-expert id and, with a
    routed scaling factor, the sum of the row's other weights divided by it.
    Returns (topk_weights, topk_ids)."""
    M, K = topk_ids.shape
    if topk_weights.dtype != torch.float32 or topk_ids.dtype != torch.int32:
        raise ValueError("topk_weights must be float32 and topk_ids int32")
    if shared_expert_ids.dtype != torch.int32 or shared_expert_ids.numel() != M:
        raise ValueError(f"shared_expert_ids must be int32 with {M} entries")
    _need_device(topk_weights, topk_ids, shared_expert_ids)
    rsf = 0.0 if routed_scaling_factor is None else float(routed_scaling_factor)
    _check(lib().route_fuse_shared_expert(_ptr(topk_weights), _ptr(topk_ids), M, K,
                                          _ptr(shared_expert_ids), rsf,
                                          _stream(topk_ids.device, stream)),
           "route_fuse_shared_expert")
    return topk_weights, topk_ids


def route_sort_ids(topk_weights, topk_ids, stream=None):
    """In place: each row's (id, weight) pairs in ascending id order."""
    M, K = topk_ids.shape
    if topk_weights.dtype != torch.float32 or topk_ids.dtype != torch.int32:
        raise ValueError("topk_weights must be float32 and topk_ids int32")
    _need_device(topk_weights, topk_ids)
    _check(lib().route_sort_ids(_ptr(topk_weights), _ptr(topk_ids), M, K,
                                _stream(topk_ids.device, stream)), "route_sort_ids")
    return topk_weights, topk_ids
