"""Seeded synthetic inputs for the MoE routing workloads.

This module holds no routing arithmetic: it only draws random numbers and
rounds fp32 draws to bf16.  Both the oracle-side tests and the GPU path read
the very same bytes it produces.

Distributions follow the workload descriptions, read as N(mean, variance):
logits ~ N(0, 2) means standard deviation sqrt(2); a router weight
~ N(0, 1/7168) has standard deviation 1/sqrt(7168), which makes the router
logits unit-scale.  Draws are numpy PCG64 (``default_rng(seed)``) in fp32;
bf16 values are the round-to-nearest-even of those fp32 draws.

Seeds: logits 0, bias 1, router weight 2 (the fused router's hidden states
use seed 0).  They stand in for real router logits of the models the pages
name (MiniMax-M2.5, DeepSeek-V2/V3); no model weights are used.
"""
from __future__ import annotations

import dataclasses

import numpy as np

SEED_LOGITS, SEED_BIAS, SEED_W = 0, 1, 2


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32
    )


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    entry: str             # C-ABI entry point that serves it
    M: int
    E: int
    K: int
    G: int = 1             # num_expert_group
    TG: int = 1            # topk_group
    scoring: str = "softmax"
    group_rule: str = "max"
    renormalize: bool = False
    dtype: str = "f32"     # logits dtype: "f32" or "bf16"
    logit_std: float = 1.0
    bias: str | None = None  # None, "uniform:<a>" (U(-a, a)) or "normal:<std>"
    hidden_dim: int = 0    # fused router only
    w_std: float = 0.0     # fused router only
    softcap: float = 0.0   # fused router only: logits -> c * tanh(logits / c)


WORKLOADS = {
    # Softmax top-k, Mixtral-like small case.
    "softmax_e8_k2": Workload("softmax_e8_k2", "route_topk_softmax", M=128, E=8, K=2,
                              scoring="softmax", renormalize=True, dtype="f32"),
    # Sigmoid + correction bias, ungrouped (MiniMax-M2.5-like call with G=1, TG=1).
    "sigmoid_bias_e256_k8": Workload("sigmoid_bias_e256_k8", "route_biased_grouped_topk",
                                     M=4096, E=256, K=8, G=1, TG=1, scoring="sigmoid",
                                     group_rule="top2sum", renormalize=True, dtype="bf16",
                                     logit_std=2.0 ** 0.5, bias="uniform:0.05"),
    # Grouped softmax top-k, DeepSeek-V2 shape.
    "grouped_softmax_e160": Workload("grouped_softmax_e160", "route_grouped_topk",
                                     M=16384, E=160, K=6, G=8, TG=3, scoring="softmax",
                                     group_rule="max", renormalize=False, dtype="f32"),
    # Biased grouped top-k, DeepSeek-V3 shape (M is swept).
    "biased_grouped_e256": Workload("biased_grouped_e256", "route_biased_grouped_topk",
                                    M=65536, E=256, K=8, G=8, TG=4, scoring="sigmoid",
                                    group_rule="top2sum", renormalize=True, dtype="bf16",
                                    logit_std=2.0 ** 0.5, bias="normal:" + repr(0.02 ** 0.5)),
    # Fused router projection + biased grouped top-k epilogue.
    "fused_router_h7168": Workload("fused_router_h7168", "route_fused_router",
                                   M=8192, E=256, K=8, G=8, TG=4, scoring="sigmoid",
                                   group_rule="top2sum", renormalize=True, dtype="bf16",
                                   bias="normal:" + repr(0.02 ** 0.5), hidden_dim=7168,
                                   w_std=(1.0 / 7168) ** 0.5),
    # Fused router with few experts (Mixtral/Grok-like: hidden 4096, 8
    # experts, top-2 softmax, logits soft-capped at 30), the vector-ALU path.
    "fused_router_e8_h4096": Workload("fused_router_e8_h4096", "route_fused_router",
                                      M=8192, E=8, K=2, scoring="softmax", renormalize=False,
                                      dtype="bf16", hidden_dim=4096, w_std=(1.0 / 4096) ** 0.5,
                                      softcap=30.0),
    # 16 experts (DBRX-like: hidden 6144, top-4 softmax, renormalised).
    "fused_router_e16_h6144": Workload("fused_router_e16_h6144", "route_fused_router",
                                       M=8192, E=16, K=4, scoring="softmax", renormalize=True,
                                       dtype="bf16", hidden_dim=6144,
                                       w_std=(1.0 / 6144) ** 0.5),
}

BIASED_GROUPED_M_SWEEP = (1, 4, 16, 64, 128, 1024, 8192, 65536)


def _draw_normal(seed: int, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def make_bias(wl: Workload, seed: int = SEED_BIAS):
    if wl.bias is None:
        return None
    kind, val = wl.bias.split(":")
    rng = np.random.default_rng(seed)
    if kind == "uniform":
        a = float(val)
        return rng.uniform(-a, a, size=wl.E).astype(np.float32)
    if kind == "normal":
        return rng.standard_normal(wl.E, dtype=np.float32) * np.float32(float(val))
    raise ValueError(wl.bias)


def make_logits(wl: Workload, M: int | None = None, seed: int = SEED_LOGITS) -> np.ndarray:
    """[M, E] logits: float32, or uint16 bf16 bit patterns when wl.dtype == 'bf16'."""
    M = wl.M if M is None else M
    x = _draw_normal(seed, (M, wl.E), wl.logit_std)
    return bf16_bits_from_f32(x) if wl.dtype == "bf16" else x


def make_router_inputs(wl: Workload, M: int | None = None, seed_hidden: int = SEED_LOGITS,
                       seed_w: int = SEED_W):
    """(hidden [M,H] bf16 bits, W [H,E] bf16 bits) for the fused router."""
    M = wl.M if M is None else M
    hidden = bf16_bits_from_f32(_draw_normal(seed_hidden, (M, wl.hidden_dim), 1.0))
    w = bf16_bits_from_f32(_draw_normal(seed_w, (wl.hidden_dim, wl.E), wl.w_std))
    return hidden, w


def random_logits(rng: np.random.Generator, M: int, E: int, dtype: str, std: float = 1.0):
    """Small random cases for parity sweeps (same conventions as above)."""
    x = rng.standard_normal((M, E), dtype=np.float32) * np.float32(std)
    return bf16_bits_from_f32(x) if dtype == "bf16" else x
