"""Helpers for the GPU tests: move the shared seeded inputs to the device and
call the binding for a workload."""
import sys

import numpy as np
import torch

import moe_expert_routing_amd as mr
import oracle


def oracle_router_logits(hidden, w, chunk=64):
    """The oracle's exact router logits of every row, computed in row chunks
    on a pool of host threads (the oracle's C routine releases the GIL); the
    arithmetic is the oracle's own, row by row."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    M = hidden.shape[0]
    starts = range(0, M, chunk)
    workers = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(lambda s: oracle.router_logits(hidden[s:s + chunk], w), starts))
    return np.concatenate(parts, axis=0) if parts else np.empty((0, w.shape[1]))


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(a: np.ndarray) -> torch.Tensor:
    """float32 stays float32; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


SCORING = {"softmax": oracle.SOFTMAX, "sigmoid": oracle.SIGMOID}
RULE = {"max": oracle.GROUP_MAX, "top2sum": oracle.GROUP_TOP2SUM}


def route_gpu(entry, x, *, K, G=1, TG=1, scoring="softmax", bias=None, renorm=False,
              stream=None, out=None):
    """Call one routing entry point; returns (weights, ids) as numpy arrays."""
    w, ids = (None, None) if out is None else out
    if entry == "route_topk_softmax":
        assert G == 1 and scoring == "softmax"
        w, ids = mr.route_topk_softmax(x, K, renorm, w, ids, stream=stream)
    elif entry == "route_grouped_topk":
        w, ids = mr.route_grouped_topk(x, K, G, TG, renorm, scoring, w, ids, stream=stream)
    elif entry == "route_biased_grouped_topk":
        w, ids = mr.route_biased_grouped_topk(x, bias, K, G, TG, renorm, w, ids, stream=stream)
    else:
        raise ValueError(entry)
    torch.cuda.synchronize()
    return w.cpu().numpy(), ids.cpu().numpy()


def oracle_args(entry, scoring):
    """(scoring code, group rule code) the oracle uses for an entry point."""
    if entry == "route_biased_grouped_topk":
        return oracle.SIGMOID, oracle.GROUP_TOP2SUM
    return SCORING[scoring], oracle.GROUP_MAX
