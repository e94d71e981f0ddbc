"""CPU oracle for MoE routing top-k -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``moe_expert_routing_amd``)
never imports it; the two share no code.

The arithmetic lives in ``route_oracle.c`` (plain C99, double precision, one
row at a time); this module only builds/loads that library with ctypes and
marshals numpy arrays.  Every function cites the page section it follows in
the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "route_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_route.so")

F32, BF16, F64 = 0, 1, 2
SOFTMAX, SIGMOID = 0, 1
GROUP_MAX, GROUP_TOP2SUM = 0, 1

_lib = None


def build(force: bool = False) -> str:
    """Compile route_oracle.c with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        p, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.oracle_route.argtypes = [p, i32, i64, i32, p, i32, i32, i32, i32, i32, i32, p, p, p]
        lib.oracle_route.restype = i32
        lib.oracle_row_scores.argtypes = [p, i32, i32, p, i32, p, p]
        lib.oracle_row_scores.restype = i32
        lib.oracle_group_scores.argtypes = [p, i32, i32, i32, p]
        lib.oracle_group_scores.restype = i32
        lib.oracle_router_logits.argtypes = [p, p, i64, i32, i32, p]
        lib.oracle_router_logits.restype = i32
        lib.oracle_dispatch.argtypes = [p, p, i64, i32, p, p, p, p, p]
        lib.oracle_dispatch.restype = i32
        lib.oracle_fuse_shared_expert.argtypes = [p, p, i64, i32, p, ctypes.c_double]
        lib.oracle_fuse_shared_expert.restype = i32
        lib.oracle_sort_ids.argtypes = [p, p, i64, i32]
        lib.oracle_sort_ids.restype = i32
        lib.oracle_softcap.argtypes = [p, i64, ctypes.c_double]
        lib.oracle_softcap.restype = i32
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # raw bf16 bit patterns
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle logits must be float32, float64 or uint16(bf16 bits), got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def route(logits, top_k, *, scoring=SOFTMAX, bias=None, num_expert_group=1, topk_group=1,
          group_rule=GROUP_MAX, renormalize=False, with_gaps=False):
    """Route every row of ``logits`` [M, E].

    Returns (weights float32 [M,K], ids int32 [M,K]) and, with ``with_gaps``,
    a float64 [M,3] array: (K-boundary gap, smallest in-order gap, group-boundary gap).
    """
    lib = _load()
    x = np.ascontiguousarray(logits)
    if x.ndim != 2:
        raise ValueError("logits must be 2-D [M, E]")
    M, E = x.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    if b is not None and b.shape != (E,):
        raise ValueError("bias must have shape [E]")
    w = np.empty((M, top_k), np.float32)
    ids = np.empty((M, top_k), np.int32)
    gaps = np.empty((M, 3), np.float64) if with_gaps else None
    rc = lib.oracle_route(_ptr(x), _dtype_code(x), M, E, _ptr(b), scoring, group_rule,
                          num_expert_group, topk_group, top_k, int(bool(renormalize)),
                          _ptr(w), _ptr(ids), _ptr(gaps))
    if rc != 0:
        raise ValueError("oracle_route: arguments outside the method's definition")
    return (w, ids, gaps) if with_gaps else (w, ids)


def row_scores(logits_row, *, scoring=SOFTMAX, bias=None):
    """(s, c) float64 [E] for one row: unbiased scores and selection scores."""
    lib = _load()
    x = np.ascontiguousarray(logits_row)
    E = x.shape[0]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    s = np.empty(E, np.float64)
    c = np.empty(E, np.float64)
    if lib.oracle_row_scores(_ptr(x), _dtype_code(x), E, _ptr(b), scoring, _ptr(s), _ptr(c)):
        raise ValueError("oracle_row_scores: bad arguments")
    return s, c


def group_scores(c_row, num_expert_group, group_rule):
    """Group scores float64 [G] of one row's selection scores."""
    lib = _load()
    c = np.ascontiguousarray(c_row, dtype=np.float64)
    h = np.empty(num_expert_group, np.float64)
    if lib.oracle_group_scores(_ptr(c), c.shape[0], num_expert_group, group_rule, _ptr(h)):
        raise ValueError("oracle_group_scores: bad arguments")
    return h


def router_logits(hidden_bits, w_bits):
    """float64 [M,E] = hidden [M,H] (bf16 bits) @ W [H,E] (bf16 bits), exact products."""
    lib = _load()
    a = np.ascontiguousarray(hidden_bits, dtype=np.uint16)
    b = np.ascontiguousarray(w_bits, dtype=np.uint16)
    M, H = a.shape
    H2, E = b.shape
    if H != H2:
        raise ValueError("hidden and W disagree on H")
    out = np.empty((M, E), np.float64)
    if lib.oracle_router_logits(_ptr(a), _ptr(b), M, H, E, _ptr(out)):
        raise ValueError("oracle_router_logits: bad arguments")
    return out


def dispatch(topk_ids, num_experts, topk_weights=None):
    """Expert-sorted dispatch metadata of a routing result (stable counting
    sort of the flattened assignments by expert id; ids outside
    [0, num_experts) are dropped).  Returns (counts [E], offsets [E+1],
    gather [n], scatter [n], sorted_weights [n] or None), n = topk_ids.size."""
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32).reshape(-1)
    n = ids.size
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights,
                                                               dtype=np.float32).reshape(-1)
    counts = np.empty(num_experts, np.int32)
    offsets = np.empty(num_experts + 1, np.int32)
    gather = np.empty(n, np.int32)
    scatter = np.empty(n, np.int32)
    sw = None if w is None else np.empty(n, np.float32)
    rc = _load().oracle_dispatch(_ptr(ids), _ptr(w), n, num_experts, _ptr(counts),
                                 _ptr(offsets), _ptr(gather), _ptr(scatter), _ptr(sw))
    if rc != 0:
        raise ValueError(f"oracle_dispatch rejected its arguments (code {rc})")
    return counts, offsets, gather, scatter, sw


def fuse_shared_expert(topk_weights, topk_ids, shared_ids, routed_scaling_factor=None):
    """The shared-expert slot: returns copies of (weights, ids) whose last slot
    holds shared_ids[m] and, when routed_scaling_factor is given, the sum of
    the row's other weights divided by it."""
    w = np.array(topk_weights, dtype=np.float32, copy=True, order="C")
    ids = np.array(topk_ids, dtype=np.int32, copy=True, order="C")
    sid = np.ascontiguousarray(shared_ids, dtype=np.int32).reshape(-1)
    M, K = ids.shape
    if sid.size != M:
        raise ValueError("shared_ids needs one id per token")
    rsf = 0.0 if routed_scaling_factor is None else float(routed_scaling_factor)
    rc = _load().oracle_fuse_shared_expert(_ptr(w), _ptr(ids), M, K, _ptr(sid), rsf)
    if rc != 0:
        raise ValueError(f"oracle_fuse_shared_expert rejected its arguments (code {rc})")
    return w, ids


def sort_ids(topk_weights, topk_ids):
    """Copies of (weights, ids) with each row's pairs in ascending id order."""
    w = np.array(topk_weights, dtype=np.float32, copy=True, order="C")
    ids = np.array(topk_ids, dtype=np.int32, copy=True, order="C")
    M, K = ids.shape
    rc = _load().oracle_sort_ids(_ptr(w), _ptr(ids), M, K)
    if rc != 0:
        raise ValueError(f"oracle_sort_ids rejected its arguments (code {rc})")
    return w, ids


def softcap(logits, cap):
    """cap * tanh(logits / cap) in double (cap == 0: unchanged); returns a copy."""
    x = np.array(logits, dtype=np.float64, copy=True, order="C")
    rc = _load().oracle_softcap(_ptr(x), x.size, float(cap))
    if rc != 0:
        raise ValueError(f"oracle_softcap rejected its arguments (code {rc})")
    return x
