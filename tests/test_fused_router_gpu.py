"""GPU parity of route_fused_router (bf16 router projection on MFMA + routing
epilogue) against the oracle: the oracle's logits are the exact double
products summed in double, then routed exactly like the standalone oracle."""
import numpy as np
import pytest
import torch

import moe_expert_routing_amd as mr
import oracle
from gpu_util import log, oracle_router_logits, to_device
from parity_check import compare
from workloads import (WORKLOADS, bf16_bits_from_f32, make_bias, make_router_inputs)

pytestmark = pytest.mark.gpu

SC = {"sigmoid": oracle.SIGMOID, "softmax": oracle.SOFTMAX}
RU = {"top2sum": oracle.GROUP_TOP2SUM, "max": oracle.GROUP_MAX}


def _inputs(rng, M, H, E=256, bias=True):
    hidden = bf16_bits_from_f32(rng.standard_normal((M, H), dtype=np.float32))
    w = bf16_bits_from_f32(rng.standard_normal((H, E), dtype=np.float32) * np.float32(H ** -0.5))
    b = (rng.standard_normal(E, dtype=np.float32) * np.float32(0.02 ** 0.5)) if bias else None
    return hidden, w, b


def _run(hidden, w, b, K, G, TG, renorm, scoring, rule, workspace=None, cap=0.0):
    wt, ids = mr.route_fused_router(to_device(hidden), to_device(w), K, G, TG, renorm, scoring,
                                    None if b is None else to_device(b), rule,
                                    logit_softcap=cap, workspace=workspace)
    torch.cuda.synchronize()
    return wt.cpu().numpy(), ids.cpu().numpy()


def _check(hidden, w, b, wt, ids, rows, K, G, TG, renorm, scoring, rule):
    logits = oracle.router_logits(hidden[rows], w)
    rep = compare(logits, wt[rows], ids[rows], scoring=SC[scoring], bias=b, G=G, TG=TG,
                  rule=RU[rule], K=K, renorm=renorm)
    log(f"[gpu]   {rep.summary()}")
    assert rep.ok(), rep.summary()
    return rep


@pytest.mark.parametrize("M,H,G,TG,K,scoring,rule,bias,renorm", [
    (77, 128, 8, 4, 8, "sigmoid", "top2sum", True, True),     # ragged last block
    (32, 64, 8, 4, 8, "sigmoid", "top2sum", True, False),     # one step of K
    (200, 512, 1, 1, 8, "sigmoid", "top2sum", True, True),    # ungrouped
    (65, 256, 8, 3, 6, "softmax", "max", False, False),       # softmax, group max
    (96, 192, 8, 2, 4, "sigmoid", "max", False, True),        # sigmoid, no bias
    (1, 64, 8, 4, 8, "sigmoid", "top2sum", True, True),       # single token
])
@pytest.mark.parametrize("path", ["one_kernel", "default"])
def test_fused_router_small(M, H, G, TG, K, scoring, rule, bias, renorm, path):
    """path one_kernel passes no workspace (projection and routing in one
    kernel); default lets the binding pass the workspace the library asks for
    (the split path whenever H spans two or more steps of 64)."""
    rng = np.random.default_rng(M * 1000 + H)
    hidden, w, b = _inputs(rng, M, H, bias=bias)
    log(f"[gpu] route_fused_router M={M} H={H} G={G} TG={TG} K={K} {scoring} {rule} "
        f"bias={bias} {path}")
    wt, ids = _run(hidden, w, b, K, G, TG, renorm, scoring, rule,
                   workspace=False if path == "one_kernel" else None)
    _check(hidden, w, b, wt, ids, np.arange(M), K, G, TG, renorm, scoring, rule)


@pytest.mark.parametrize("K", [1, 5])
@pytest.mark.parametrize("G,TG", [(8, 4), (1, 1)])
@pytest.mark.parametrize("path", ["one_kernel", "default"])
def test_fused_router_biased_k_below_eight(K, G, TG, path):
    """The biased epilogues unroll their merge rounds to eight and leave after
    the K-th."""
    M, H = 130, 512
    rng = np.random.default_rng(700 + 10 * K + G)
    hidden, w, b = _inputs(rng, M, H, bias=True)
    log(f"[gpu] route_fused_router M={M} H={H} G={G} TG={TG} K={K} biased {path}")
    wt, ids = _run(hidden, w, b, K, G, TG, True, "sigmoid", "top2sum",
                   workspace=False if path == "one_kernel" else None)
    _check(hidden, w, b, wt, ids, np.arange(M), K, G, TG, True, "sigmoid", "top2sum")


@pytest.mark.parametrize("M,H,G,TG,K,scoring,rule,bias,renorm,cap", [
    (200, 256, 1, 1, 2, "softmax", "max", False, False, 30.0),   # top-2 softmax, cap 30
    (77, 512, 1, 1, 1, "softmax", "max", False, False, 5.0),     # top-1 softmax
    (96, 128, 8, 4, 8, "sigmoid", "top2sum", True, True, 2.0),   # a cap that saturates
    (3000, 256, 1, 1, 4, "softmax", "max", False, False, 5.0),   # 64-row tiles, 4 splits
    (6200, 256, 8, 4, 8, "sigmoid", "top2sum", True, True, 30.0),  # 128-row tiles, 4 splits
])
def test_fused_router_softcap(M, H, G, TG, K, scoring, rule, bias, renorm, cap):
    """Soft-capped logits: the oracle caps its exact logits in double."""
    rng = np.random.default_rng(M + H)
    hidden, w, b = _inputs(rng, M, H, bias=bias)
    hidden = bf16_bits_from_f32(rng.standard_normal((M, H), dtype=np.float32) * np.float32(3))
    log(f"[gpu] route_fused_router softcap={cap} M={M} H={H} K={K} {scoring}")
    wt, ids = mr.route_fused_router(to_device(hidden), to_device(w), K, G, TG, renorm, scoring,
                                    None if b is None else to_device(b), rule,
                                    logit_softcap=cap)
    torch.cuda.synchronize()
    logits = oracle.softcap(oracle.router_logits(hidden, w), cap)
    rep = compare(logits, wt.cpu().numpy(), ids.cpu().numpy(), scoring=SC[scoring], bias=b, G=G,
                  TG=TG, rule=RU[rule], K=K, renorm=renorm)
    log(f"[gpu]   {rep.summary()}")
    assert rep.ok(), rep.summary()


@pytest.mark.parametrize("G,TG", [(8, 4), (1, 1)])
def test_fused_router_one_lane_holds_most_picks(G, TG):
    """A bias that lifts the first 16 experts puts most of the top 8 of a
    row in one lane's candidates, more than its short list keeps: the
    epilogue must take its exact path there."""
    rng = np.random.default_rng(5 + G)
    M, H = 160, 256
    hidden, w, b = _inputs(rng, M, H)
    b[:16] += np.float32(0.6)
    log(f"[gpu] route_fused_router skewed bias G={G} TG={TG}")
    wt, ids = _run(hidden, w, b, 8, G, TG, True, "sigmoid", "top2sum", workspace=False)
    assert (ids < 16).sum(axis=1).mean() > 6  # most rows take 5+ picks from one lane
    _check(hidden, w, b, wt, ids, np.arange(M), 8, G, TG, True, "sigmoid", "top2sum")


@pytest.mark.parametrize("M,H,G,TG,K,scoring,rule,bias,renorm,cap", [
    (1, 7168, 8, 4, 8, "sigmoid", "top2sum", True, True, 0.0),      # 112 one-step splits
    (7, 448, 8, 4, 8, "sigmoid", "top2sum", True, False, 0.0),      # 7 one-step splits
    (77, 1024, 1, 1, 8, "sigmoid", "top2sum", True, True, 0.0),     # 3 tiles, 4 splits, ungrouped
    (300, 640, 8, 3, 6, "softmax", "max", False, False, 0.0),       # 10 tiles, 3 uneven splits
    (1000, 384, 1, 1, 2, "softmax", "max", False, False, 30.0),     # top-2 softmax, capped
    pytest.param(130, 7168, 8, 4, 8, "sigmoid", "top2sum", True, True, 2.0,  # saturating cap
                 marks=pytest.mark.skip(reason=(
                     "an experimental main-loop variant (lighter copies past a split's last "
                     "step) faulted the GPU on this case; the variant was removed and the case "
                     "stays off the GPU until that fault's cause is shown"))),
    (130, 2048, 8, 4, 8, "sigmoid", "top2sum", True, True, 2.0),    # saturating cap, 8 splits
    (400, 7168, 8, 4, 8, "sigmoid", "top2sum", True, True, 0.0),    # 19 splits, a block per row
    (3000, 640, 8, 4, 8, "sigmoid", "top2sum", True, True, 0.0),    # 64-row tiles, ragged
    (2100, 1024, 1, 1, 2, "softmax", "max", False, False, 30.0),    # 64-row tiles, capped
])
def test_fused_router_split_path(M, H, G, TG, K, scoring, rule, bias, renorm, cap):
    """Few tokens: the hidden dimension is split over workgroups, partial
    logits summed by a second kernel and routed by the routing kernel."""
    assert mr.route_fused_router_workspace_size(M, H, 256) > 0
    rng = np.random.default_rng(M * 7 + H)
    hidden, w, b = _inputs(rng, M, H, bias=bias)
    if cap:
        hidden = bf16_bits_from_f32(rng.standard_normal((M, H), dtype=np.float32) * np.float32(3))
    log(f"[gpu] route_fused_router split path M={M} H={H} G={G} TG={TG} K={K} {scoring} "
        f"cap={cap}")
    wt, ids = _run(hidden, w, b, K, G, TG, renorm, scoring, rule, cap=cap)
    logits = oracle.router_logits(hidden, w)
    if cap:
        logits = oracle.softcap(logits, cap)
    rep = compare(logits, wt, ids, scoring=SC[scoring], bias=b, G=G, TG=TG, rule=RU[rule], K=K,
                  renorm=renorm)
    log(f"[gpu]   {rep.summary()}")
    assert rep.ok(), rep.summary()
    # the single fused kernel on the same input agrees with the oracle as well
    wt1, ids1 = _run(hidden, w, b, K, G, TG, renorm, scoring, rule, workspace=False, cap=cap)
    rep1 = compare(logits, wt1, ids1, scoring=SC[scoring], bias=b, G=G, TG=TG, rule=RU[rule],
                   K=K, renorm=renorm)
    assert rep1.ok(), rep1.summary()


@pytest.fixture(scope="module")
def h7168():
    """The full 8192-token, 7168-wide workload and the oracle's exact logits
    of every row (computed once for the module)."""
    wl = WORKLOADS["fused_router_h7168"]
    hidden, w = make_router_inputs(wl)
    log(f"[gpu] oracle logits of all {wl.M} rows of {wl.name} ...")
    logits = oracle_router_logits(hidden, w)
    return wl, hidden, w, make_bias(wl), logits


def _check_all_rows(wl, logits, b, wt, ids, label):
    rep = compare(logits, wt, ids, scoring=oracle.SIGMOID, bias=b, G=wl.G, TG=wl.TG,
                  rule=oracle.GROUP_TOP2SUM, K=wl.K, renorm=wl.renormalize, label=label)
    log(f"[gpu]   {rep.summary()}")
    assert rep.ok(), rep.summary()
    assert rep.near_tie <= max(2, rep.rows // 1000), rep.summary()


@pytest.mark.parametrize("M,splits", [(4096, 4), (6144, 2), (7001, 4), (8192, 4)])
def test_fused_router_split_path_full_width(h7168, M, splits):
    """The 7168-wide router on the split path, every row against the oracle:
    64-row tiles at 4096 tokens (4 splits of 28 steps) and 6144 (2 of 56);
    128-row tiles at 7001 tokens (4 splits, a ragged last tile) and 8192 (4
    splits of 28 steps: the full workload, the library's default launch for
    it)."""
    wl, hidden, w, b, logits = h7168
    assert mr.route_fused_router_workspace_size(M, wl.hidden_dim, wl.E) == \
        4 * 256 * M * splits
    log(f"[gpu] route_fused_router split path M={M} H={wl.hidden_dim} ({splits} splits)")
    wt, ids = _run(hidden[:M], w, b, wl.K, wl.G, wl.TG, wl.renormalize, "sigmoid", "top2sum")
    _check_all_rows(wl, logits[:M], b, wt, ids, f"{wl.name} M={M} split path ({splits} splits)")


@pytest.mark.parametrize("M,H,G,TG,K,scoring,rule,bias", [
    (6500, 512, 8, 4, 8, "sigmoid", "top2sum", True),   # 51 tiles of 128 rows, 4 splits
    (6145, 256, 1, 1, 6, "softmax", "max", False),      # 49 tiles, 4 one-step splits
])
def test_fused_router_128_row_tiles(M, H, G, TG, K, scoring, rule, bias):
    """The partial kernel's 128-row tiles (above 6144 tokens), every row
    against the oracle, ragged last tile included."""
    rng = np.random.default_rng(M + H)
    hidden, w, b = _inputs(rng, M, H, bias=bias)
    log(f"[gpu] route_fused_router 128-row tiles M={M} H={H} G={G} TG={TG} K={K} {scoring}")
    wt, ids = _run(hidden, w, b, K, G, TG, True, scoring, rule)
    _check(hidden, w, b, wt, ids, np.arange(M), K, G, TG, True, scoring, rule)


def test_fused_router_128_row_tiles_workspace_contents():
    """128-row tiles in 4 splits: a workspace full of arbitrary bytes, and
    one reused across calls of other sizes, give the results of a fresh one,
    every row against the oracle."""
    rng = np.random.default_rng(29)
    M, H = 7001, 512
    hidden, w, b = _inputs(rng, M, H)
    need = mr.route_fused_router_workspace_size(M, H, 256)
    assert need == 4 * 256 * M * 4  # 55 tiles of 128 rows, 4 splits of 2 steps
    ws = torch.from_numpy(rng.integers(0, 256, need, dtype=np.uint8)).to("cuda")
    log(f"[gpu] route_fused_router 128-row tiles M={M} H={H}: arbitrary workspace bytes, reuse")
    first = _run(hidden, w, b, 8, 8, 4, True, "sigmoid", "top2sum", workspace=ws)
    _check(hidden, w, b, first[0], first[1], np.arange(M), 8, 8, 4, True, "sigmoid", "top2sum")
    smaller = _run(hidden[:6500], w, b, 8, 8, 4, True, "sigmoid", "top2sum", workspace=ws)
    again = _run(hidden, w, b, 8, 8, 4, True, "sigmoid", "top2sum", workspace=ws)
    fresh = _run(hidden[:6500], w, b, 8, 8, 4, True, "sigmoid", "top2sum")
    assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])
    assert np.array_equal(smaller[0], fresh[0]) and np.array_equal(smaller[1], fresh[1])
    assert np.array_equal(smaller[1], first[1][:6500])


# every epilogue instantiation (scoring, bias, group rule) on every path:
# the single kernel, the split path reduced a block per row (8 splits) and
# a wave per 8 rows (4 splits)
_COMBOS = [("softmax", False, 1, "max"), ("sigmoid", True, 1, "top2sum"), ("sigmoid", False, 1, "max"),
           ("sigmoid", True, 8, "top2sum"), ("sigmoid", False, 8, "top2sum"),
           ("softmax", False, 8, "max"), ("sigmoid", True, 8, "max"), ("sigmoid", False, 8, "max")]
_PATHS = [(96, 256, False), (130, 2048, None), (77, 1024, None)]


@pytest.mark.parametrize("scoring,bias,G,rule", _COMBOS)
@pytest.mark.parametrize("M,H,workspace", _PATHS)
def test_fused_router_every_epilogue(M, H, workspace, scoring, bias, G, rule):
    """Each (scoring, bias, group rule) instantiation of the routing epilogue
    on the single kernel and on both split-path reductions."""
    rng = np.random.default_rng(M * 31 + G * 7 + len(rule) + (3 if bias else 0))
    hidden, w, b = _inputs(rng, M, H, bias=bias)
    TG = 3 if G == 8 else 1
    log(f"[gpu] route_fused_router epilogue {scoring} bias={bias} G={G} {rule} M={M} H={H} "
        f"{'one kernel' if workspace is False else 'split'}")
    wt, ids = _run(hidden, w, b, 6, G, TG, True, scoring, rule, workspace=workspace)
    _check(hidden, w, b, wt, ids, np.arange(M), 6, G, TG, True, scoring, rule)


@pytest.mark.parametrize("M,H,G,TG,workspace", [
    (130, 512, 8, 4, False),   # one kernel
    (130, 2048, 8, 4, None),   # split path, 8 splits: a block per row
    (77, 1024, 1, 1, None),    # split path, 4 splits: a wave per 8 rows, ungrouped
    (3000, 640, 8, 4, None),   # split path, 5 splits: a wave per 8 rows
])
def test_fused_router_wide_bias(M, H, G, TG, workspace):
    """A bias spread wider than 4 takes the exact-comparison selection in the
    routing epilogue of every path."""
    rng = np.random.default_rng(M + H)
    hidden, w, _ = _inputs(rng, M, H, bias=False)
    b = rng.uniform(-3.0, 3.0, 256).astype(np.float32)
    log(f"[gpu] route_fused_router wide bias M={M} H={H} G={G} TG={TG} "
        f"{'one kernel' if workspace is False else 'default'}")
    wt, ids = _run(hidden, w, b, 8, G, TG, True, "sigmoid", "top2sum", workspace=workspace)
    _check(hidden, w, b, wt, ids, np.arange(M), 8, G, TG, True, "sigmoid", "top2sum")


@pytest.mark.parametrize("M,M2,H", [
    (130, 40, 2048),    # 8 splits: a block per row sums them
    (3000, 1000, 640),  # 5 splits each (64- and 32-row tiles): a wave per 8 rows
])
def test_fused_router_split_path_deterministic_and_reused_workspace(M, M2, H):
    """Two calls through one caller-owned workspace, the second smaller:
    bit-identical to fresh calls (the sums run in a fixed order)."""
    rng = np.random.default_rng(13)
    hidden, w, b = _inputs(rng, M, H)
    ws = torch.empty(mr.route_fused_router_workspace_size(M, H, 256), dtype=torch.uint8,
                     device="cuda")
    log(f"[gpu] route_fused_router split path reused workspace M={M} then {M2}, H={H}")
    a = _run(hidden, w, b, 8, 8, 4, True, "sigmoid", "top2sum", workspace=ws)
    c = _run(hidden[:M2], w, b, 8, 8, 4, True, "sigmoid", "top2sum", workspace=ws)
    a2 = _run(hidden, w, b, 8, 8, 4, True, "sigmoid", "top2sum")
    c2 = _run(hidden[:M2], w, b, 8, 8, 4, True, "sigmoid", "top2sum")
    assert np.array_equal(a[0], a2[0]) and np.array_equal(a[1], a2[1])
    assert np.array_equal(c[0], c2[0]) and np.array_equal(c[1], c2[1])


def test_fused_router_full_workload_one_kernel(h7168):
    """The single fused kernel (no workspace) on the full 8192-token workload,
    every row against the oracle."""
    wl, hidden, w, b, logits = h7168
    log(f"[gpu] route_fused_router workload={wl.name} M={wl.M} H={wl.hidden_dim} one kernel")
    wt, ids = _run(hidden, w, b, wl.K, wl.G, wl.TG, wl.renormalize, "sigmoid", "top2sum",
                   workspace=False)
    _check_all_rows(wl, logits, b, wt, ids, f"{wl.name} M={wl.M} one kernel")
    # properties on every row
    assert np.all((ids >= 0) & (ids < wl.E))
    srt = np.sort(ids, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1])                        # distinct experts
    groups = ids // (wl.E // wl.G)
    assert max(len(set(r)) for r in groups.tolist()) <= wl.TG       # within TG groups
    np.testing.assert_allclose(wt.astype(np.float64).sum(1), 1.0, atol=1e-5)
    assert np.all(wt > 0)


def test_fused_router_deterministic():
    rng = np.random.default_rng(9)
    hidden, w, b = _inputs(rng, 300, 448)
    a = _run(hidden, w, b, 8, 8, 4, True, "sigmoid", "top2sum")
    c = _run(hidden, w, b, 8, 8, 4, True, "sigmoid", "top2sum")
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_fused_router_rejects_outside_range():
    x = torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((100, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="compiled range"):
        mr.route_fused_router(x, wr, 8, 8, 4, True)      # H % 64 != 0
