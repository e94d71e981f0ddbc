"""GPU parity of route_fused_router with 8 or 16 experts against the
oracle's exact double logits: the MFMA kernel (hidden_dim <= 8192) and the
vector-ALU kernel (larger hidden_dim), optional soft-cap, per-token top-k."""
import numpy as np
import pytest
import torch

import moe_expert_routing_amd as mr
import oracle
from gpu_util import log, oracle_router_logits, to_device
from parity_check import compare
from workloads import WORKLOADS, bf16_bits_from_f32, make_router_inputs

pytestmark = pytest.mark.gpu

SC = {"sigmoid": oracle.SIGMOID, "softmax": oracle.SOFTMAX}


def _inputs(rng, M, H, E, scale=1.0, bias=False):
    hidden = bf16_bits_from_f32(rng.standard_normal((M, H), dtype=np.float32) *
                                np.float32(scale))
    w = bf16_bits_from_f32(rng.standard_normal((H, E), dtype=np.float32) * np.float32(H ** -0.5))
    b = (rng.standard_normal(E, dtype=np.float32) * np.float32(0.1)) if bias else None
    return hidden, w, b


def _run_check(hidden, w, b, E, K, scoring, renorm, cap, label=None, workspace=None):
    wt, ids = mr.route_fused_router(to_device(hidden), to_device(w), K, 1, 1, renorm, scoring,
                                    None if b is None else to_device(b), "max",
                                    logit_softcap=cap, workspace=workspace)
    torch.cuda.synchronize()
    wt, ids = wt.cpu().numpy(), ids.cpu().numpy()
    logits = oracle_router_logits(hidden, w)
    if cap:
        logits = oracle.softcap(logits, cap)
    rep = compare(logits, wt, ids, scoring=SC[scoring], bias=b, G=1, TG=1,
                  rule=oracle.GROUP_MAX, K=K, renorm=renorm, label=label)
    log(f"[gpu]   {rep.summary()}")
    assert rep.ok(), rep.summary()
    return wt, ids


@pytest.mark.parametrize("M,H,E,K,scoring,bias,renorm,cap,scale", [
    (1, 4096, 8, 2, "softmax", False, False, 0.0, 1.0),     # one token
    (37, 4096, 8, 2, "softmax", False, True, 30.0, 1.0),    # ragged block of 8 tokens
    (100, 4104, 8, 1, "softmax", False, False, 5.0, 3.0),   # H past a 512 chunk; top-1
    (64, 8, 8, 2, "softmax", False, False, 0.0, 1.0),       # H = 8: one lane's units
    (300, 2048, 8, 8, "sigmoid", True, True, 0.0, 1.0),     # sigmoid + bias, K = E
    (50, 6144, 16, 4, "softmax", False, True, 0.0, 1.0),    # 16 experts
    (19, 1000, 16, 2, "sigmoid", False, False, 2.0, 3.0),   # 16 experts, saturating cap
    (256, 512, 16, 16, "softmax", False, False, 0.0, 1.0),  # K = E = 16
    (4000, 7168, 16, 2, "softmax", False, True, 0.0, 1.0),  # LDS ring: 250 tiles, 7 chunks
    (4100, 1000, 8, 2, "softmax", False, False, 5.0, 3.0),  # 8 experts on MFMA, ragged H
    # MFMA kernel, every batch count (4 fragments of 32 units a batch, 8 waves)
    (70, 1056, 16, 2, "softmax", False, True, 0.0, 1.0),    # 2 batches
    (70, 2080, 16, 4, "sigmoid", True, True, 0.0, 1.0),     # 3 batches
    (70, 4128, 16, 2, "softmax", False, False, 30.0, 1.0),  # 5 batches
    (70, 8192, 16, 4, "softmax", False, True, 0.0, 1.0),    # LDS ring: 8 chunks
    (70, 3072, 16, 4, "sigmoid", True, True, 0.0, 1.0),     # LDS ring: 3 chunks, bias
    (4100, 2048, 8, 2, "sigmoid", True, True, 0.0, 1.0),    # LDS ring, 8 experts, ragged tile
    (4096, 1024, 8, 1, "softmax", False, False, 30.0, 1.0), # LDS ring, one chunk, cap
    (1500, 3072, 8, 2, "softmax", False, True, 5.0, 1.0),   # LDS ring, 8 experts from 1024 tokens
    (20000, 2048, 8, 2, "softmax", False, True, 0.0, 1.0),  # LDS ring, ~5 tiles a block
    (9001, 1024, 16, 4, "sigmoid", True, True, 0.0, 1.0),   # LDS ring, 3 tiles a block, ragged
    (1, 2048, 16, 4, "sigmoid", True, True, 0.0, 1.0),      # LDS ring, a single token
    (1000, 4096, 16, 4, "sigmoid", True, False, 0.0, 3.0),  # LDS ring, 4 chunks, wide logits
    (70, 8000, 16, 2, "sigmoid", False, True, 0.0, 1.0),    # 8 batches, ragged H
    (33, 9000, 8, 2, "softmax", False, False, 30.0, 1.0),   # H > 8192: vector-ALU kernel
    (20, 8704, 16, 3, "sigmoid", True, True, 0.0, 1.0),     # H > 8192, 16 experts
])
def test_small_router(M, H, E, K, scoring, bias, renorm, cap, scale):
    rng = np.random.default_rng(M * 31 + H + E)
    hidden, w, b = _inputs(rng, M, H, E, scale, bias)
    log(f"[gpu] route_fused_router E={E} M={M} H={H} K={K} {scoring} bias={bias} cap={cap}")
    _run_check(hidden, w, b, E, K, scoring, renorm, cap)


@pytest.mark.parametrize("name", ["fused_router_e8_h4096", "fused_router_e16_h6144"])
def test_small_router_workload(name):
    """The full 8192-token workload, every row against the oracle."""
    wl = WORKLOADS[name]
    hidden, w = make_router_inputs(wl)
    log(f"[gpu] route_fused_router workload={wl.name} M={wl.M} H={wl.hidden_dim}")
    wt, ids = _run_check(hidden, w, None, wl.E, wl.K, wl.scoring, wl.renormalize, wl.softcap,
                         label=f"{wl.name} M={wl.M}")
    # every row: distinct ids in range, softmax weights in (0, 1], descending
    srt = np.sort(ids, axis=1)
    assert np.all((ids >= 0) & (ids < wl.E)) and np.all(srt[:, 1:] != srt[:, :-1])
    assert np.all((wt > 0) & (wt <= 1)) and np.all(wt[:, :-1] >= wt[:, 1:])
    if wl.renormalize:
        np.testing.assert_allclose(wt.astype(np.float64).sum(1), 1.0, atol=1e-5)


def test_small_router_ignores_a_workspace():
    """8 or 16 experts use no workspace; one passed anyway is accepted and
    changes nothing."""
    rng = np.random.default_rng(23)
    hidden, w, _ = _inputs(rng, 64, 4096, 8)
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    log("[gpu] route_fused_router E=8 M=64 H=4096 with a 64 KiB workspace")
    a = _run_check(hidden, w, None, 8, 2, "softmax", False, 30.0, workspace=ws)
    c = _run_check(hidden, w, None, 8, 2, "softmax", False, 30.0, workspace=False)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_small_router_deterministic():
    rng = np.random.default_rng(17)
    hidden, w, _ = _inputs(rng, 77, 3072, 8)
    x, wr = to_device(hidden), to_device(w)
    a = mr.route_fused_router(x, wr, 2, 1, 1, False, "softmax", None, "max")
    c = mr.route_fused_router(x, wr, 2, 1, 1, False, "softmax", None, "max")
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])


def test_small_router_rejects_outside_range():
    x = torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda")
    for E in (8, 12):                               # H % 8 != 0; 12 experts
        wr = torch.zeros((100, E), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(ValueError, match="compiled range"):
            mr.route_fused_router(x, wr, 2, 1, 1)
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((64, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="compiled range"):
        mr.route_fused_router(x, wr, 2, 2, 1)      # expert groups
