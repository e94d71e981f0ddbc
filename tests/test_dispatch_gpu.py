"""GPU parity of route_dispatch_metadata (expert-sorted dispatch metadata)
against the oracle's stable counting sort: integer outputs bit-exact, sorted
weights exact copies."""
import numpy as np
import pytest
import torch

import moe_expert_routing_amd as mr
import oracle
from gpu_util import log, to_device
from workloads import WORKLOADS, make_bias, make_logits

pytestmark = pytest.mark.gpu


def _compare(ids_np, E, w_np=None, workspace=None):
    ids_t = torch.from_numpy(np.ascontiguousarray(ids_np, np.int32)).cuda()
    w_t = None if w_np is None else torch.from_numpy(np.ascontiguousarray(w_np)).cuda()
    c, o, g, s, sw = mr.route_dispatch_metadata(ids_t, E, w_t, workspace=workspace)
    torch.cuda.synchronize()
    rc, ro, rg, rs, rsw = oracle.dispatch(ids_np, E, w_np)
    np.testing.assert_array_equal(c.cpu().numpy(), rc)
    np.testing.assert_array_equal(o.cpu().numpy(), ro)
    np.testing.assert_array_equal(g.cpu().numpy(), rg)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    if w_np is not None:
        np.testing.assert_array_equal(sw.cpu().numpy(), rsw)
    return c, o, g, s, sw


@pytest.mark.parametrize("M,K,E,lo,hi,seed", [
    (1, 1, 1, 0, 1, 0),          # a single assignment
    (3, 2, 4, -1, 6, 1),         # dropped ids on both sides
    (37, 3, 8, 0, 8, 2),         # fewer than one 64-lane step
    (1000, 6, 160, -3, 170, 3),  # ragged chunks, some dropped
    (4096, 8, 256, 0, 256, 4),   # whole 512-assignment chunks
    (513, 1, 1024, -5, 1024, 5), # widest expert id (11 bits)
    (20000, 2, 1, -1, 1, 6),     # one expert, half the ids dropped
    (70001, 8, 256, -2, 258, 7), # 274 blocks: the scan reads its columns in two batches
    (98000, 8, 160, 0, 160, 8),  # two kernels: 96 coarse rows, every reducing thread's last
    (40000, 8, 384, -1, 385, 10),  # two kernels: 40 coarse rows over 5 reducing groups
    (65536, 8, 252, 0, 252, 11), # two kernels: 64 coarse rows of 63 quads (not a power of 2)
    (20000, 8, 1024, -3, 1030, 12),  # three kernels at the widest expert range (79 blocks)
    (2304, 8, 256, -1, 256, 15),  # two kernels: the last coarse row holds one place block
    (2305, 8, 256, 0, 256, 16),   # two kernels: the last coarse row holds two, the second ragged
    (65536, 8, 250, -2, 252, 17), # three kernels: E not a multiple of 4
])
def test_dispatch_random_ids(M, K, E, lo, hi, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(lo, hi, size=(M, K)).astype(np.int32)
    w = rng.random((M, K), dtype=np.float32)
    log(f"[gpu] dispatch random M={M} K={K} E={E} ids in [{lo},{hi})")
    _compare(ids, E, w)
    _compare(ids, E)  # without weights


def test_dispatch_of_full_size_routing_output():
    """Route the 65536-token biased grouped workload on the GPU, then dispatch
    its ids; the oracle sorts the same ids."""
    wl = WORKLOADS["biased_grouped_e256"]
    x, b = make_logits(wl), make_bias(wl)
    log("[gpu] dispatch of route_biased_grouped_topk output, M=65536 E=256 K=8")
    w, ids = mr.route_biased_grouped_topk(to_device(x), to_device(b), wl.K, wl.G, wl.TG, True)
    torch.cuda.synchronize()
    c, o, g, s, sw = _compare(ids.cpu().numpy(), wl.E, w.cpu().numpy())
    assert int(c.sum()) == 65536 * 8


def test_dispatch_skewed_experts():
    """A few experts take most assignments (Zipf-like ranks), so a block's
    runs range from hundreds of entries to none, on both launch paths."""
    rng = np.random.default_rng(13)
    for M, E in ((65536, 256), (30000, 1024)):
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        ids = rng.choice(E, size=(M, 8), p=p / p.sum()).astype(np.int32)
        w = rng.random((M, 8), dtype=np.float32)
        log(f"[gpu] dispatch skewed ids M={M} E={E}")
        _compare(ids, E, w)


def test_dispatch_all_to_one_expert():
    """One expert takes every assignment: one run across every chunk."""
    ids = np.full((8192, 8), 5, np.int32)
    log("[gpu] dispatch all ids = 5")
    _compare(ids, 256, np.arange(8192 * 8, dtype=np.float32).reshape(8192, 8))


def test_dispatch_into_given_outputs():
    """Outputs passed in are filled and returned; they match a call that
    allocates its own."""
    rng = np.random.default_rng(14)
    M, K, E = 3000, 8, 256
    ids = torch.from_numpy(rng.integers(-1, E, size=(M, K)).astype(np.int32)).cuda()
    w = torch.from_numpy(rng.random((M, K), dtype=np.float32)).cuda()
    out = (torch.full((E,), 7, dtype=torch.int32, device="cuda"),
           torch.full((E + 1,), 7, dtype=torch.int32, device="cuda"),
           torch.full((M * K,), 7, dtype=torch.int32, device="cuda"),
           torch.full((M * K,), 7, dtype=torch.int32, device="cuda"),
           torch.full((M * K,), 7.0, dtype=torch.float32, device="cuda"))
    log("[gpu] dispatch into given outputs M=3000 K=8 E=256")
    got = mr.route_dispatch_metadata(ids, E, w, out=out)
    ref = mr.route_dispatch_metadata(ids, E, w)
    torch.cuda.synchronize()
    for g, o, r in zip(got, out, ref):
        assert g is o and torch.equal(g, r)
    with pytest.raises(ValueError):
        mr.route_dispatch_metadata(ids, E, w, out=out[:4] + (None,))
    with pytest.raises(ValueError):
        mr.route_dispatch_metadata(ids, E, w, out=(out[0][:-1],) + out[1:])


def test_dispatch_empty():
    ids = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    c, o, g, s, sw = mr.route_dispatch_metadata(ids, 16)
    torch.cuda.synchronize()
    assert (c.cpu() == 0).all() and (o.cpu() == 0).all() and g.numel() == 0


def test_dispatch_reuses_workspace_and_is_deterministic():
    rng = np.random.default_rng(9)
    ws = torch.empty(mr.route_dispatch_workspace_size(5000, 8, 256), dtype=torch.uint8,
                     device="cuda")
    big = rng.integers(0, 256, size=(5000, 8)).astype(np.int32)
    small = rng.integers(0, 256, size=(700, 8)).astype(np.int32)
    log("[gpu] dispatch workspace reuse")
    a = _compare(big, 256, workspace=ws)
    _compare(small, 256, workspace=ws)
    b = _compare(big, 256, workspace=ws)
    for x, y in zip(a[:4], b[:4]):
        assert torch.equal(x, y)


def test_dispatch_rejects_small_workspace():
    ids = torch.zeros((100, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        mr.route_dispatch_metadata(ids, 256, workspace=torch.empty(16, dtype=torch.uint8,
                                                                   device="cuda"))
