"""GPU parity of the post-routing steps against the oracle: the shared-expert
slot, the ascending id order, the correction bias in bf16 (the logits' dtype,
as the aiter-style call passes it), and the whole chain route -> shared slot
-> dispatch metadata."""
import numpy as np
import pytest
import torch

import moe_expert_routing_amd as mr
import oracle
from gpu_util import log, to_device
from parity_check import compare
from workloads import (WORKLOADS, bf16_bits_from_f32, bf16_bits_to_f32, make_bias, make_logits,
                       random_logits)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,rsf", [(4096, 9, 2.5), (77, 9, None), (1, 2, 1.0), (1000, 13, 0.3),
                                     (300, 4, 2.5), (1000, 8, 1.0), (200, 20, 2.5), (65, 33, None),
                                     (40, 64, 0.5)])  # every row width: 2 .. 64 lanes
def test_fuse_shared_expert(M, K, rsf):
    wl = WORKLOADS["biased_grouped_e256"]
    x, b = make_logits(wl, M), make_bias(wl)
    w, ids = mr.route_biased_grouped_topk(to_device(x), to_device(b), K, 8, 4, True)
    torch.cuda.synchronize()
    w0, i0 = w.cpu().numpy(), ids.cpu().numpy()
    sid = np.random.default_rng(M).integers(256, 258, size=M).astype(np.int32)
    log(f"[gpu] shared-expert slot M={M} K={K} rsf={rsf}")
    mr.route_fuse_shared_expert(w, ids, torch.from_numpy(sid).cuda(), rsf)
    torch.cuda.synchronize()
    rw, ri = oracle.fuse_shared_expert(w0, i0, sid, rsf)
    np.testing.assert_array_equal(ids.cpu().numpy(), ri)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=0, atol=1e-6)


@pytest.mark.parametrize("M,K,hi", [(5000, 8, 256), (333, 2, 4), (1000, 13, 30), (64, 16, 10),
                                    (100, 17, 50), (257, 40, 30), (31, 64, 1000), (700, 3, 5),
                                    (99, 4, 3)])
def test_sort_ids(M, K, hi):
    rng = np.random.default_rng(K)
    i0 = rng.integers(0, hi, size=(M, K)).astype(np.int32)   # repeats: stable by slot
    w0 = rng.random((M, K), dtype=np.float32)
    w, ids = torch.from_numpy(w0).cuda(), torch.from_numpy(i0).cuda()
    log(f"[gpu] ascending ids M={M} K={K}")
    mr.route_sort_ids(w, ids)
    torch.cuda.synchronize()
    rw, ri = oracle.sort_ids(w0, i0)
    np.testing.assert_array_equal(ids.cpu().numpy(), ri)
    np.testing.assert_array_equal(w.cpu().numpy(), rw)


def _bf16_bias_tensor(bits, offset):
    """bf16 bias tensor on the device; offset 1 starts it one element into a
    larger allocation (2-byte aligned only)."""
    t = torch.from_numpy(np.concatenate([np.zeros(offset, np.uint16), bits]).view(np.int16))
    return t.view(torch.bfloat16).cuda()[offset:]


def _f32_bias_tensor(b, offset):
    """float32 bias tensor on the device; offset 1 starts it one element into
    a larger allocation (4-byte aligned only)."""
    return torch.from_numpy(np.concatenate([np.zeros(offset, np.float32), b])).cuda()[offset:]


@pytest.mark.parametrize("M,E,K,G,TG,dtype,offset", [
    (65536, 256, 8, 8, 4, "bf16", 0),   # the DeepSeek-V3 shape, 65536 tokens
    (4096, 256, 8, 1, 1, "bf16", 0),    # the aiter call's ungrouped shape
    (1000, 256, 8, 8, 4, "f32", 0),     # fp32 logits, bf16 bias (one row per wave)
    (3000, 256, 8, 8, 4, "f32", 0),     # fp32 logits, bf16 bias (8-row kernel)
    (1000, 256, 8, 1, 1, "bf16", 0),    # ungrouped, one row per wave
    (1000, 256, 8, 8, 4, "bf16", 1),    # bias 2-byte aligned only: the generic kernel
    (300, 384, 8, 8, 4, "bf16", 0),     # the generic kernel
    (1000, 8, 2, 1, 1, "f32", 0),       # one lane per row (8 experts)
])
def test_bf16_correction_bias(M, E, K, G, TG, dtype, offset):
    """The aiter-style call casts correction_bias to the logits' dtype and
    passes that tensor; the library takes it as bf16 and widens it exactly,
    so the result equals the oracle's on the widened values and is
    bit-identical to passing those values as float32 to the same kernel (a
    misaligned bias, bf16 or float32, takes the generic kernel)."""
    rng = np.random.default_rng(M + E + offset)
    if dtype == "bf16" and E == 256:
        wl = WORKLOADS["biased_grouped_e256"]
        x = make_logits(wl, M)
        bias_f32 = make_bias(wl)
    else:
        x = random_logits(rng, M, E, dtype, std=1.5)
        bias_f32 = (rng.standard_normal(E) * 0.1).astype(np.float32)
    bits = bf16_bits_from_f32(bias_f32)
    b = bf16_bits_to_f32(bits)                     # the exact values of the bf16 bias
    bd = _bf16_bias_tensor(bits, offset)
    assert bd.dtype == torch.bfloat16 and (bd.data_ptr() % 8 != 0) == bool(offset)
    log(f"[gpu] bf16 correction bias M={M} E={E} K={K} G={G} TG={TG} logits={dtype} "
        f"offset={offset}")
    xd = to_device(x)
    w, ids = mr.route_biased_grouped_topk(xd, bd, K, G, TG, True)
    w2, ids2 = mr.route_biased_grouped_topk(xd, _f32_bias_tensor(b, offset), K, G, TG, True)
    torch.cuda.synchronize()
    assert torch.equal(w, w2) and torch.equal(ids, ids2)
    rep = compare(x, w.cpu().numpy(), ids.cpu().numpy(), scoring=oracle.SIGMOID, bias=b, G=G,
                  TG=TG, rule=oracle.GROUP_TOP2SUM, K=K, renorm=True,
                  label=f"bf16 bias M={M} E={E} G={G} logits={dtype} offset={offset}")
    log(f"[gpu]   {rep.summary()}")
    assert rep.ok(), rep.summary()


@pytest.mark.parametrize("M,H,E,K,G,TG,workspace,offset", [
    (130, 512, 256, 8, 8, 4, False, 0),    # one fused kernel
    (130, 2048, 256, 8, 8, 4, None, 0),    # split path: a block per row, row routed by one wave
    (130, 2048, 256, 8, 8, 4, None, 1),    # the same, bias 2-byte aligned: the 8-lane epilogue
    (3000, 640, 256, 8, 8, 4, None, 0),    # split path: a wave per 8 rows
    (300, 2048, 16, 4, 1, 1, None, 0),     # 16 experts
])
def test_bf16_correction_bias_fused_router(M, H, E, K, G, TG, workspace, offset):
    """A bf16 correction bias on every fused-router path (a misaligned one
    takes the epilogue that loads it entry by entry and gives the same
    bits)."""
    rng = np.random.default_rng(M * 3 + H + E)
    hidden = bf16_bits_from_f32(rng.standard_normal((M, H), dtype=np.float32))
    wr = bf16_bits_from_f32(rng.standard_normal((H, E), dtype=np.float32) *
                            np.float32(H ** -0.5))
    bits = bf16_bits_from_f32((rng.standard_normal(E) * 0.1).astype(np.float32))
    b = bf16_bits_to_f32(bits)
    log(f"[gpu] bf16 correction bias, fused router M={M} H={H} E={E} "
        f"{'one kernel' if workspace is False else 'default'}")
    hd, wd = to_device(hidden), to_device(wr)
    w, ids = mr.route_fused_router(hd, wd, K, G, TG, True, "sigmoid",
                                   _bf16_bias_tensor(bits, offset), "top2sum",
                                   workspace=workspace)
    w2, ids2 = mr.route_fused_router(hd, wd, K, G, TG, True, "sigmoid",
                                     _f32_bias_tensor(b, offset), "top2sum", workspace=workspace)
    torch.cuda.synchronize()
    assert torch.equal(w, w2) and torch.equal(ids, ids2)
    if offset:
        w3, ids3 = mr.route_fused_router(hd, wd, K, G, TG, True, "sigmoid", to_device(b),
                                         "top2sum", workspace=workspace)
        torch.cuda.synchronize()
        assert torch.equal(w, w3) and torch.equal(ids, ids3)
    logits = oracle.router_logits(hidden, wr)
    rep = compare(logits, w.cpu().numpy(), ids.cpu().numpy(), scoring=oracle.SIGMOID, bias=b,
                  G=G, TG=TG, rule=oracle.GROUP_TOP2SUM, K=K, renorm=True)
    log(f"[gpu]   {rep.summary()}")
    assert rep.ok(), rep.summary()


def test_route_shared_slot_then_dispatch():
    """DeepSeek-V3-like chain: 8 routed experts + 1 shared slot (ids 256, 257)
    per token, then dispatch metadata over 258 experts."""
    wl = WORKLOADS["biased_grouped_e256"]
    M = 16384
    x, b = make_logits(wl, M), make_bias(wl)
    w, ids = mr.route_biased_grouped_topk(to_device(x), to_device(b), 9, 8, 4, True)
    sid = np.random.default_rng(3).integers(256, 258, size=M).astype(np.int32)
    mr.route_fuse_shared_expert(w, ids, torch.from_numpy(sid).cuda(), 2.5)
    c, o, g, s, sw = mr.route_dispatch_metadata(ids, 258, w)
    torch.cuda.synchronize()
    log("[gpu] route -> shared slot -> dispatch, M=16384")
    rc, ro, rg, rs, rsw = oracle.dispatch(ids.cpu().numpy(), 258, w.cpu().numpy())
    np.testing.assert_array_equal(c.cpu().numpy(), rc)
    np.testing.assert_array_equal(g.cpu().numpy(), rg)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(sw.cpu().numpy(), rsw)
    assert int(c[256:].sum()) == M            # every token has one shared slot
