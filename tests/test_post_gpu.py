"""GPU parity of the post-routing steps against the oracle: the shared-expert
slot, the ascending id order, the bias rounded to the logit dtype, and the
whole chain route -> shared slot -> dispatch metadata."""
import numpy as np
import pytest
import torch

import moe_expert_routing_amd as mr
import oracle
from gpu_util import log, to_device
from parity_check import compare
from workloads import WORKLOADS, bf16_bits_from_f32, bf16_bits_to_f32, make_bias, make_logits

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


def test_bias_rounded_to_logit_dtype():
    """The aiter-style call casts the correction bias to the logits' dtype; a
    bf16-rounded bias passed as float32 is the same numbers."""
    wl = WORKLOADS["biased_grouped_e256"]
    x = make_logits(wl, 8192)
    b = bf16_bits_to_f32(bf16_bits_from_f32(make_bias(wl)))
    log("[gpu] biased grouped top-k with a bf16-rounded bias")
    w, ids = mr.route_biased_grouped_topk(to_device(x), to_device(b), 8, 8, 4, True)
    torch.cuda.synchronize()
    rep = compare(x, w.cpu().numpy(), ids.cpu().numpy(), scoring=oracle.SIGMOID, bias=b, G=8,
                  TG=4, rule=oracle.GROUP_TOP2SUM, K=8, renorm=True)
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
