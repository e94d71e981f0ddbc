"""route_dispatch_metadata_noalloc (no workspace argument, a static device
buffer instead) against route_dispatch_metadata with a caller workspace:
bit-identical outputs on two calls in a row, the second smaller, through
the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import moe_expert_routing_amd as mr

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _outputs(M, K, E, with_w, dev):
    n = M * K
    return (torch.full((E,), -7, dtype=torch.int32, device=dev),
            torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
            torch.full((n,), -7, dtype=torch.int32, device=dev),
            torch.full((n,), -7, dtype=torch.int32, device=dev),
            torch.full((n,), -7.0, dtype=torch.float32, device=dev) if with_w else None)


def _noalloc(ids, w, E, outs, stream):
    M, K = ids.shape
    c, o, g, s, sw = outs
    return mr.lib().route_dispatch_metadata_noalloc(_p(ids), _p(w), M, K, E, _p(c), _p(o), _p(g),
                                                    _p(s), _p(sw), stream)


def _with_workspace(ids, w, E, outs, stream):
    M, K = ids.shape
    c, o, g, s, sw = outs
    ws = torch.empty(max(mr.route_dispatch_workspace_size(M, K, E), 4), dtype=torch.uint8,
                     device=ids.device)
    return mr.lib().route_dispatch_metadata(_p(ids), _p(w), M, K, E, _p(c), _p(o), _p(g), _p(s),
                                            _p(sw), _p(ws), ws.numel(), stream)


@pytest.mark.parametrize("first,second", [
    ((65536, 8, 256, True), (4099, 8, 256, True)),     # the routing output size, then ragged
    ((20000, 6, 1024, False), (777, 2, 1024, False)),  # the largest expert count, no weights
    ((3000, 9, 258, True), (1, 9, 258, True)),         # shared slot ids, then a single token
])
def test_noalloc_matches_workspace_entry_point(first, second):
    dev = torch.device("cuda", 0)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rng = np.random.default_rng(first[0] + second[0])
    for M, K, E, with_w in (first, second):
        print(f"[gpu] route_dispatch_metadata_noalloc M={M} K={K} E={E} weights={with_w}",
              flush=True)
        ids_np = rng.integers(-1, E + 1, size=(M, K)).astype(np.int32)  # a few dropped ids
        ids = torch.from_numpy(ids_np).to(dev)
        w = torch.from_numpy(rng.random((M, K), dtype=np.float32)).to(dev) if with_w else None
        a = _outputs(M, K, E, with_w, dev)
        b = _outputs(M, K, E, with_w, dev)
        assert _noalloc(ids, w, E, a, stream) == mr.ROUTE_OK
        assert _with_workspace(ids, w, E, b, stream) == mr.ROUTE_OK
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            if x is not None:
                assert torch.equal(x, y)
