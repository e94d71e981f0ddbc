"""C-ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import moe_expert_routing_amd as mr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")

# Fake, suitably aligned device addresses: validation never dereferences them.
# Every call below is rejected, or has num_tokens == 0, so none reaches a HIP
# call; never add a call here with valid arguments and num_tokens > 0.
P = ctypes.c_void_p(0x10000)
Q = ctypes.c_void_p(0x20000)
R = ctypes.c_void_p(0x30000)
NULL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(route_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_exported_set():
    assert declared_functions() == sorted(mr.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = mr.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    assert mr.status_str(mr.ROUTE_OK) == "ROUTE_OK"
    assert "invalid" in mr.status_str(mr.ROUTE_EINVAL)
    assert "compiled range" in mr.status_str(mr.ROUTE_ENOTSUP)
    assert "launch" in mr.status_str(mr.ROUTE_ELAUNCH)
    assert mr.status_str(99).startswith("unknown")


F = mr.ROUTE_F32


def bgt(M=4, E=256, K=8, G=8, TG=4, logits=P, dtype=mr.ROUTE_BF16, bias=R, bias_dtype=F, w=Q,
        ids=R):
    return mr.lib().route_biased_grouped_topk(logits, dtype, bias, bias_dtype, M, E, K, G, TG, 1,
                                              w, ids, None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), mr.ROUTE_EINVAL),
    (dict(E=0), mr.ROUTE_EINVAL),
    (dict(K=0), mr.ROUTE_EINVAL),
    (dict(G=3), mr.ROUTE_EINVAL),                 # 256 % 3 != 0
    (dict(TG=0), mr.ROUTE_EINVAL),
    (dict(TG=9), mr.ROUTE_EINVAL),                # TG > G
    (dict(K=129), mr.ROUTE_EINVAL),               # K > TG * E/G = 128
    (dict(E=8, G=8, TG=4, K=2), mr.ROUTE_EINVAL),  # top-2 sum needs 2 experts per group
    (dict(logits=NULL), mr.ROUTE_EINVAL),
    (dict(w=NULL), mr.ROUTE_EINVAL),
    (dict(ids=NULL), mr.ROUTE_EINVAL),
    (dict(logits=ctypes.c_void_p(0x10001)), mr.ROUTE_EINVAL),  # misaligned bf16
    (dict(w=ctypes.c_void_p(0x20002)), mr.ROUTE_EINVAL),
    (dict(bias=ctypes.c_void_p(0x30001)), mr.ROUTE_EINVAL),
    (dict(bias=ctypes.c_void_p(0x30002)), mr.ROUTE_EINVAL),   # fp32 bias needs 4 bytes
    (dict(bias=ctypes.c_void_p(0x30001), bias_dtype=mr.ROUTE_BF16), mr.ROUTE_EINVAL),
    (dict(bias_dtype=7), mr.ROUTE_EINVAL),                    # unknown bias dtype
    (dict(bias=NULL, bias_dtype=-1), mr.ROUTE_EINVAL),        # ... also with no bias
    (dict(M=0, bias_dtype=7), mr.ROUTE_EINVAL),
    (dict(dtype=7), mr.ROUTE_EINVAL),
    (dict(E=2048, G=8, TG=4, K=8), mr.ROUTE_ENOTSUP),          # E beyond 1024
    (dict(E=256, G=1, TG=1, K=65), mr.ROUTE_ENOTSUP),          # K beyond 64
    (dict(E=256, G=128, TG=4, K=8), mr.ROUTE_ENOTSUP),         # G beyond 64
    (dict(M=0, logits=NULL, w=NULL, ids=NULL), mr.ROUTE_OK),   # empty: no launch
])
def test_biased_grouped_validation(kw, code):
    assert bgt(**kw) == code


def test_softmax_and_grouped_validation():
    L = mr.lib()
    assert L.route_topk_softmax(P, mr.ROUTE_F32, 10, 8, 9, 1, Q, R, None) == mr.ROUTE_EINVAL
    assert L.route_topk_softmax(P, mr.ROUTE_F32, 0, 8, 2, 1, Q, R, None) == mr.ROUTE_OK
    assert L.route_topk_softmax(NULL, mr.ROUTE_F32, 0, 8, 2, 1, NULL, NULL, None) == mr.ROUTE_OK
    assert L.route_topk_softmax(ctypes.c_void_p(0x10002), mr.ROUTE_F32, 5, 8, 2, 1, Q, R,
                                None) == mr.ROUTE_EINVAL
    # scoring enum
    assert L.route_grouped_topk(P, mr.ROUTE_F32, 5, 160, 6, 8, 3, 0, 5, Q, R, None) == \
        mr.ROUTE_EINVAL
    # grouped with the max rule accepts groups of one expert
    assert L.route_grouped_topk(P, mr.ROUTE_F32, 0, 8, 2, 8, 4, 0, mr.ROUTE_SOFTMAX, Q, R,
                                None) == mr.ROUTE_OK
    assert L.route_grouped_topk(P, mr.ROUTE_F32, 5, 160, 61, 8, 3, 0, mr.ROUTE_SOFTMAX, Q, R,
                                None) == mr.ROUTE_EINVAL


def test_fused_router_validation():
    L = mr.lib()
    f = L.route_fused_router
    sig, top2 = mr.ROUTE_SIGMOID, mr.ROUTE_GROUP_TOP2_SUM
    assert f(P, Q, 8, 0, 256, sig, R, F, top2, 8, 8, 4, 1, 0.0, Q, R, NULL, 0, None) == mr.ROUTE_EINVAL
    assert f(P, NULL, 8, 7168, 256, sig, R, F, top2, 8, 8, 4, 1, 0.0, Q, R, NULL, 0, None) == mr.ROUTE_EINVAL
    assert f(P, Q, 8, 7168, 256, 4, R, F, top2, 8, 8, 4, 1, 0.0, Q, R, NULL, 0, None) == mr.ROUTE_EINVAL
    assert f(P, Q, 8, 7168, 256, sig, R, F, 9, 8, 8, 4, 1, 0.0, Q, R, NULL, 0, None) == mr.ROUTE_EINVAL
    assert f(P, Q, 8, 7168, 256, sig, R, F, top2, 200, 8, 4, 1, 0.0, Q, R, NULL, 0, None) == mr.ROUTE_EINVAL
    # outside the compiled range
    assert f(P, Q, 8, 7168, 128, sig, R, F, top2, 8, 8, 4, 1, 0.0, Q, R, NULL, 0, None) == mr.ROUTE_ENOTSUP
    assert f(P, Q, 8, 7000, 256, sig, R, F, top2, 8, 8, 4, 1, 0.0, Q, R, NULL, 0, None) == mr.ROUTE_ENOTSUP
    assert f(NULL, NULL, 0, 7168, 256, sig, NULL, F, top2, 8, 8, 4, 1, 0.0, NULL, NULL, NULL, 0, None) == \
        mr.ROUTE_OK
    # an unknown bias dtype, with or without a bias
    assert f(P, Q, 8, 7168, 256, sig, R, 5, top2, 8, 8, 4, 1, 0.0, Q, R, NULL, 0, None) == \
        mr.ROUTE_EINVAL
    assert f(P, Q, 8, 7168, 256, sig, NULL, -1, top2, 8, 8, 4, 1, 0.0, Q, R, NULL, 0, None) == \
        mr.ROUTE_EINVAL
    # a bf16 bias needs 2-byte alignment, an fp32 one 4
    assert f(P, Q, 8, 7168, 256, sig, ctypes.c_void_p(0x30001), mr.ROUTE_BF16, top2, 8, 8, 4, 1,
             0.0, Q, R, NULL, 0, None) == mr.ROUTE_EINVAL
    assert f(P, Q, 8, 7168, 256, sig, ctypes.c_void_p(0x30002), F, top2, 8, 8, 4, 1, 0.0, Q, R,
             NULL, 0, None) == mr.ROUTE_EINVAL
    # NaN or infinite caps
    for cap in (float("nan"), float("inf"), -float("inf")):
        assert f(P, Q, 8, 7168, 256, sig, R, F, top2, 8, 8, 4, 1, cap, Q, R, NULL, 0, None) == \
            mr.ROUTE_EINVAL
    # workspace: a size without a pointer, a misaligned one, one too small
    need = L.route_fused_router_workspace_size(8, 7168, 256)
    assert need > 0
    W = ctypes.c_void_p(0x40000)
    assert f(P, Q, 8, 7168, 256, sig, R, F, top2, 8, 8, 4, 1, 0.0, Q, R, NULL, need, None) == \
        mr.ROUTE_EINVAL
    assert f(P, Q, 8, 7168, 256, sig, R, F, top2, 8, 8, 4, 1, 0.0, Q, R, ctypes.c_void_p(0x40008),
             need, None) == mr.ROUTE_EINVAL
    assert f(P, Q, 8, 7168, 256, sig, R, F, top2, 8, 8, 4, 1, 0.0, Q, R, W, need - 4, None) == \
        mr.ROUTE_EINVAL


def test_fused_router_few_experts_range():
    """8 or 16 experts go to the vector-ALU router: H a multiple of 8, no
    expert groups; other expert counts below 256 are outside the range."""
    f = mr.lib().route_fused_router
    sm, top2, mx = mr.ROUTE_SOFTMAX, mr.ROUTE_GROUP_TOP2_SUM, mr.ROUTE_GROUP_MAX
    ok = mr.ROUTE_OK
    assert f(NULL, NULL, 0, 4096, 8, sm, NULL, F, mx, 2, 1, 1, 0, 30.0, NULL, NULL, NULL, 0,
             None) == ok
    assert f(NULL, NULL, 0, 4096, 16, sm, NULL, F, mx, 2, 1, 1, 0, 0.0, NULL, NULL, NULL, 0,
             None) == ok
    assert f(P, Q, 8, 4100, 8, sm, NULL, F, mx, 2, 1, 1, 0, 0.0, Q, R, NULL, 0, None) == \
        mr.ROUTE_ENOTSUP                                  # H % 8 != 0
    assert f(P, Q, 8, 4096, 12, sm, NULL, F, mx, 2, 1, 1, 0, 0.0, Q, R, NULL, 0, None) == \
        mr.ROUTE_ENOTSUP                                  # 12 experts
    assert f(P, Q, 8, 4096, 8, sm, NULL, F, top2, 2, 2, 1, 0, 0.0, Q, R, NULL, 0, None) == \
        mr.ROUTE_ENOTSUP                                  # expert groups
    assert f(P, Q, 8, 4096, 8, sm, R, F, mx, 2, 1, 1, 0, 0.0, Q, R, NULL, 0, None) == \
        mr.ROUTE_ENOTSUP                                  # softmax with a bias
    assert f(P, Q, 8, 4096, 8, sm, NULL, F, mx, 9, 1, 1, 0, 0.0, Q, R, NULL, 0, None) == \
        mr.ROUTE_EINVAL                                   # K > E
    assert mr.lib().route_fused_router_workspace_size(64, 4096, 8) == 0


def test_fused_router_workspace_size():
    ws = mr.lib().route_fused_router_workspace_size
    assert ws(0, 7168, 256) == 0
    assert ws(-1, 7168, 256) == 0
    assert ws(8, 7168, 128) == 0          # outside the compiled range
    assert ws(8, 7000, 256) == 0
    assert ws(1, 64, 256) == 0            # one hidden step: nothing to split
    assert ws(8193, 7168, 256) == 0       # above 8192 tokens: the single kernel
    assert ws(65536, 7168, 256) == 0
    # fp32 partials of every split, [M][256] each.
    # Up to 2048 tokens, tiles of 32 rows.  One tile and 112 steps of 64:
    # 112 splits of one step for up to 8 tokens, then at least 4 steps per
    # split (28 splits).
    assert ws(1, 7168, 256) == 4 * 256 * 1 * 112
    assert ws(8, 7168, 256) == 4 * 256 * 8 * 112
    assert ws(9, 7168, 256) == 4 * 256 * 9 * 28
    assert ws(32, 7168, 256) == 4 * 256 * 32 * 28
    # 3 tiles: 28 splits of four steps (84 workgroups)
    assert ws(65, 7168, 256) == 4 * 256 * 65 * 28
    # 16 tiles: 16 splits of seven steps (one round of 256 workgroups)
    assert ws(512, 7168, 256) == 4 * 256 * 512 * 16
    # above 2048 tokens, tiles of 64 rows: 43 tiles -> 5 splits of 23 steps
    assert ws(2720, 7168, 256) == 4 * 256 * 2720 * 5
    # 64 tiles: 4 splits of 28 steps; 65 tiles: 3 of 38; 96 tiles: 2 of 56
    assert ws(4096, 7168, 256) == 4 * 256 * 4096 * 4
    assert ws(4097, 7168, 256) == 4 * 256 * 4097 * 3
    assert ws(6144, 7168, 256) == 4 * 256 * 6144 * 2
    # above 6144 tokens, tiles of 128 rows: 49 tiles -> 5 splits of 23 steps;
    # 64 tiles -> 4 of 28
    assert ws(6145, 7168, 256) == 4 * 256 * 6145 * 5
    assert ws(8192, 7168, 256) == 4 * 256 * 8192 * 4


def test_binding_has_no_cpu_fallback():
    import torch
    x = torch.zeros(2, 8)
    with pytest.raises(ValueError, match="must live on the GPU"):
        mr.route_topk_softmax(x, 2)
    with pytest.raises(ValueError, match="must live on the GPU"):
        mr.route_biased_grouped_topk(x.bfloat16(), torch.zeros(8), 2, 2, 1)
    with pytest.raises(ValueError, match="must live on the GPU"):
        mr.route_biased_grouped_topk(x.bfloat16(), torch.zeros(8, dtype=torch.bfloat16), 2)


def test_binding_bias_dtypes():
    """The binding passes float32 or bfloat16 biases of shape [E] and rejects
    anything else before any device work."""
    import torch
    x = torch.zeros(2, 8)
    for bad in (torch.zeros(8, dtype=torch.float16), torch.zeros(8, dtype=torch.float64),
                torch.zeros(7), torch.zeros(2, 4)):
        with pytest.raises(ValueError, match="correction_bias"):
            mr.route_biased_grouped_topk(x, bad, 2)
    assert mr._bias_code(None, 8) == mr.ROUTE_F32
    assert mr._bias_code(torch.zeros(8), 8) == mr.ROUTE_F32
    assert mr._bias_code(torch.zeros(8, dtype=torch.bfloat16), 8) == mr.ROUTE_BF16


def test_dispatch_workspace_size():
    ws = mr.lib().route_dispatch_workspace_size
    assert ws(-1, 8, 256) == 0
    assert ws(10, 0, 256) == 0
    assert ws(10, 8, 0) == 0
    assert ws(10, 8, 2048) == 0
    assert ws(1 << 28, 8, 256) == 0                      # M*K beyond 2^31
    # int32 counts per (block of 2048 assignments, expert) plus per-expert totals
    assert ws(65536, 8, 256) == 4 * 256 * (256 + 1)
    assert ws(0, 8, 256) == 4 * 256
    assert ws(3, 2, 8) == 4 * 8 * 2


def disp(M=4, K=8, E=256, ids=P, w=NULL, counts=Q, offsets=R, gather=P, scatter=Q, sw=NULL,
         ws=R, wsb=1 << 20):
    return mr.lib().route_dispatch_metadata(ids, w, M, K, E, counts, offsets, gather, scatter,
                                            sw, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), mr.ROUTE_EINVAL),
    (dict(K=0), mr.ROUTE_EINVAL),
    (dict(E=0), mr.ROUTE_EINVAL),
    (dict(E=1025), mr.ROUTE_ENOTSUP),
    (dict(M=1 << 28), mr.ROUTE_ENOTSUP),
    (dict(ids=NULL), mr.ROUTE_EINVAL),
    (dict(counts=NULL), mr.ROUTE_EINVAL),
    (dict(offsets=NULL), mr.ROUTE_EINVAL),
    (dict(gather=NULL), mr.ROUTE_EINVAL),
    (dict(scatter=NULL), mr.ROUTE_EINVAL),
    (dict(ws=NULL), mr.ROUTE_EINVAL),
    (dict(wsb=4 * 256), mr.ROUTE_EINVAL),                  # workspace too small
    (dict(sw=P), mr.ROUTE_EINVAL),                         # sorted weights need weights
    (dict(ids=ctypes.c_void_p(0x10002)), mr.ROUTE_EINVAL),  # misaligned
    (dict(counts=ctypes.c_void_p(0x20001)), mr.ROUTE_EINVAL),
])
def test_dispatch_validation(kw, code):
    assert disp(**kw) == code


def test_dispatch_binding_has_no_cpu_fallback():
    import torch
    with pytest.raises(ValueError, match="must live on the GPU"):
        mr.route_dispatch_metadata(torch.zeros(2, 2, dtype=torch.int32), 4,
                                   workspace=torch.zeros(64, dtype=torch.uint8))


def test_dispatch_noalloc_validation():
    """The allocation-free dispatch entry point: the same argument checks as
    route_dispatch_metadata, and problems whose scratch exceeds its static
    4 MiB buffer are refused with their own status code, all on the host."""
    f = mr.lib().route_dispatch_metadata_noalloc
    assert f(P, NULL, -1, 8, 256, Q, R, P, Q, NULL, None) == mr.ROUTE_EINVAL
    assert f(P, NULL, 4, 8, 1025, Q, R, P, Q, NULL, None) == mr.ROUTE_ENOTSUP
    assert f(NULL, NULL, 4, 8, 256, Q, R, P, Q, NULL, None) == mr.ROUTE_EINVAL
    assert f(P, NULL, 4, 8, 256, Q, R, P, Q, P, None) == mr.ROUTE_EINVAL  # weights missing
    # 2^22 tokens x 8 slots over 1024 experts: 64 MiB of scratch
    assert mr.route_dispatch_workspace_size(1 << 22, 8, 1024) > (4 << 20)
    rc = f(P, NULL, 1 << 22, 8, 1024, Q, R, P, Q, NULL, None)
    assert rc == mr.ROUTE_ETOOBIG and "static scratch" in mr.status_str(rc)
    # the largest problem that fits: B + 1 rows of 256 counts in 4 MiB
    assert mr.route_dispatch_workspace_size(4095 * 2048 // 8, 8, 256) == 4 << 20


def test_post_routing_validation():
    L = mr.lib()
    f, s = L.route_fuse_shared_expert, L.route_sort_ids
    assert f(P, Q, -1, 8, R, 2.5, None) == mr.ROUTE_EINVAL
    assert f(P, Q, 4, 1, R, 2.5, None) == mr.ROUTE_EINVAL          # needs two slots
    assert f(P, Q, 4, 65, R, 2.5, None) == mr.ROUTE_ENOTSUP
    assert f(P, Q, 4, 8, R, float("nan"), None) == mr.ROUTE_EINVAL
    assert f(P, Q, 4, 8, R, float("inf"), None) == mr.ROUTE_EINVAL
    assert f(P, Q, 4, 8, NULL, 2.5, None) == mr.ROUTE_EINVAL
    assert f(ctypes.c_void_p(0x10002), Q, 4, 8, R, 2.5, None) == mr.ROUTE_EINVAL
    assert f(NULL, NULL, 0, 8, NULL, 2.5, None) == mr.ROUTE_OK       # empty: no launch
    assert s(P, Q, -1, 8, None) == mr.ROUTE_EINVAL
    assert s(P, Q, 4, 0, None) == mr.ROUTE_EINVAL
    assert s(P, Q, 4, 65, None) == mr.ROUTE_ENOTSUP
    assert s(P, NULL, 4, 8, None) == mr.ROUTE_EINVAL
    assert s(NULL, NULL, 0, 8, None) == mr.ROUTE_OK
