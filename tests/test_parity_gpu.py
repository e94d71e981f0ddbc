"""GPU parity: every routing entry point against the CPU oracle on the same
seeded inputs (full workload sizes, an M sweep, random shapes with ragged
tails, ties, edge cases)."""
import numpy as np
import pytest
import torch

import moe_expert_routing_amd as mr
import oracle
from gpu_util import log, oracle_args, route_gpu, to_device
from parity_check import compare
from workloads import (BIASED_GROUPED_M_SWEEP, WORKLOADS, bf16_bits_from_f32,
                       bf16_bits_to_f32, make_bias, make_logits, random_logits)

pytestmark = pytest.mark.gpu


def _check_workload(wl, M=None):
    x = make_logits(wl, M)
    b = make_bias(wl)
    log(f"[gpu] {wl.entry} workload={wl.name} M={x.shape[0]} E={wl.E} K={wl.K} G={wl.G} "
        f"TG={wl.TG}")
    w, ids = route_gpu(wl.entry, to_device(x), K=wl.K, G=wl.G, TG=wl.TG, scoring=wl.scoring,
                       bias=None if b is None else to_device(b), renorm=wl.renormalize)
    sc, rule = oracle_args(wl.entry, wl.scoring)
    rep = compare(x, w, ids, scoring=sc, bias=b, G=wl.G, TG=wl.TG, rule=rule, K=wl.K,
                  renorm=wl.renormalize, label=f"{wl.name} M={x.shape[0]}")
    log(f"[gpu]   {rep.summary()}")
    assert rep.ok(), rep.summary()
    # near ties must stay rare: they come only from sub-1e-6 gaps
    assert rep.near_tie <= max(2, rep.rows // 1000), rep.summary()
    return rep


@pytest.mark.parametrize("name", ["softmax_e8_k2", "sigmoid_bias_e256_k8", "grouped_softmax_e160"])
def test_workload_full_size(name):
    _check_workload(WORKLOADS[name])


@pytest.mark.parametrize("M", BIASED_GROUPED_M_SWEEP)
def test_biased_grouped_m_sweep(M):
    _check_workload(WORKLOADS["biased_grouped_e256"], M)


def _random_cases():
    cases = []
    rng = np.random.default_rng(2024)
    shapes = [(8, 1), (8, 2), (16, 4), (60, 1), (60, 6), (64, 8), (128, 8), (160, 8), (160, 1),
              (192, 6), (256, 1), (256, 8), (256, 16), (384, 8), (512, 16), (1024, 32), (100, 5),
              (72, 9), (256, 64), (48, 3)]
    entries = ["route_topk_softmax", "route_grouped_topk", "route_biased_grouped_topk"]
    for i, (E, G) in enumerate(shapes):
        for entry in entries:
            if entry == "route_topk_softmax" and G != 1:
                continue
            if entry == "route_biased_grouped_topk" and G > 1 and E // G < 2:
                continue
            TG = int(rng.integers(1, G + 1))
            K = int(rng.integers(1, min(TG * (E // G), 64) + 1))
            dtype = ["f32", "bf16"][(i + len(cases)) % 2]
            scoring = "softmax" if entry == "route_topk_softmax" else \
                ["softmax", "sigmoid"][len(cases) % 2]
            M = int(rng.choice([1, 3, 63, 65, 257, 1000]))
            cases.append((entry, E, G, TG, K, dtype, scoring, bool(len(cases) % 2), M,
                          int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("entry,E,G,TG,K,dtype,scoring,renorm,M,seed", _random_cases())
def test_random_shapes(entry, E, G, TG, K, dtype, scoring, renorm, M, seed):
    rng = np.random.default_rng(seed)
    x = random_logits(rng, M, E, dtype, std=1.5)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32) \
        if entry == "route_biased_grouped_topk" and seed % 3 else None
    log(f"[gpu] {entry} E={E} G={G} TG={TG} K={K} {dtype} {scoring} renorm={renorm} M={M} "
        f"seed={seed}")
    w, ids = route_gpu(entry, to_device(x), K=K, G=G, TG=TG, scoring=scoring,
                       bias=None if b is None else to_device(b), renorm=renorm)
    sc, rule = oracle_args(entry, scoring)
    rep = compare(x, w, ids, scoring=sc, bias=b, G=G, TG=TG, rule=rule, K=K, renorm=renorm)
    assert rep.ok(), rep.summary()


def _kernel_variants():
    """(entry, dtype, E, G, TG, K, scoring, with_bias): every specialised
    routing kernel the entry points reach (bf16 and fp32 at 256 experts,
    fp32 at 160 and at 8)."""
    out = []
    for dtype, E in (("bf16", 256), ("f32", 256), ("f32", 160)):
        out += [("route_topk_softmax", dtype, E, 1, 1, 8, "softmax", False),
                ("route_biased_grouped_topk", dtype, E, 1, 1, 8, "sigmoid", True),
                ("route_biased_grouped_topk", dtype, E, 1, 1, 8, "sigmoid", False),
                ("route_biased_grouped_topk", dtype, E, 8, 4, 8, "sigmoid", True),
                ("route_biased_grouped_topk", dtype, E, 8, 4, 8, "sigmoid", False),
                ("route_grouped_topk", dtype, E, 8, 3, 6, "softmax", False),
                ("route_grouped_topk", dtype, E, 8, 3, 6, "sigmoid", False)]
    out += [("route_topk_softmax", "f32", 8, 1, 1, 2, "softmax", False),
            ("route_biased_grouped_topk", "f32", 8, 1, 1, 2, "sigmoid", True),
            ("route_grouped_topk", "f32", 8, 1, 1, 1, "sigmoid", False)]
    return out


# Row counts for each layout of 256 experts: up to 2048 tokens sigmoid
# scoring takes the one-row-per-wave kernel; up to 4096 tokens ungrouped rows
# take 16 lanes a row; the rest 8 lanes a row.
SMALL_M, MID_M, LARGE_M = 1000, 3000, 5000


@pytest.mark.parametrize("M", [SMALL_M, MID_M, LARGE_M])
@pytest.mark.parametrize("entry,dtype,E,G,TG,K,scoring,with_bias", _kernel_variants())
def test_every_specialised_kernel(entry, dtype, E, G, TG, K, scoring, with_bias, M):
    rng = np.random.default_rng(E * 100 + G * 10 + K + (1 if with_bias else 0) + len(scoring))
    # ragged last tile for every layout
    x = random_logits(rng, M, E, dtype, std=1.5)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32) if with_bias else None
    log(f"[gpu] {entry} {dtype} E={E} G={G} TG={TG} K={K} {scoring} bias={with_bias}")
    w, ids = route_gpu(entry, to_device(x), K=K, G=G, TG=TG, scoring=scoring,
                       bias=None if b is None else to_device(b), renorm=True)
    sc, rule = oracle_args(entry, scoring)
    rep = compare(x, w, ids, scoring=sc, bias=b, G=G, TG=TG, rule=rule, K=K, renorm=True)
    assert rep.ok(), rep.summary()


@pytest.mark.parametrize("M", [777, 2777, 4777])
@pytest.mark.parametrize("K", [1, 3, 5, 7])
@pytest.mark.parametrize("G,TG", [(8, 4), (1, 1)])
def test_biased_kernel_every_k(K, G, TG, M):
    """The biased kernels unroll their merge rounds to eight and leave after
    the K-th: every K below eight, grouped and ungrouped."""
    rng = np.random.default_rng(300 + 10 * K + G)
    x = random_logits(rng, M, 256, "bf16", std=1.5)
    b = (rng.standard_normal(256) * 0.1).astype(np.float32)
    log(f"[gpu] route_biased_grouped_topk bf16 E=256 G={G} TG={TG} K={K} M={M}")
    w, ids = route_gpu("route_biased_grouped_topk", to_device(x), K=K, G=G, TG=TG,
                       scoring="sigmoid", bias=to_device(b), renorm=True)
    sc, rule = oracle_args("route_biased_grouped_topk", "sigmoid")
    rep = compare(x, w, ids, scoring=sc, bias=b, G=G, TG=TG, rule=rule, K=K, renorm=True)
    assert rep.ok(), rep.summary()


@pytest.mark.parametrize("E,G,TG,K,dtype,M,half", [
    (256, 8, 4, 8, "bf16", 3000, 3.0),   # 8-row kernel, top-2-sum groups
    (256, 1, 1, 8, "bf16", 3000, 3.0),   # 16 lanes a row, ungrouped
    (256, 1, 1, 8, "bf16", 5000, 3.0),   # 8-row kernel, ungrouped
    (256, 8, 4, 8, "bf16", 1000, 3.0),   # one row per wave, top-2-sum groups
    (256, 1, 1, 8, "f32", 1000, 3.0),    # one row per wave, ungrouped
    (256, 8, 4, 8, "bf16", 3000, 1.2),   # 8-row kernel, coarsest key window
    (160, 8, 3, 6, "f32", 777, 3.0),     # 160 experts in groups of 20
    (384, 8, 4, 8, "bf16", 300, 3.0),    # generic kernel
    (256, 8, 4, 8, "bf16", 1000, 1.2),   # widest window that keeps the keys (R = 4)
])
def test_wide_bias_takes_the_exact_path(E, G, TG, K, dtype, M, half):
    """A selection-score spread wider than 4 (bias U(-3, 3)) makes the
    fixed-point keys too coarse; the kernels then select on exact fp32
    comparisons.  With U(-1.2, 1.2) the spread is about 3.4: keys on the
    coarsest window, a step of 4 * 2^-23."""
    rng = np.random.default_rng(E * 1000 + M)
    x = random_logits(rng, M, E, dtype, std=1.5)
    b = rng.uniform(-half, half, E).astype(np.float32)
    assert (b.max() - b.min() > 4.0) == (half > 2.0)
    log(f"[gpu] route_biased_grouped_topk wide bias E={E} G={G} TG={TG} K={K} {dtype} M={M} "
        f"U(-{half}, {half})")
    w, ids = route_gpu("route_biased_grouped_topk", to_device(x), K=K, G=G, TG=TG,
                       scoring="sigmoid", bias=to_device(b), renorm=True)
    sc, rule = oracle_args("route_biased_grouped_topk", "sigmoid")
    rep = compare(x, w, ids, scoring=sc, bias=b, G=G, TG=TG, rule=rule, K=K, renorm=True)
    assert rep.ok(), rep.summary()


@pytest.mark.parametrize("M", [512, 2560, 4600])
@pytest.mark.parametrize("entry,scoring", [("route_biased_grouped_topk", "sigmoid"),
                                           ("route_grouped_topk", "softmax"),
                                           ("route_topk_softmax", "softmax")])
def test_exact_ties_resolve_by_index(entry, scoring, M):
    """Logits drawn from 5 values: most scores tie exactly and the lower
    expert index must win, with no tolerance."""
    rng = np.random.default_rng(77)
    E = 256
    G, TG, K = (1, 1, 8) if entry == "route_topk_softmax" else (8, 4, 8)
    x = bf16_bits_from_f32((rng.integers(-2, 3, size=(M, E)) * 0.5).astype(np.float32))
    log(f"[gpu] ties {entry} M={M} E={E}")
    w, ids = route_gpu(entry, to_device(x), K=K, G=G, TG=TG, scoring=scoring, renorm=True)
    sc, rule = oracle_args(entry, scoring)
    rep = compare(x, w, ids, scoring=sc, G=G, TG=TG, rule=rule, K=K, renorm=True)
    assert rep.ok() and rep.exact == M, rep.summary()


@pytest.mark.parametrize("M", [SMALL_M, MID_M, LARGE_M])
@pytest.mark.parametrize("entry,E,G,TG,K,scoring,dtype,hot", [
    ("route_biased_grouped_topk", 256, 8, 4, 8, "sigmoid", "bf16", 16),
    ("route_grouped_topk", 256, 8, 4, 8, "sigmoid", "f32", 16),
    ("route_biased_grouped_topk", 256, 1, 1, 8, "sigmoid", "bf16", 32),
    ("route_topk_softmax", 256, 1, 1, 8, "softmax", "f32", 32),
    ("route_grouped_topk", 160, 8, 3, 6, "softmax", "f32", 10),
])
def test_one_lane_holds_most_picks(entry, E, G, TG, K, scoring, dtype, hot, M):
    """About half the rows have their whole top K among the first `hot`
    experts, the candidates one lane of the kernel holds: more picks than
    its short list keeps, so those waves must take the exact path.  The
    other rows are ordinary, so waves mix both kinds."""
    rng = np.random.default_rng(E * 10 + K)
    xf = rng.standard_normal((M, E), dtype=np.float32)
    hot_rows = rng.random(M) < 0.5
    xf[hot_rows, :hot] += np.float32(6.0)
    x = bf16_bits_from_f32(xf) if dtype == "bf16" else xf
    b = None
    if entry == "route_biased_grouped_topk":
        # small, so that the bias does not undo the lift of the hot experts
        b = rng.standard_normal(E, dtype=np.float32) * np.float32(0.01)
    log(f"[gpu] one lane holds most picks: {entry} E={E} G={G} TG={TG} K={K} hot={hot}")
    w, ids = route_gpu(entry, to_device(x), K=K, G=G, TG=TG, scoring=scoring,
                       bias=None if b is None else to_device(b), renorm=True)
    # the premise: most hot rows take all K picks from the hot experts
    assert (ids[hot_rows] < hot).all(axis=1).mean() > 0.9
    sc, rule = oracle_args(entry, scoring)
    rep = compare(x, w, ids, scoring=sc, bias=b, G=G, TG=TG, rule=rule, K=K, renorm=True)
    log(f"[gpu]   {rep.summary()}")
    assert rep.ok(), rep.summary()


def test_empty_batch():
    wl = WORKLOADS["biased_grouped_e256"]
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    b = to_device(make_bias(wl))
    w, ids = mr.route_biased_grouped_topk(x, b, 8, 8, 4, True)
    torch.cuda.synchronize()
    assert w.shape == (0, 8) and ids.shape == (0, 8)


def test_k_equals_all_candidates():
    rng = np.random.default_rng(3)
    x = random_logits(rng, 33, 64, "f32")
    log("[gpu] K = TG*E/G")
    w, ids = route_gpu("route_grouped_topk", to_device(x), K=16, G=8, TG=2, scoring="sigmoid",
                       renorm=True)
    rep = compare(x, w, ids, scoring=1, G=8, TG=2, rule=0, K=16, renorm=True)
    assert rep.ok(), rep.summary()


def test_deterministic_and_stream_and_row_independent():
    wl = WORKLOADS["biased_grouped_e256"]
    x = to_device(make_logits(wl, 4099))
    b = to_device(make_bias(wl))
    log("[gpu] determinism / side stream / row subsets")
    w1, i1 = mr.route_biased_grouped_topk(x, b, 8, 8, 4, True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        w2, i2 = mr.route_biased_grouped_topk(x, b, 8, 8, 4, True, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(w1, w2) and torch.equal(i1, i2)
    w3, i3 = mr.route_biased_grouped_topk(x[1000:1777].contiguous(), b, 8, 8, 4, True)
    torch.cuda.synchronize()
    assert torch.equal(w3, w1[1000:1777]) and torch.equal(i3, i1[1000:1777])


def test_bad_arguments_raise_before_launch():
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(256, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        mr.route_biased_grouped_topk(x, b, 8, 3, 1, True)      # 256 % 3
    with pytest.raises(ValueError):
        mr.route_biased_grouped_topk(x, b, 200, 8, 4, True)    # K > TG*E/G
    with pytest.raises(ValueError):
        mr.route_grouped_topk(x, 8, 8, 4, True, scoring_func="tanh")
    with pytest.raises(ValueError):
        mr.route_topk_softmax(x.t(), 2)                         # not contiguous


@pytest.mark.parametrize("M", [1000, 4096])
@pytest.mark.parametrize("logit_dtype", ["bf16", "f32"])
def test_near_tied_picks_keep_the_exact_order(logit_dtype, M):
    """Pairs of experts (2j, 2j+1) whose biases differ by 3e-8 .. 6e-7 in
    favour of the higher index, given equal high logits in every row: their
    selection scores are closer than the kernel's fixed-point step, so the
    keys tie and would put the lower index first.  Every row must still come
    out in the exact order (the strict rule: only the K-th pick may differ
    on a near tie, as it does where a planted pair straddles it)."""
    rng = np.random.default_rng(2024)
    E, K, G, TG = 256, 8, 8, 4
    base = (rng.standard_normal(E // 2) * 0.05).astype(np.float32)
    gap = rng.uniform(3e-8, 6e-7, size=E // 2)
    b = np.empty(E, np.float32)
    b[0::2] = base
    b[1::2] = (base.astype(np.float64) + gap).astype(np.float32)   # odd expert ahead
    assert (b[1::2].astype(np.float64) > b[0::2]).all()
    xf = rng.standard_normal((M, E)).astype(np.float32)
    for r in range(M):  # two random pairs per row get equal high logits
        for j in rng.choice(E // 2, size=2, replace=False):
            xf[r, 2 * j] = xf[r, 2 * j + 1] = 4.0
    x = bf16_bits_from_f32(xf) if logit_dtype == "bf16" else xf
    log(f"[gpu] near-tied picks M={M} logits={logit_dtype}")
    w, ids = mr.route_biased_grouped_topk(to_device(x), to_device(b), K, G, TG, True)
    torch.cuda.synchronize()
    rep = compare(x, w.cpu().numpy(), ids.cpu().numpy(), scoring=oracle.SIGMOID, bias=b, G=G,
                  TG=TG, rule=oracle.GROUP_TOP2SUM, K=K, renorm=True,
                  label=f"planted near ties M={M} logits={logit_dtype}")
    log(f"[gpu]   {rep.summary()}")
    # planted pairs that straddle the K-th pick are the one allowed exception
    assert rep.strict_ok and rep.exact + rep.near_tie_k == M, rep.summary()


def _row_kernel_cases():
    """(dtype, bias kind, G, TG, K, entry, half-width of a uniform bias or 0)"""
    out = []
    for dtype in ("bf16", "f32"):
        for bias in ("f32", "bf16", None):
            out += [(dtype, bias, 8, 4, 8, "route_biased_grouped_topk", 0.0),
                    (dtype, bias, 1, 1, 8, "route_biased_grouped_topk", 0.0),
                    (dtype, bias, 8, 2, 5, "route_biased_grouped_topk", 0.0)]
        out += [(dtype, None, 8, 3, 6, "route_grouped_topk", 0.0),
                (dtype, "f32", 8, 4, 8, "route_biased_grouped_topk", 3.0),
                (dtype, "f32", 1, 1, 8, "route_biased_grouped_topk", 3.0)]
    return out


@pytest.mark.parametrize("dtype,bias_kind,G,TG,K,entry,half", _row_kernel_cases())
def test_row_kernel_matches_the_8_row_kernel(dtype, bias_kind, G, TG, K, entry, half):
    """Up to 2048 tokens a row goes to the one-row-per-wave kernel, up to 4096
    ungrouped rows to 16 lanes a row, and otherwise to 8 lanes a row; all take
    the same decisions with the same arithmetic, so rows routed in a batch of
    5000 and again in slices of 3000, 1500 or 7 give the same bits (and the
    oracle's result)."""
    rng = np.random.default_rng(len(_row_kernel_cases()) + G * 7 + TG * 3 + K + int(half))
    M = 5000
    x = random_logits(rng, M, 256, dtype, std=1.5)
    b = None
    if bias_kind is not None:
        b = (rng.uniform(-half, half, 256) if half else rng.standard_normal(256) * 0.1
             ).astype(np.float32)
        if bias_kind == "bf16":
            b = bf16_bits_to_f32(bf16_bits_from_f32(b))
    log(f"[gpu] row kernel vs 8-row kernel {entry} {dtype} bias={bias_kind} G={G} TG={TG} "
        f"K={K} half={half}")
    bd = None
    if b is not None:
        bd = to_device(bf16_bits_from_f32(b)) if bias_kind == "bf16" else to_device(b)
    xd = to_device(x)

    def run(xs):
        if entry == "route_grouped_topk":
            return mr.route_grouped_topk(xs, K, G, TG, True, "sigmoid")
        return mr.route_biased_grouped_topk(xs, bd, K, G, TG, True)
    w_all, i_all = run(xd)
    w_3k, i_3k = run(xd[1500:4500].contiguous())
    w_mid, i_mid = run(xd[500:2000].contiguous())
    w_few, i_few = run(xd[1234:1241].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(w_3k, w_all[1500:4500]) and torch.equal(i_3k, i_all[1500:4500])
    assert torch.equal(w_mid, w_all[500:2000]) and torch.equal(i_mid, i_all[500:2000])
    assert torch.equal(w_few, w_all[1234:1241]) and torch.equal(i_few, i_all[1234:1241])
    sc, rule = oracle_args(entry, "sigmoid")
    rep = compare(x, w_all.cpu().numpy(), i_all.cpu().numpy(), scoring=sc, bias=b, G=G, TG=TG,
                  rule=rule, K=K, renorm=True)
    assert rep.ok(), rep.summary()
