"""Pins for the CPU oracle: it is checked against things other than itself.

* hand-worked cases with closed-form answers (tests/golden/worked_cases.json);
* closed forms of the scoring functions;
* an independent brute force (pure Python, all subsets) on tiny rows, plus
  the rank-count definition of top-K;
* numpy's stable argsort as an independent sort for the ungrouped case;
* invariants that hold at any size;
* numpy's float64 matmul for the router projection.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import bf16_bits_from_f32, bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_cases.json")
SCORING = {"softmax": oracle.SOFTMAX, "sigmoid": oracle.SIGMOID}
RULE = {"max": oracle.GROUP_MAX, "top2sum": oracle.GROUP_TOP2SUM}


def _logit(tok):
    if tok.startswith("ln"):
        return np.float32(math.log(int(tok[2:])))
    return np.float32(float(tok))


def _golden_cases():
    with open(GOLDEN) as f:
        data = json.load(f)
    for case in data["cases"]:
        for exp in case["expect"]:
            p = {k: v for k, v in case.items() if k not in ("expect",)}
            p.update(exp)
            yield pytest.param(p, id=f"{case['name']}-{json.dumps({k: exp[k] for k in exp if k not in ('ids', 'weights')})}")


@pytest.mark.parametrize("p", list(_golden_cases()))
def test_worked_cases(p):
    x = np.array([[_logit(t) for t in p["logits"]]], np.float32)
    bias = None if p["bias"] is None else np.array(p["bias"], np.float32)
    w, ids = oracle.route(x, p["K"], scoring=SCORING[p["scoring"]], bias=bias,
                          num_expert_group=p["G"], topk_group=p["TG"], group_rule=RULE[p["rule"]],
                          renormalize=p["renormalize"])
    assert ids[0].tolist() == p["ids"]
    want = np.array([float(Fraction(v)) for v in p["weights"]])
    np.testing.assert_allclose(w[0], want, atol=1e-6, rtol=0)


def test_gap_diagnostics_worked():
    # W5: picks 4,5 tie at .7 (in-order gap 0); best unpicked is .5 (K gap .2);
    # kept group sum 1.4 vs dropped 1.3 (group gap .1).
    x = np.zeros((1, 8), np.float32)
    b = np.array([0.3, 0, 0, 0, 0.2, 0.2, 0, 0], np.float32)
    _, ids, gaps = oracle.route(x, 2, scoring=oracle.SIGMOID, bias=b, num_expert_group=2,
                                topk_group=1, group_rule=oracle.GROUP_TOP2SUM, with_gaps=True)
    assert ids[0].tolist() == [4, 5]
    np.testing.assert_allclose(gaps[0], [0.2, 0.0, 0.1], atol=1e-7)


# ---------------------------------------------------------------- closed forms

def test_softmax_closed_forms():
    x = np.array([0.0, math.log(3.0)], np.float64)
    s, c = oracle.row_scores(x, scoring=oracle.SOFTMAX)
    np.testing.assert_allclose(s, [0.25, 0.75], rtol=1e-15)
    np.testing.assert_array_equal(s, c)
    rng = np.random.default_rng(5)
    y = rng.standard_normal(37) * 3
    s1, _ = oracle.row_scores(y, scoring=oracle.SOFTMAX)
    s2, _ = oracle.row_scores(y + 11.5, scoring=oracle.SOFTMAX)
    assert abs(s1.sum() - 1.0) < 1e-14
    np.testing.assert_allclose(s1, s2, rtol=1e-12)
    # log-ratio of two probabilities is the logit difference
    np.testing.assert_allclose(np.log(s1[3] / s1[7]), y[3] - y[7], rtol=1e-12)


def test_sigmoid_closed_forms():
    x = np.array([0.0, math.log(3.0), -math.log(3.0), 20.0, -20.0], np.float64)
    b = np.array([0.5, -0.25, 0, 0, 0], np.float32)
    s, c = oracle.row_scores(x, scoring=oracle.SIGMOID, bias=b)
    np.testing.assert_allclose(s[:3], [0.5, 0.75, 0.25], rtol=1e-15)
    assert abs(s[3] + s[4] - 1.0) < 1e-15
    np.testing.assert_allclose(c, s + b.astype(np.float64), rtol=0, atol=0)


def test_bf16_widening_is_exact():
    bits = np.array([[0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F]], np.uint16)
    s, _ = oracle.row_scores(bits[0], scoring=oracle.SIGMOID)
    x = bf16_bits_to_f32(bits[0]).astype(np.float64)
    np.testing.assert_allclose(s, 1 / (1 + np.exp(-x)), rtol=1e-15)


def test_group_scores_worked():
    c = np.array([3.0, 1.0, 2.0, 5.0, 4.0, 0.0])
    np.testing.assert_array_equal(oracle.group_scores(c, 2, oracle.GROUP_MAX), [3.0, 5.0])
    np.testing.assert_array_equal(oracle.group_scores(c, 2, oracle.GROUP_TOP2SUM), [5.0, 9.0])
    np.testing.assert_array_equal(oracle.group_scores(c, 3, oracle.GROUP_TOP2SUM), [4.0, 7.0, 4.0])


# ---------------------------------------------------------------- brute force

def _beats(a, b):
    """(value, index) a ranks before b: larger value, then lower index."""
    return a[0] > b[0] or (a[0] == b[0] and a[1] < b[1])


def _brute_route(x, scoring, bias, G, TG, rule, K, renorm):
    """Independent definition: enumerate every subset and keep the one whose
    members all outrank every non-member."""
    E = len(x)
    if scoring == "softmax":
        mx = max(x)
        e = [math.exp(v - mx) for v in x]
        tot = 0.0
        for v in e:
            tot += v
        s = [v / tot for v in e]
    else:
        s = [1.0 / (1.0 + math.exp(-v)) for v in x]
    c = [s[i] + (float(bias[i]) if bias is not None else 0.0) for i in range(E)]
    gs = E // G
    h = []
    for g in range(G):
        vals = sorted(c[g * gs:(g + 1) * gs], reverse=True)
        h.append(vals[0] if rule == "max" else vals[0] + vals[1])
    winners = []
    for sub in itertools.combinations(range(G), TG):
        rest = [g for g in range(G) if g not in sub]
        if all(_beats((h[a], a), (h[r], r)) for a in sub for r in rest):
            winners.append(set(sub))
    assert len(winners) == 1
    kept = winners[0] if G > 1 else {0}
    cand = [i for i in range(E) if i // gs in kept]
    picks = []
    for sub in itertools.combinations(cand, K):
        rest = [i for i in cand if i not in sub]
        if all(_beats((c[a], a), (c[r], r)) for a in sub for r in rest):
            picks.append(sub)
    assert len(picks) == 1
    ids = sorted(picks[0], key=lambda i: (-c[i], i))
    # rank-count definition agrees
    for i in cand:
        rank = sum(1 for j in cand if _beats((c[j], j), (c[i], i)))
        assert (rank < K) == (i in ids)
    w = [s[i] for i in ids]
    if renorm:
        tot = 0.0
        for v in w:
            tot += v
        w = [v / tot for v in w]
    return ids, w


def _tiny_cases():
    rng = np.random.default_rng(1234)
    out = []
    for E in (4, 6, 8, 9, 10, 12):
        divisors = [g for g in range(1, E + 1) if E % g == 0]
        for trial in range(10):
            G = int(rng.choice(divisors))
            TG = int(rng.integers(1, G + 1))
            scoring = ["softmax", "sigmoid"][trial % 2]
            rule = "max" if (scoring == "softmax" or E // G < 2) else ["max", "top2sum"][trial % 3 == 0]
            if G > 1 and rule == "top2sum" and E // G < 2:
                rule = "max"
            K = int(rng.integers(1, min(TG * (E // G), 6) + 1))
            tied = trial % 3 == 1  # many exact ties
            out.append((E, G, TG, K, scoring, rule, bool(trial % 4 < 2), tied, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("E,G,TG,K,scoring,rule,renorm,tied,seed", _tiny_cases())
def test_brute_force_tiny(E, G, TG, K, scoring, rule, renorm, tied, seed):
    rng = np.random.default_rng(seed)
    M = 6
    if tied:
        x = (rng.integers(-3, 4, size=(M, E)) / 4.0).astype(np.float32)
    else:
        x = rng.standard_normal((M, E)).astype(np.float32) * 2
    use_bias = scoring == "sigmoid" and seed % 2 == 0
    bias = None
    if use_bias:
        bias = (rng.integers(-2, 3, size=E) / 8.0).astype(np.float32) if tied else \
            (rng.standard_normal(E) * 0.1).astype(np.float32)
    w, ids = oracle.route(x, K, scoring=SCORING[scoring], bias=bias, num_expert_group=G,
                          topk_group=TG, group_rule=RULE[rule], renormalize=renorm)
    for m in range(M):
        bids, bw = _brute_route([float(v) for v in x[m]], scoring, bias, G, TG, rule, K, renorm)
        assert ids[m].tolist() == bids, (m, x[m], bias)
        np.testing.assert_allclose(w[m], np.array(bw, np.float32), rtol=0, atol=0)


def test_brute_force_bf16_ties():
    """bf16 inputs repeat values within a row; ties must resolve by index."""
    rng = np.random.default_rng(99)
    bits = bf16_bits_from_f32((rng.integers(-2, 3, size=(8, 12)) * 0.5).astype(np.float32))
    x = bf16_bits_to_f32(bits)
    w, ids = oracle.route(bits, 4, scoring=oracle.SIGMOID, num_expert_group=3, topk_group=2,
                          group_rule=oracle.GROUP_TOP2SUM, renormalize=True)
    for m in range(8):
        bids, bw = _brute_route([float(v) for v in x[m]], "sigmoid", None, 3, 2, "top2sum", 4, True)
        assert ids[m].tolist() == bids
        np.testing.assert_allclose(w[m], np.array(bw, np.float32), rtol=0, atol=0)


# ------------------------------------------------------ library cross-checks

@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
def test_ungrouped_matches_stable_argsort(scoring):
    rng = np.random.default_rng(7)
    M, E, K = 64, 96, 7
    x = bf16_bits_from_f32(rng.standard_normal((M, E)).astype(np.float32))  # ties present
    bias = (rng.standard_normal(E) * 0.05).astype(np.float32) if scoring == "sigmoid" else None
    w, ids = oracle.route(x, K, scoring=SCORING[scoring], bias=bias)
    for m in range(M):
        s, c = oracle.row_scores(x[m], scoring=SCORING[scoring], bias=bias)
        want = np.argsort(-c, kind="stable")[:K]
        assert ids[m].tolist() == want.tolist()
        np.testing.assert_array_equal(w[m], s[want].astype(np.float32))


def test_router_logits_match_numpy_matmul():
    rng = np.random.default_rng(3)
    M, H, E = 5, 200, 24
    a = bf16_bits_from_f32(rng.standard_normal((M, H)).astype(np.float32))
    b = bf16_bits_from_f32((rng.standard_normal((H, E)) * 0.07).astype(np.float32))
    got = oracle.router_logits(a, b)
    want = bf16_bits_to_f32(a).astype(np.float64) @ bf16_bits_to_f32(b).astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_router_logits_exact_on_integers():
    rng = np.random.default_rng(4)
    M, H, E = 3, 64, 10
    ai = rng.integers(-8, 9, size=(M, H))
    bi = rng.integers(-8, 9, size=(H, E))
    a = bf16_bits_from_f32(ai.astype(np.float32))
    b = bf16_bits_from_f32(bi.astype(np.float32))
    got = oracle.router_logits(a, b)
    np.testing.assert_array_equal(got, (ai @ bi).astype(np.float64))
    # layout: W is [H, E]; a one-hot hidden row picks out one row of W
    one = np.zeros((1, H), np.float32)
    one[0, 5] = 1.0
    got1 = oracle.router_logits(bf16_bits_from_f32(one), b)
    np.testing.assert_array_equal(got1[0], bi[5].astype(np.float64))


# ---------------------------------------------------------------- invariants

def _kept_groups(c, G, TG, rule):
    h = oracle.group_scores(c, G, rule)
    return set(np.argsort(-h, kind="stable")[:TG].tolist())


@pytest.mark.parametrize("E,G,TG,K,scoring,rule,dtype", [
    (256, 8, 4, 8, "sigmoid", "top2sum", "bf16"),
    (160, 8, 3, 6, "softmax", "max", "f32"),
    (64, 4, 2, 5, "sigmoid", "max", "f32"),
    (128, 16, 5, 9, "sigmoid", "top2sum", "f32"),
])
def test_invariants(E, G, TG, K, scoring, rule, dtype):
    rng = np.random.default_rng(E + G + K)
    M = 200
    xf = (rng.standard_normal((M, E)) * 1.4).astype(np.float32)
    x = bf16_bits_from_f32(xf) if dtype == "bf16" else xf
    bias = (rng.standard_normal(E) * 0.14).astype(np.float32) if scoring == "sigmoid" else None
    args = dict(scoring=SCORING[scoring], bias=bias, num_expert_group=G, topk_group=TG,
                group_rule=RULE[rule])
    w, ids = oracle.route(x, K, renormalize=True, **args)
    w0, ids0 = oracle.route(x, K, renormalize=False, **args)
    np.testing.assert_array_equal(ids, ids0)
    gs = E // G
    for m in range(M):
        row = ids[m].tolist()
        assert len(set(row)) == K                                     # I1 unique
        s, c = oracle.row_scores(x[m], scoring=SCORING[scoring], bias=bias)
        kept = _kept_groups(c, G, TG, RULE[rule])
        assert all(i // gs in kept for i in row)                      # I2 in kept groups
        assert abs(float(w[m].astype(np.float64).sum()) - 1.0) < 1e-6  # I3 renorm sums to 1
        for a, b in zip(row, row[1:]):                                # I4 ordered
            assert c[a] > c[b] or (c[a] == c[b] and a < b)
        np.testing.assert_allclose(w0[m], s[row].astype(np.float32), rtol=0, atol=0)
        if scoring == "softmax":
            assert float(w0[m].astype(np.float64).sum()) <= 1.0 + 1e-7  # I10
    # I6: keeping every group equals ungrouped routing
    w6, ids6 = oracle.route(x, K, renormalize=True, **dict(args, topk_group=G))
    wu, idsu = oracle.route(x, K, renormalize=True, scoring=SCORING[scoring], bias=bias)
    np.testing.assert_array_equal(ids6, idsu)
    np.testing.assert_array_equal(w6, wu)
    # I11: rows are independent
    perm = rng.permutation(M)
    wp, idsp = oracle.route(x[perm], K, renormalize=True, **args)
    np.testing.assert_array_equal(idsp, ids[perm])
    np.testing.assert_array_equal(wp, w[perm])


def test_group_max_with_tg_ge_k_is_plain_topk():   # I7
    rng = np.random.default_rng(11)
    x = rng.standard_normal((300, 64)).astype(np.float32)
    for G, TG, K in ((8, 4, 4), (8, 6, 5), (4, 3, 2)):
        _, ids_g = oracle.route(x, K, scoring=oracle.SIGMOID, num_expert_group=G, topk_group=TG,
                                group_rule=oracle.GROUP_MAX)
        _, ids_u = oracle.route(x, K, scoring=oracle.SIGMOID)
        np.testing.assert_array_equal(ids_g, ids_u)


def test_unbiased_topk_is_topk_of_logits():        # I8, I9, I5
    rng = np.random.default_rng(12)
    x = rng.standard_normal((300, 40)).astype(np.float32)
    want = np.argsort(-x, axis=1, kind="stable")[:, :6]
    _, ids_soft = oracle.route(x, 6, scoring=oracle.SOFTMAX)
    _, ids_sig = oracle.route(x, 6, scoring=oracle.SIGMOID)
    _, ids_bg1 = oracle.route(x, 6, scoring=oracle.SIGMOID, bias=np.zeros(40, np.float32),
                              group_rule=oracle.GROUP_TOP2SUM)
    np.testing.assert_array_equal(ids_soft, want)
    np.testing.assert_array_equal(ids_sig, want)
    np.testing.assert_array_equal(ids_bg1, want)


def test_permuting_within_group_permutes_ids():    # I12
    rng = np.random.default_rng(13)
    E, G = 32, 4
    x = rng.standard_normal((50, E)).astype(np.float32)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    perm = np.arange(E)
    for g in range(G):
        perm[g * 8:(g + 1) * 8] = g * 8 + rng.permutation(8)
    args = dict(scoring=oracle.SIGMOID, num_expert_group=G, topk_group=2,
                group_rule=oracle.GROUP_TOP2SUM, renormalize=True)
    w, ids = oracle.route(x, 5, bias=b, **args)
    wp, idsp = oracle.route(x[:, perm], 5, bias=b[perm], **args)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(perm[idsp], ids)
    assert np.all(inv[ids] == idsp)
    np.testing.assert_array_equal(wp, w)


@pytest.mark.parametrize("kw", [
    dict(num_expert_group=3),                      # E % G != 0
    dict(num_expert_group=4, topk_group=5),        # TG > G
    dict(num_expert_group=4, topk_group=1, K=3),   # K > TG * E/G
    dict(num_expert_group=8, topk_group=2, group_rule=oracle.GROUP_TOP2SUM),  # groups of 1
    dict(K=0),
])
def test_rejects_undefined_arguments(kw):
    x = np.zeros((2, 8), np.float32)
    K = kw.pop("K", 2)
    with pytest.raises(ValueError):
        oracle.route(x, K, **kw)
