"""The parity comparison itself: it accepts the oracle's own answer, accepts a
near-tie resolved the other way, and rejects real mistakes."""
import numpy as np

import oracle
from parity_check import compare


def _case():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((40, 32)) * 1.4).astype(np.float32)
    b = (rng.standard_normal(32) * 0.1).astype(np.float32)
    kw = dict(scoring=oracle.SIGMOID, bias=b, G=4, TG=2, rule=oracle.GROUP_TOP2SUM, K=4,
              renorm=True)
    w, ids = oracle.route(x, 4, scoring=oracle.SIGMOID, bias=b, num_expert_group=4, topk_group=2,
                          group_rule=oracle.GROUP_TOP2SUM, renormalize=True)
    return x, b, w, ids, kw


def test_accepts_oracle_output():
    x, b, w, ids, kw = _case()
    rep = compare(x, w, ids, **kw)
    assert rep.ok() and rep.exact == 40


def test_rejects_swapped_order_and_wrong_ids():
    x, b, w, ids, kw = _case()
    ids2 = ids.copy()
    ids2[3, [0, 1]] = ids2[3, [1, 0]]
    w2 = w.copy()
    w2[3, [0, 1]] = w2[3, [1, 0]]
    ids2[7, 2] = (ids2[7, 2] + 1) % 32
    rep = compare(x, w2, ids2, **kw)
    assert {f[0] for f in rep.failures} == {3, 7}


def test_rejects_weight_error():
    x, b, w, ids, kw = _case()
    w2 = w.copy()
    w2[5, 1] += 2e-5
    rep = compare(x, w2, ids, **kw)
    assert [f[0] for f in rep.failures] == [5]


def test_accepts_near_tie_other_way_but_not_far():
    # two experts whose selection scores differ by ~1e-7 at the K boundary
    x = np.zeros((1, 8), np.float32)
    b = np.array([0.3, 0.2, 0.2 + 1e-7, 0, 0, 0, 0, 0], np.float32)
    args = dict(scoring=oracle.SIGMOID, bias=b, G=1, TG=1, rule=oracle.GROUP_TOP2SUM, K=2,
                renorm=False)
    w, ids = oracle.route(x, 2, scoring=oracle.SIGMOID, bias=b)
    assert ids[0].tolist() == [0, 2]
    other = np.array([[0, 1]], np.int32)
    rep = compare(x, w, other, **args)
    assert rep.ok() and rep.near_tie_k == 1
    far = np.array([[0, 3]], np.int32)
    assert not compare(x, w, far, **args).ok()
