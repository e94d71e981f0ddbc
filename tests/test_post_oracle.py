"""Pins of the oracle's post-routing steps: the shared-expert slot and the
ascending id order (hand-worked cases, closed forms, invariants)."""
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "post_cases.json")))


@pytest.mark.parametrize("case", GOLD["shared"], ids=[c["name"] for c in GOLD["shared"]])
def test_shared_expert_worked(case):
    w, ids = oracle.fuse_shared_expert(case["topk_weights"], case["topk_ids"],
                                       case["shared_ids"], case["routed_scaling_factor"])
    np.testing.assert_allclose(w, np.array(case["weights"], np.float32), rtol=0, atol=1e-7)
    assert ids.tolist() == case["ids"]


def test_shared_expert_invariants():
    rng = np.random.default_rng(0)
    M, K = 500, 9
    w0 = rng.random((M, K), dtype=np.float32)
    i0 = rng.integers(0, 256, size=(M, K)).astype(np.int32)
    sid = rng.integers(256, 258, size=M).astype(np.int32)
    w, ids = oracle.fuse_shared_expert(w0, i0, sid, 1.0)
    np.testing.assert_array_equal(ids[:, :-1], i0[:, :-1])       # other slots untouched
    np.testing.assert_array_equal(w[:, :-1], w0[:, :-1])
    np.testing.assert_array_equal(ids[:, -1], sid)
    # factor 1: the slot carries exactly the sum of the others (fp32-rounded)
    np.testing.assert_array_equal(w[:, -1], w0[:, :-1].astype(np.float64).sum(1).astype(np.float32))
    w2, _ = oracle.fuse_shared_expert(w0, i0, sid, 2.0)
    np.testing.assert_array_equal(w2[:, -1], w[:, -1] / np.float32(2))  # halving is exact
    with pytest.raises(ValueError):
        oracle.fuse_shared_expert(w0[:, :1], i0[:, :1], sid)            # needs K >= 2


@pytest.mark.parametrize("case", GOLD["sort"], ids=[c["name"] for c in GOLD["sort"]])
def test_sort_ids_worked(case):
    w, ids = oracle.sort_ids(case["topk_weights"], case["topk_ids"])
    np.testing.assert_array_equal(w, np.array(case["weights"], np.float32))
    assert ids.tolist() == case["ids"]


def test_sort_ids_matches_stable_argsort():
    rng = np.random.default_rng(1)
    w0 = rng.random((300, 8), dtype=np.float32)
    i0 = rng.integers(0, 20, size=(300, 8)).astype(np.int32)  # repeats: stable by slot
    w, ids = oracle.sort_ids(w0, i0)
    order = np.argsort(i0, axis=1, kind="stable")
    np.testing.assert_array_equal(ids, np.take_along_axis(i0, order, 1))
    np.testing.assert_array_equal(w, np.take_along_axis(w0, order, 1))


def test_softcap_closed_forms():
    cap = 30.0
    l = np.array([0.0, cap * np.arctanh(0.5), -cap * np.arctanh(0.25), 1e-9, 1e4])
    y = oracle.softcap(l, cap)
    np.testing.assert_allclose(y, [0.0, cap / 2, -cap / 4, 1e-9, cap], rtol=1e-14, atol=1e-20)
    np.testing.assert_array_equal(oracle.softcap(l, 0.0), l)           # cap 0: unchanged
    x = np.linspace(-5, 5, 101)
    np.testing.assert_array_equal(oracle.softcap(-x, 7.0), -oracle.softcap(x, 7.0))  # odd
    assert (np.diff(oracle.softcap(x, 7.0)) > 0).all()                  # strictly increasing
    assert np.abs(oracle.softcap(x, 1e6) - x).max() < 1e-9               # large cap: identity


def test_softcapped_softmax_keeps_topk_ids():
    """tanh is increasing, so capping changes the softmax weights, never the ids."""
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((200, 64)) * 3
    w0, i0 = oracle.route(lg, 2, scoring=oracle.SOFTMAX, renormalize=False)
    w1, i1 = oracle.route(oracle.softcap(lg, 5.0), 2, scoring=oracle.SOFTMAX,
                          renormalize=False)
    np.testing.assert_array_equal(i0, i1)
    assert np.abs(w0 - w1).max() > 1e-3
