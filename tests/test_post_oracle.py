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
