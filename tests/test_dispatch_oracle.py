"""Pins of the oracle's dispatch metadata (stable counting sort of the routing
assignments by expert id): hand-worked cases, a library routine, brute force
against the rank-count definition, and invariants."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = json.load(open(os.path.join(HERE, "golden", "dispatch_cases.json")))["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_dispatch_worked_cases(case):
    ids = np.array(case["topk_ids"], np.int32)
    w = np.array(case["topk_weights"], np.float32)
    counts, offsets, gather, scatter, sw = oracle.dispatch(ids, case["num_experts"], w)
    assert counts.tolist() == case["counts"]
    assert offsets.tolist() == case["offsets"]
    assert gather.tolist() == case["gather"]
    assert scatter.tolist() == case["scatter"]
    np.testing.assert_array_equal(sw, np.array(case["sorted_weights"], np.float32))


def _rank_definition(ids, E):
    """Sorted position of assignment a, written directly: the number of valid
    assignments with a smaller expert id, plus those with the same id and a
    smaller index."""
    n = len(ids)
    pos = []
    for a in range(n):
        if not 0 <= ids[a] < E:
            pos.append(-1)
            continue
        pos.append(sum(1 for b in range(n) if 0 <= ids[b] < ids[a])
                   + sum(1 for b in range(a) if ids[b] == ids[a]))
    return pos


def test_dispatch_brute_force_tiny():
    """Every id vector of length 6 over {-1, 0, 1, 2} with E = 3 (4096 cases)."""
    for ids in itertools.product((-1, 0, 1, 2), repeat=6):
        ids = np.array(ids, np.int32)
        _, _, gather, scatter, _ = oracle.dispatch(ids, 3)
        assert scatter.tolist() == _rank_definition(ids.tolist(), 3)
        nv = int((ids >= 0).sum())
        assert sorted(gather[:nv].tolist()) == [a for a in range(6) if ids[a] >= 0]


@pytest.mark.parametrize("M,K,E,seed", [(1, 1, 1, 0), (64, 8, 256, 1), (1000, 6, 160, 2),
                                        (4096, 8, 256, 3), (333, 2, 8, 4)])
def test_dispatch_matches_stable_argsort(M, K, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, E + 2, size=(M, K)).astype(np.int32)   # some out of range
    w = rng.random((M, K), dtype=np.float32)
    counts, offsets, gather, scatter, sw = oracle.dispatch(ids, E, w)
    flat, fw = ids.reshape(-1), w.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    idx = np.nonzero(valid)[0]
    order = idx[np.argsort(flat[idx], kind="stable")]
    nv = order.size
    np.testing.assert_array_equal(counts, np.bincount(flat[valid], minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    np.testing.assert_array_equal(gather[:nv], order)
    assert (gather[nv:] == -1).all()
    # invariants
    np.testing.assert_array_equal(scatter[gather[:nv]], np.arange(nv))
    assert ((scatter == -1) == ~valid).all()
    np.testing.assert_array_equal(sw[:nv], fw[order])
    assert (sw[nv:] == 0).all()
    s = flat[gather[:nv]]
    assert (np.diff(s) >= 0).all()
    same = np.diff(s) == 0
    assert (np.diff(gather[:nv])[same] > 0).all()


def test_dispatch_rejects_undefined_arguments():
    with pytest.raises(ValueError):
        oracle.dispatch(np.zeros((2, 2), np.int32), 0)
