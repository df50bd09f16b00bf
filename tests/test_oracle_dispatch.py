"""Pins for the oracle's dispatch step (counts, capacity drop, permutation).

Brute force over every capacity-sized subset on tiny inputs with tied scores,
plus the structural invariants on random routings.
"""
import itertools

import numpy as np
import pytest

import oracle

from routing_expert_ffn_sigmoid_amd.workloads import capacity_for


def _random_routing(rng, T, N, k):
    idx = np.stack([rng.choice(N, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    return idx


def _check_structure(idx, score, N, C, d):
    T, k = idx.shape
    counts = np.bincount(idx.ravel(), minlength=N)
    np.testing.assert_array_equal(d["counts"], counts)
    kept = np.minimum(counts, C) if C > 0 else counts
    np.testing.assert_array_equal(np.diff(d["offsets"]), kept)
    assert d["offsets"][0] == 0
    assert d["n_dropped"] == int((counts - kept).sum())
    inv = d["inv_row"]
    rt = d["row_token"]
    M = int(d["offsets"][-1])
    assert rt.shape == (M,)
    # inv_row and row_token are mutually inverse on kept slots
    seen = np.zeros(M, bool)
    for t in range(T):
        for j in range(k):
            r = inv[t, j]
            if r >= 0:
                assert rt[r] == t and not seen[r]
                seen[r] = True
                e = idx[t, j]
                assert d["offsets"][e] <= r < d["offsets"][e + 1]
    assert seen.all()
    # token order inside each expert segment
    for e in range(N):
        seg = rt[d["offsets"][e]:d["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
    # every dropped score <= every kept score of the same expert
    for e in range(N):
        ks = [score[t, j] for t in range(T) for j in range(k) if idx[t, j] == e and inv[t, j] >= 0]
        ds = [score[t, j] for t in range(T) for j in range(k) if idx[t, j] == e and inv[t, j] < 0]
        if ks and ds:
            assert max(ds) <= min(ks)
    all_dropped = int(np.sum(np.all(inv < 0, axis=1))) if k > 0 else 0
    assert d["n_tok_all_dropped"] == all_dropped


@pytest.mark.parametrize("T,N,k,C", [(50, 8, 2, 0), (50, 8, 2, 9), (200, 16, 4, 40),
                                     (300, 32, 6, 0), (64, 4, 4, 64), (17, 16, 3, 1)])
def test_dispatch_structure_random(T, N, k, C):
    rng = np.random.default_rng(T + N + k + C)
    idx = _random_routing(rng, T, N, k)
    score = rng.integers(0, 5, size=(T, k)).astype(np.float32) * 0.125
    d = oracle.dispatch(idx, score, N, C)
    _check_structure(idx, score, N, C, d)


def _brute_kept(idx, score, N, C):
    """Per expert: the C-subset of its assignments with the largest score sum,
    ties -> lexicographically smallest token tuple."""
    T, k = idx.shape
    kept = np.zeros_like(idx, dtype=bool)
    for e in range(N):
        items = [(t, j) for t in range(T) for j in range(k) if idx[t, j] == e]
        if len(items) <= C:
            for (t, j) in items:
                kept[t, j] = True
            continue
        best, best_sum = None, None
        for comb in itertools.combinations(range(len(items)), C):
            s = sum(float(score[items[i]]) for i in comb)
            if best is None or s > best_sum:
                best, best_sum = comb, s
        for i in best:
            kept[items[i]] = True
    return kept


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("C", [1, 2, 3])
def test_capacity_matches_bruteforce(seed, C):
    rng = np.random.default_rng(100 + seed)
    T, N, k = 9, 4, 2
    idx = _random_routing(rng, T, N, k)
    score = rng.integers(0, 3, size=(T, k)).astype(np.float32) * 0.25  # many ties
    d = oracle.dispatch(idx, score, N, C)
    np.testing.assert_array_equal(d["inv_row"] >= 0, _brute_kept(idx, score, N, C))
    _check_structure(idx, score, N, C, d)


def test_capacity_at_least_T_drops_nothing():
    rng = np.random.default_rng(5)
    T, N, k = 120, 8, 3
    idx = _random_routing(rng, T, N, k)
    score = rng.random((T, k)).astype(np.float32)
    for C in (0, T, T + 5):
        d = oracle.dispatch(idx, score, N, C)
        assert d["n_dropped"] == 0 and d["n_tok_all_dropped"] == 0
        assert d["offsets"][-1] == T * k


def test_capacity_factor_formula():
    # 1.25 * 16384 * 8 / 256 = 640 exactly; the ceiling matters off-grid
    assert capacity_for(16384, 8, 256) == 640
    assert capacity_for(100, 3, 7) == int(np.ceil(1.25 * 100 * 3 / 7))
