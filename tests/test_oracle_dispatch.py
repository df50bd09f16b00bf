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


# ------------------------------------------- v2 device-level token dropping

def _drop_key(score, t, e):
    # higher score first, then lower token, then lower expert
    return (float(score), -t, -e)


@pytest.mark.parametrize("T,N,G,k,cap", [(12, 8, 2, 3, 7), (20, 12, 3, 4, 9), (9, 8, 4, 2, 2),
                                         (30, 16, 4, 4, 11), (6, 4, 2, 2, 1)])
def test_grouped_drop_pairwise_dominance(T, N, G, k, cap):
    """[EVO] §DeepSeek-v2 device-level token dropping: in a group over its
    cap, every kept assignment outranks every dropped one, exactly cap stay;
    groups within their cap keep everything.  Scores on a coarse grid so
    that ties between tokens (and between two experts of one token) occur."""
    rng = np.random.default_rng(T * 100 + N + cap)
    idx = _random_routing(rng, T, N, k)
    score = (rng.integers(0, 4, size=(T, k)) * 0.25).astype(np.float32)
    d = oracle.dispatch_grouped(idx, score, N, G, cap)
    gs = N // G
    inv = d["inv_row"]
    n_drop = 0
    for g in range(G):
        members = [(t, j) for t in range(T) for j in range(k) if idx[t, j] // gs == g]
        kept = [(t, j) for (t, j) in members if inv[t, j] >= 0]
        dropped = [(t, j) for (t, j) in members if inv[t, j] < 0]
        assert len(kept) == min(len(members), cap)
        n_drop += len(dropped)
        for (ta, ja) in kept:
            for (tb, jb) in dropped:
                assert _drop_key(score[ta, ja], ta, idx[ta, ja]) > \
                    _drop_key(score[tb, jb], tb, idx[tb, jb])
    assert d["n_dropped"] == n_drop
    # rows: expert-major, token order inside an expert, counts before dropping
    counts = np.bincount(idx.ravel(), minlength=N)
    np.testing.assert_array_equal(d["counts"], counts)
    kept_e = np.zeros(N, np.int64)
    for t in range(T):
        for j in range(k):
            if inv[t, j] >= 0:
                kept_e[idx[t, j]] += 1
    np.testing.assert_array_equal(np.diff(d["offsets"]), kept_e)
    rt = d["row_token"]
    for e in range(N):
        toks = rt[d["offsets"][e]:d["offsets"][e + 1]]
        assert list(toks) == sorted(toks)
        for r, t in enumerate(toks):
            j = list(idx[t]).index(e)
            assert inv[t, j] == d["offsets"][e] + r
    all_dropped = sum(1 for t in range(T) if k > 0 and (inv[t] < 0).all())
    assert d["n_tok_all_dropped"] == all_dropped


@pytest.mark.parametrize("cap", [1, 3, 5, 40])
def test_grouped_drop_with_one_expert_per_group_is_expert_capacity(cap):
    # a device holding a single expert: the device cap is that expert's capacity
    rng = np.random.default_rng(cap)
    T, N, k = 50, 8, 3
    idx = _random_routing(rng, T, N, k)
    score = (rng.integers(0, 6, size=(T, k)) * 0.125).astype(np.float32)
    a = oracle.dispatch_grouped(idx, score, N, N, cap)
    b = oracle.dispatch(idx, score, N, capacity=cap)
    for key in ("counts", "offsets", "row_token", "inv_row", "n_dropped", "n_tok_all_dropped"):
        np.testing.assert_array_equal(np.asarray(a[key]), np.asarray(b[key]), err_msg=key)


def test_grouped_drop_cap_at_max_load_drops_nothing():
    rng = np.random.default_rng(3)
    T, N, G, k = 64, 16, 4, 4
    idx = _random_routing(rng, T, N, k)
    score = rng.random((T, k)).astype(np.float32)
    gs = N // G
    max_load = int(np.bincount(idx.ravel() // gs, minlength=G).max())
    a = oracle.dispatch_grouped(idx, score, N, G, max_load)
    b = oracle.dispatch(idx, score, N, capacity=0)
    assert a["n_dropped"] == 0
    for key in ("counts", "offsets", "row_token", "inv_row"):
        np.testing.assert_array_equal(np.asarray(a[key]), np.asarray(b[key]), err_msg=key)
    c = oracle.dispatch_grouped(idx, score, N, G, max_load - 1)
    assert c["n_dropped"] >= 1
