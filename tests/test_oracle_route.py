"""Pins for the oracle's routing step (scores, group limit, top-k, gates).

* brute force: every subset of groups and of experts, on integer-valued keys
  where ties really occur;
* the uniform-routing constructions whose load-balance loss is exactly 1;
* invariants on random inputs (k distinct experts, kept groups only, gate
  sums, bias used for selection only);
* special cases that reduce to numpy's stable argsort.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- brute force

def _best_subset(vals, size):
    """Subset (sorted index tuple) of `size` indices maximising the sum of
    vals; ties -> lexicographically smallest tuple."""
    best, best_sum = None, None
    for comb in itertools.combinations(range(len(vals)), size):
        s = sum(vals[i] for i in comb)
        if best is None or s > best_sum:
            best, best_sum = comb, s
    return best


def _brute_route(keys, N, G, keep, topn, k):
    gs = N // G
    if G > 1:
        gscore = []
        for q in range(G):
            grp = keys[q * gs:(q + 1) * gs]
            gscore.append(max(sum(c) for c in itertools.combinations(grp, topn)))
        kept = set(_best_subset(gscore, keep))
    else:
        kept = {0}
    cands = [e for e in range(N) if e // gs in kept]
    sel = _best_subset([keys[e] for e in cands], k)
    chosen = [cands[i] for i in sel]
    # slot order: key descending, then index ascending
    chosen.sort(key=lambda e: (-keys[e], e))
    return chosen, kept


@pytest.mark.parametrize("N,G,keep,topn,k", [
    (8, 2, 1, 2, 3), (12, 3, 2, 2, 4), (16, 4, 2, 2, 4), (16, 4, 1, 1, 2),
    (16, 2, 1, 2, 5), (8, 1, 1, 2, 4), (16, 4, 3, 2, 7)])
@pytest.mark.parametrize("score_fn", [oracle.SIGMOID, oracle.SOFTMAX])
def test_route_matches_bruteforce_with_ties(N, G, keep, topn, k, score_fn):
    rng = np.random.default_rng(N * 1000 + G * 100 + keep * 10 + k + score_fn)
    T = 40
    if score_fn == oracle.SOFTMAX:
        # key = logit: small integers, many ties
        logits = rng.integers(-3, 4, size=(T, N)).astype(np.float32)
        bias = None
        keys = logits.astype(np.float64)
    else:
        # every logit 0 -> score exactly 0.5; key = 0.5 + integer bias.
        # vary the bias per token by routing one token per call
        logits = np.zeros((T, N), np.float32)
        bias = None
        keys = None
    for t in range(T):
        if score_fn == oracle.SIGMOID:
            b = rng.integers(-2, 3, size=N).astype(np.float32)
            r = oracle.route(logits[t:t + 1], b, k, G, keep, topn, score_fn, 1, 1.0)
            kt = [0.5 + float(v) for v in b]
        else:
            r = oracle.route(logits[t:t + 1], None, k, G, keep, topn, score_fn, 1, 1.0)
            kt = list(keys[t])
        chosen, kept = _brute_route(kt, N, G, keep, topn, k)
        assert list(r["topk_idx"][0]) == chosen, (t, kt)
        assert set(np.nonzero(r["kept_groups"][0])[0]) == kept


# ----------------------------------------------------------------- exact-1 L_B

def test_uniform_softmax_routing_has_balance_loss_exactly_one():
    """Construction (i): every token puts logit 0 on 4 experts, -1000 on the
    rest; exp underflows to 0 so each chosen probability is exactly 1/4 and
    every expert is chosen 16 times."""
    T, N, k = 64, 16, 4
    logits = np.full((T, N), -1000.0, np.float32)
    for t in range(T):
        for j in range(k):
            logits[t, (4 * t + j) % N] = 0.0
    r = oracle.route(logits, None, k, 1, 1, 2, oracle.SOFTMAX, 0, 1.0)
    assert np.all(r["topk_gate"] == 0.25)
    d = oracle.dispatch(r["topk_idx"], r["topk_score"], N)
    assert np.all(d["counts"] == T * k // N)
    st = oracle.load_stats(logits, d["counts"], k, oracle.SOFTMAX)
    assert st["L_B"] == 1.0
    assert abs(st["z"] - math.log(4)) < 1e-12
    gold = json.load(open(os.path.join(GOLDEN, "st_moe_uniform_balance.json")))
    assert st["L_B"] == gold["L_B_uniform"]
    assert abs(float(np.sum(st["f"] * st["P"])) - 1.0 / N) < 1e-15


def test_uniform_grouped_sigmoid_routing_has_balance_loss_one():
    """Construction (ii): 16 experts in 4 groups of 4, keep 2, top-4, no bias.
    Token (a, b) sees the base vector rotated by a over groups and by b inside
    groups, so every expert is chosen equally often with the same multiset of
    scores."""
    N, G, k = 16, 4, 4
    v = np.array([0.9, -0.3, 0.5, 1.7, -1.1, 0.2, 1.3, -0.6,
                  0.05, 2.1, -1.9, 0.7, 1.05, -0.15, 0.35, -2.4], np.float32)
    rows = []
    for a in range(4):
        for b in range(4):
            rows.append([v[4 * ((q + a) % 4) + ((e + b) % 4)] for q in range(4) for e in range(4)])
    logits = np.array(rows, np.float32)
    r = oracle.route(logits, np.zeros(N, np.float32), k, G, 2, 2, oracle.SIGMOID, 1, 1.0)
    d = oracle.dispatch(r["topk_idx"], r["topk_score"], N)
    assert np.all(d["counts"] == d["counts"][0])
    st = oracle.load_stats(logits, d["counts"], k, oracle.SIGMOID)
    assert abs(st["L_B"] - 1.0) < 1e-12
    gs = N // G
    for t in range(logits.shape[0]):
        for e in r["topk_idx"][t]:
            assert r["kept_groups"][t, e // gs]


# ----------------------------------------------------------------- invariants

def _indep_kept_groups(keys, G, keep, topn):
    """Independent recomputation of the kept groups (numpy sort)."""
    T, N = keys.shape
    gs = N // G
    g = np.sort(keys.reshape(T, G, gs), axis=2)[:, :, ::-1][:, :, :topn]
    gsc = g[:, :, 0].copy()
    for j in range(1, topn):
        gsc = (gsc + g[:, :, j]).astype(np.float32)
    order = np.argsort(-gsc.astype(np.float64), axis=1, kind="stable")
    kept = np.zeros((T, G), bool)
    np.put_along_axis(kept, order[:, :keep], True, axis=1)
    return kept


@pytest.mark.parametrize("N,G,keep,k,fn,norm,scale", [
    (256, 8, 4, 8, oracle.SIGMOID, 1, 2.5),
    (64, 1, 1, 6, oracle.SOFTMAX, 0, 1.0),
    (16, 4, 2, 4, oracle.SIGMOID, 1, 1.0),
    (160, 8, 3, 6, oracle.SOFTMAX, 0, 1.0)])
def test_route_invariants_random(N, G, keep, k, fn, norm, scale):
    rng = np.random.default_rng(7)
    T = 300
    logits = (0.5 * rng.standard_normal((T, N))).astype(np.float32)
    bias = rng.uniform(-0.05, 0.05, N).astype(np.float32)
    r = oracle.route(logits, bias, k, G, keep, 2, fn, norm, scale)
    idx = r["topk_idx"]
    assert idx.min() >= 0 and idx.max() < N
    assert all(len(set(row)) == k for row in idx)
    # experts only from kept groups (recomputed independently)
    s = oracle.sigmoid32(logits) if fn == oracle.SIGMOID else None
    keys = (s + bias).astype(np.float32) if fn == oracle.SIGMOID else (logits + bias).astype(np.float32)
    if G > 1:
        kept = _indep_kept_groups(keys, G, keep, 2)
        assert np.array_equal(kept, r["kept_groups"])
        gs = N // G
        assert np.all(np.take_along_axis(kept, idx // gs, axis=1))
    # slots are in descending key order
    ksel = np.take_along_axis(keys, idx, axis=1)
    assert np.all(np.diff(ksel, axis=1) <= 0)
    # gates
    g = r["topk_gate"]
    if norm:
        np.testing.assert_allclose(g.sum(axis=1), scale, rtol=1e-12)
    else:
        # the fp32 softmax score (within its error bound of the fp64 one)
        ref = np.exp(logits.astype(np.float64) - logits.max(1, keepdims=True))
        ref /= ref.sum(1, keepdims=True)
        np.testing.assert_allclose(g, np.take_along_axis(ref, idx, 1) * scale, rtol=2e-6)
    # the bias changes the selection only: z and P do not depend on it
    r0 = oracle.route(logits, None, k, G, keep, 2, fn, norm, scale)
    np.testing.assert_array_equal(r0["lse"], r["lse"])
    d = oracle.dispatch(idx, r["topk_score"], N)
    st1 = oracle.load_stats(logits, d["counts"], k, fn)
    d0 = oracle.dispatch(r0["topk_idx"], r0["topk_score"], N)
    st0 = oracle.load_stats(logits, d0["counts"], k, fn)
    np.testing.assert_array_equal(st0["P"], st1["P"])
    assert st0["z"] == st1["z"]
    # the reported score is the unbiased score of the chosen expert
    s_all = s if fn == oracle.SIGMOID else oracle.softmax32(logits)
    np.testing.assert_array_equal(r["topk_score"], np.take_along_axis(s_all, idx, 1))
    if not norm:
        np.testing.assert_array_equal(g, r["topk_score"].astype(np.float64) * scale)


@pytest.mark.parametrize("fn", [oracle.SIGMOID, oracle.SOFTMAX])
def test_ungrouped_unbiased_topk_is_stable_argsort(fn):
    rng = np.random.default_rng(3)
    T, N, k = 200, 64, 6
    # distinct logits spaced far enough apart that sigmoid scores are distinct
    logits = np.stack([rng.permutation(N) for _ in range(T)]).astype(np.float32) * 0.05 - 1.5
    r = oracle.route(logits, None, k, 1, 1, 2, fn, 1, 1.0)
    ref = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(r["topk_idx"], ref)


def test_v3_group_shape_golden():
    """[GLR] §1: 256 experts in 8 groups of 32; keeping 4 groups leaves 128
    candidates, from which 8 are chosen."""
    gold = json.load(open(os.path.join(GOLDEN, "v3_group_limited_routing.json")))
    N, G, keep, k = gold["n_experts"], gold["n_groups"], gold["topk_groups"], gold["topk"]
    assert N // G == gold["group_size"] and keep * N // G == gold["candidates"]
    rng = np.random.default_rng(11)
    logits = (0.5 * rng.standard_normal((64, N))).astype(np.float32)
    r = oracle.route(logits, None, k, G, keep, 2, oracle.SIGMOID, 1, 2.5)
    assert np.all(r["kept_groups"].sum(1) == keep)
    n_cand = r["kept_groups"].sum(1) * (N // G)
    assert np.all(n_cand == gold["candidates"])
    assert r["topk_idx"].shape[1] == gold["topk"]


# ------------------------------------------------- v2 device-limited routing

def _walk_down_devices(keys, gs, M, k):
    """Device-limited routing as the DeepSeek-v2 passage words it: walk the
    experts from the highest key down, collecting the devices they sit on
    until M distinct devices are found; then take the top k keys among all
    experts of those devices (ties: lower index first)."""
    order = sorted(range(len(keys)), key=lambda e: (-keys[e], e))
    devices = []
    for e in order:
        d = e // gs
        if d not in devices:
            devices.append(d)
        if len(devices) == M:
            break
    cands = [e for e in range(len(keys)) if e // gs in devices]
    cands.sort(key=lambda e: (-keys[e], e))
    return cands[:k], set(devices)


@pytest.mark.parametrize("N,G,M,k", [(16, 4, 2, 3), (24, 8, 3, 6), (160, 8, 3, 6), (32, 8, 1, 4)])
@pytest.mark.parametrize("score_fn", [oracle.SIGMOID, oracle.SOFTMAX])
def test_device_limited_routing_is_top1_group_score(N, G, M, k, score_fn):
    # "DeepSeek MoE：从v1到v3的演进" §DeepSeek-v2 (device-limited routing):
    # the groups kept by a top-1 group score are the devices the walk-down
    # collects, with integer-valued logits so that ties occur
    rng = np.random.default_rng(7 * N + M + score_fn)
    T = 60
    logits = rng.integers(-4, 5, size=(T, N)).astype(np.float32)
    bias = None
    if score_fn == oracle.SIGMOID:
        bias = (rng.integers(-2, 3, size=N) * 0.25).astype(np.float32)
    r = oracle.route(logits, bias, k, n_groups=G, topk_groups=M, group_topn=1,
                     score_fn=score_fn, norm_topk=0)
    gs = N // G
    for t in range(T):
        if score_fn == oracle.SIGMOID:
            s = oracle.sigmoid32(logits[t])
            keys = [float(np.float32(s[e]) + np.float32(bias[e])) for e in range(N)]
        else:
            keys = [float(v) for v in logits[t]]
        chosen, devs = _walk_down_devices(keys, gs, M, k)
        assert list(r["topk_idx"][t]) == chosen, t
        assert set(np.nonzero(r["kept_groups"][t])[0]) == devs
        # fan-out bound: a token reaches at most M devices
        assert len({e // gs for e in r["topk_idx"][t]}) <= M
