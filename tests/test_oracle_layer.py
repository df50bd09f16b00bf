"""Pins for the oracle's expert FFN, layer output and statistics.

Special cases that reduce to plain fp64 numpy matrix products (one expert and
k = 1 is a SwiGLU MLP; k = 0 is the shared expert alone; k = N without
capacity is a dense mixture), packed shared experts equal to separate ones,
and the closed forms of the statistics.
"""
import math

import numpy as np
import pytest

import oracle


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _np_swiglu(x, w13, w2):
    I = w13.shape[0] // 2
    a = w13[:I].astype(np.float64) @ x.astype(np.float64)
    u = w13[I:].astype(np.float64) @ x.astype(np.float64)
    return w2.astype(np.float64) @ (_silu(a) * u)


def _bf16_bits(a):
    u = a.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_swiglu_row_matches_numpy(dt):
    rng = np.random.default_rng(2)
    H, I = 48, 40
    x = rng.standard_normal(H).astype(np.float32)
    w13 = (0.2 * rng.standard_normal((2 * I, H))).astype(np.float32)
    w2 = (0.2 * rng.standard_normal((H, I))).astype(np.float32)
    if dt == "bf16":
        x, w13, w2 = _bf16_bits(x), _bf16_bits(w13), _bf16_bits(w2)
        ref = _np_swiglu(_bf16_f32(x), _bf16_f32(w13), _bf16_f32(w2))
    else:
        ref = _np_swiglu(x, w13, w2)
    np.testing.assert_allclose(oracle.swiglu_row(x, w13, w2), ref, rtol=1e-12, atol=1e-14)


def test_single_expert_top1_is_plain_swiglu_mlp():
    """N = 1, k = 1, normalised gate = 1, no shared expert."""
    rng = np.random.default_rng(4)
    H, I, T = 32, 24, 5
    x = rng.standard_normal((T, H)).astype(np.float32)
    w13 = (0.3 * rng.standard_normal((1, 2 * I, H))).astype(np.float32)
    w2 = (0.3 * rng.standard_normal((1, H, I))).astype(np.float32)
    logits = rng.standard_normal((T, 1)).astype(np.float32)
    r = oracle.route(logits, None, 1, 1, 1, 1, oracle.SIGMOID, 1, 1.0)
    assert np.all(r["topk_gate"] == 1.0)
    for t in range(T):
        out = oracle.token_output(x[t], [w13[0]], [w2[0]], r["topk_gate"][t], None, None, 0, 0, I)
        np.testing.assert_allclose(out, _np_swiglu(x[t], w13[0], w2[0]), rtol=1e-12, atol=1e-14)


def test_no_routed_experts_is_shared_only_and_packing_is_sum_of_experts():
    rng = np.random.default_rng(6)
    H, I_sh, n_sh = 32, 16, 2
    x = rng.standard_normal(H).astype(np.float32)
    sep13 = [(0.3 * rng.standard_normal((2 * I_sh, H))).astype(np.float32) for _ in range(n_sh)]
    sep2 = [(0.3 * rng.standard_normal((H, I_sh))).astype(np.float32) for _ in range(n_sh)]
    # packed layout: all gate rows, then all up rows; down columns side by side
    ws13 = np.concatenate([w[:I_sh] for w in sep13] + [w[I_sh:] for w in sep13], axis=0)
    ws2 = np.concatenate(sep2, axis=1)
    out = oracle.token_output(x, [], [], np.zeros(0), ws13, ws2, n_sh, I_sh, 8)
    ref = sum(_np_swiglu(x, a, b) for a, b in zip(sep13, sep2))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_dense_mixture_k_equals_N():
    """k = N, softmax gates without renormalisation, no capacity: the layer is
    sum_e p_e E_e(x) + shared(x)."""
    rng = np.random.default_rng(8)
    H, I, N, T = 24, 16, 6, 4
    x = rng.standard_normal((T, H)).astype(np.float32)
    w13 = (0.3 * rng.standard_normal((N, 2 * I, H))).astype(np.float32)
    w2 = (0.3 * rng.standard_normal((N, H, I))).astype(np.float32)
    ws13 = (0.3 * rng.standard_normal((2 * I, H))).astype(np.float32)
    ws2 = (0.3 * rng.standard_normal((H, I))).astype(np.float32)
    logits = rng.standard_normal((T, N)).astype(np.float32)
    r = oracle.route(logits, None, N, 1, 1, 2, oracle.SOFTMAX, 0, 1.0)
    d = oracle.dispatch(r["topk_idx"], r["topk_score"], N, 0)
    assert d["offsets"][-1] == T * N
    # the gates are the fp32 softmax scores (pinned against the fp64 softmax
    # in test_oracle_softmax.py); the mixture identity is checked on them
    p = oracle.softmax32(logits).astype(np.float64)
    p64 = np.exp(logits.astype(np.float64) - logits.max(1, keepdims=True))
    np.testing.assert_allclose(p, p64 / p64.sum(1, keepdims=True), rtol=2e-6)
    for t in range(T):
        sel = r["topk_idx"][t]
        out = oracle.token_output(x[t], [w13[e] for e in sel], [w2[e] for e in sel],
                                  r["topk_gate"][t], ws13, ws2, 1, I, I)
        ref = _np_swiglu(x[t], ws13, ws2) + sum(p[t, e] * _np_swiglu(x[t], w13[e], w2[e]) for e in range(N))
        np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)


def test_dropped_slot_contributes_nothing():
    rng = np.random.default_rng(9)
    H, I = 16, 8
    x = rng.standard_normal(H).astype(np.float32)
    a13 = (0.3 * rng.standard_normal((2 * I, H))).astype(np.float32)
    a2 = (0.3 * rng.standard_normal((H, I))).astype(np.float32)
    out = oracle.token_output(x, [a13, None], [a2, None], np.array([0.7, 0.3]), None, None, 0, 0, I)
    np.testing.assert_allclose(out, 0.7 * _np_swiglu(x, a13, a2), rtol=1e-12)


# ----------------------------------------------------------------- statistics

def test_constant_logits_z_loss_closed_form():
    T, N, c = 10, 32, 0.75
    logits = np.full((T, N), c, np.float32)
    counts = np.full(N, T * 2 // N, np.int32)
    for fn in (oracle.SIGMOID, oracle.SOFTMAX):
        st = oracle.load_stats(logits, counts, 2, fn)
        assert abs(st["z"] - (c + math.log(N))) < 1e-12
        assert abs(st["z_sq"] - (c + math.log(N)) ** 2) < 1e-11


def test_zero_logits_softmax_gives_uniform_P():
    T, N = 7, 64
    st = oracle.load_stats(np.zeros((T, N), np.float32), np.zeros(N, np.int32), 4, oracle.SOFTMAX)
    assert np.all(st["P"] == 1.0 / N)


def test_stats_normalisation_and_softmax_P_is_mean_probability():
    rng = np.random.default_rng(12)
    T, N, k = 100, 16, 3
    logits = rng.standard_normal((T, N)).astype(np.float32)
    r = oracle.route(logits, None, k, 1, 1, 2, oracle.SOFTMAX, 0, 1.0)
    d = oracle.dispatch(r["topk_idx"], r["topk_score"], N)
    st = oracle.load_stats(logits, d["counts"], k, oracle.SOFTMAX)
    assert abs(st["f"].sum() - 1.0) < 1e-12 and abs(st["P"].sum() - 1.0) < 1e-12
    p = np.exp(logits.astype(np.float64) - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(st["P"], p.mean(0), rtol=1e-12)
    lse = np.log(np.exp(logits.astype(np.float64)).sum(1))
    assert abs(st["z"] - lse.mean()) < 1e-12
    np.testing.assert_allclose(r["lse"], lse, rtol=1e-12)
    # sigmoid P is each expert's share of the total score mass
    st2 = oracle.load_stats(logits, d["counts"], k, oracle.SIGMOID)
    s = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    np.testing.assert_allclose(st2["P"], s.sum(0) / s.sum(), rtol=1e-6)


# ----------------------------------------------------------------- bias update

def test_bias_update_sign_rule():
    counts = np.array([3, 1, 2, 2], np.int32)  # mean 2
    b = np.array([0.5, -0.25, 0.0, 1.0], np.float32)
    nb = oracle.bias_update(counts, b, 0.125)
    np.testing.assert_array_equal(nb, np.array([0.375, -0.125, 0.0, 1.0], np.float32))


def test_bias_update_reduces_imbalance_on_a_fixed_batch():
    rng = np.random.default_rng(13)
    T, N, k = 512, 32, 4
    logits = (0.5 * rng.standard_normal((T, N)) + np.linspace(-1, 1, N)).astype(np.float32)
    b = np.zeros(N, np.float32)
    ratios = []
    for _ in range(60):
        r = oracle.route(logits, b, k, 1, 1, 2, oracle.SIGMOID, 1, 1.0)
        c = np.bincount(r["topk_idx"].ravel(), minlength=N)
        ratios.append(c.max() / c.mean())
        b = oracle.bias_update(c.astype(np.int32), b, 0.01)
    assert ratios[-1] < 0.5 * ratios[0]


def test_combine_matches_numpy_gather_sum():
    rng = np.random.default_rng(14)
    T, H, k, M = 9, 12, 3, 30
    y = rng.standard_normal((M, H)).astype(np.float32)
    ysh = rng.standard_normal((T, H)).astype(np.float32)
    inv = rng.permutation(M)[:T * k].reshape(T, k).astype(np.int32)
    inv[2, 1] = -1
    inv[5, :] = -1
    g = rng.random((T, k))
    out = oracle.combine(y, ysh, inv, g)
    ref = ysh.astype(np.float64).copy()
    for t in range(T):
        for j in range(k):
            if inv[t, j] >= 0:
                ref[t] += g[t, j] * y[inv[t, j]].astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.combine(y, None, inv, g), ref - ysh, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fn", [oracle.SIGMOID, oracle.SOFTMAX])
def test_combine_of_expert_rows_equals_token_output(fn):
    """The layer computed the way the GPU path factors it -- dispatch, one
    SwiGLU row per kept (token, expert) assignment in the dispatch's row
    order, the shared expert per token, then the combine -- equals the
    per-token definition (shared output plus gate-weighted routed outputs,
    dropped slots contributing nothing).  The rows are rounded to fp32 once
    before the combine, hence the 1e-6 tolerance."""
    rng = np.random.default_rng(15)
    T, H, I, N, k, C = 12, 16, 8, 6, 2, 3
    x = rng.standard_normal((T, H)).astype(np.float32)
    w13 = (0.3 * rng.standard_normal((N, 2 * I, H))).astype(np.float32)
    w2 = (0.3 * rng.standard_normal((N, H, I))).astype(np.float32)
    ws13 = (0.3 * rng.standard_normal((2 * I, H))).astype(np.float32)
    ws2 = (0.3 * rng.standard_normal((H, I))).astype(np.float32)
    logits = rng.standard_normal((T, N)).astype(np.float32)
    r = oracle.route(logits, None, k, 1, 1, 2, fn, 1, 1.5)
    d = oracle.dispatch(r["topk_idx"], r["topk_score"], N, C)
    assert d["n_dropped"] > 0
    M = int(d["offsets"][-1])
    seg = np.searchsorted(d["offsets"], np.arange(M), side="right") - 1
    y = np.stack([oracle.swiglu_row(x[d["row_token"][q]], w13[seg[q]], w2[seg[q]])
                  for q in range(M)]).astype(np.float32)
    ysh = np.stack([oracle.swiglu_row(x[t], ws13, ws2) for t in range(T)]).astype(np.float32)
    got = oracle.combine(y, ysh, d["inv_row"], r["topk_gate"])
    for t in range(T):
        keep = d["inv_row"][t] >= 0
        sel = r["topk_idx"][t]
        ref = oracle.token_output(x[t], [w13[e] if kp else None for e, kp in zip(sel, keep)],
                                  [w2[e] if kp else None for e, kp in zip(sel, keep)],
                                  r["topk_gate"][t], ws13, ws2, 1, I, I)
        err = np.max(np.abs(got[t] - ref)) / np.max(np.abs(ref))
        assert err <= 1e-6, (t, err)
