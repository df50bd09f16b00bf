"""Pins for the oracle's sequence-wise and device-level balance statistics
("DeepSeek MoE：从v1到v3的演进" §DeepSeek-v3 sequence-wise balance loss and
§DeepSeek-v1 device-level balance loss; the pages print no formula for
either, so both are the expert-level f, P, L_B of §ST-MoE taken per sequence,
or per group of experts).

Pins: closed forms (a uniformly routed sequence with equal scores has L = 1;
a sequence whose tokens all pick the same k experts with all their score
mass has L = N / k), segmentation (two such sequences in one batch keep
their own values), count conservation against the batch histogram,
token-order invariance, empty sequences; device level: one expert per group
gives the expert-level L_B, one group gives 1, all load and score mass on one
group gives G."""
import numpy as np
import pytest

import oracle


def _uniform_block(Tq, N, k, base_rot):
    # token t picks experts (t*k + j + base_rot) mod N: every expert exactly
    # Tq*k/N times when N divides Tq*k
    return np.array([[(t * k + j + base_rot) % N for j in range(k)] for t in range(Tq)],
                    np.int32)


def test_uniform_sequence_has_unit_loss_and_concentrated_has_n_over_k():
    N, k = 16, 4
    Tu, Tc = 32, 24
    idx_u = _uniform_block(Tu, N, k, 0)
    logit_u = np.zeros((Tu, N), np.float32)            # softmax: equal mass on every expert
    chosen = [3, 7, 8, 12]
    idx_c = np.tile(np.array(chosen, np.int32), (Tc, 1))
    logit_c = np.full((Tc, N), -60.0, np.float32)
    logit_c[:, chosen] = 60.0                          # softmax mass ~1 on the chosen four
    logits = np.concatenate([logit_u, logit_c])
    idx = np.concatenate([idx_u, idx_c])
    cu = [0, Tu, Tu + Tc]
    st = oracle.seq_load_stats(logits, idx, cu, k, oracle.SOFTMAX)
    assert st["L"][0] == pytest.approx(1.0, abs=1e-12)
    assert st["L"][1] == pytest.approx(N / k, abs=1e-12)
    assert st["L_mean"] == pytest.approx((1.0 + N / k) / 2, abs=1e-12)
    np.testing.assert_allclose(st["f"][0], np.full(N, 1.0 / N), atol=1e-15)
    np.testing.assert_allclose(st["P"][1][chosen], np.full(k, 1.0 / k), atol=1e-12)
    # the whole batch mixes both, so its L_B lies strictly between
    counts = np.bincount(idx.ravel(), minlength=N).astype(np.int32)
    lb = oracle.load_stats(logits, counts, k, oracle.SOFTMAX)["L_B"]
    assert 1.0 < lb < N / k


def test_sigmoid_concentrated_sequence():
    N, k, Tq = 32, 8, 10
    chosen = list(range(0, 32, 4))
    idx = np.tile(np.array(chosen, np.int32), (Tq, 1))
    logits = np.full((Tq, N), -40.0, np.float32)
    logits[:, chosen] = 40.0                           # sigmoid32: 1.0 and ~4e-18
    st = oracle.seq_load_stats(logits, idx, [0, Tq], k, oracle.SIGMOID)
    assert st["L"][0] == pytest.approx(N / k, rel=1e-12)


@pytest.mark.parametrize("fn", [oracle.SIGMOID, oracle.SOFTMAX])
def test_counts_conserved_and_token_order_invariant(fn):
    rng = np.random.default_rng(5 + fn)
    T, N, k = 120, 24, 3
    idx = np.stack([rng.choice(N, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    logits = rng.normal(size=(T, N)).astype(np.float32)
    cu = [0, 17, 17, 60, 61, 120]                      # includes an empty sequence
    st = oracle.seq_load_stats(logits, idx, cu, k, fn)
    Tq = np.diff(cu)
    # sum over sequences of k * T_q * f_q reproduces the batch histogram exactly
    rebuilt = sum(k * Tq[q] * st["f"][q] for q in range(len(Tq)))
    np.testing.assert_allclose(rebuilt, np.bincount(idx.ravel(), minlength=N), atol=1e-9)
    # P of every non-empty sequence is a distribution
    for q in range(len(Tq)):
        if Tq[q]:
            assert st["P"][q].sum() == pytest.approx(1.0, abs=1e-12)
    # empty sequence: zeros, and excluded from the mean
    assert st["L"][1] == 0.0 and not st["f"][1].any() and not st["P"][1].any()
    nonempty = [q for q in range(len(Tq)) if Tq[q]]
    assert st["L_mean"] == pytest.approx(np.mean(st["L"][nonempty]), abs=1e-15)
    # reversing the tokens inside sequence 2 changes nothing
    perm = np.arange(T)
    perm[17:60] = perm[17:60][::-1]
    st2 = oracle.seq_load_stats(logits[perm], idx[perm], cu, k, fn)
    np.testing.assert_allclose(st2["L"], st["L"], rtol=1e-12)
    np.testing.assert_allclose(st2["P"], st["P"], rtol=1e-12, atol=1e-15)


def test_seq_stats_reject_bad_boundaries():
    logits = np.zeros((4, 8), np.float32)
    idx = np.zeros((4, 2), np.int32)
    idx[:, 1] = 1
    for cu in ([0, 3], [1, 4], [0, 3, 2, 4]):
        with pytest.raises(ValueError):
            oracle.seq_load_stats(logits, idx, cu, 2)


@pytest.mark.parametrize("fn", [oracle.SIGMOID, oracle.SOFTMAX])
def test_group_stats_with_one_expert_per_group_is_expert_level(fn):
    rng = np.random.default_rng(11 + fn)
    T, N, k = 90, 16, 4
    idx = np.stack([rng.choice(N, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    logits = rng.normal(size=(T, N)).astype(np.float32)
    counts = np.bincount(idx.ravel(), minlength=N).astype(np.int32)
    st = oracle.load_stats(logits, counts, k, fn)
    g = oracle.group_load_stats(st["f"], st["P"], N)
    assert g["L_dev"] == pytest.approx(st["L_B"], rel=1e-14)
    one = oracle.group_load_stats(st["f"], st["P"], 1)
    assert one["L_dev"] == pytest.approx(1.0, abs=1e-12)
    g4 = oracle.group_load_stats(st["f"], st["P"], 4)
    np.testing.assert_allclose(g4["F"], st["f"].reshape(4, 4).sum(1), rtol=1e-15)
    assert g4["F"].sum() == pytest.approx(1.0) and g4["P"].sum() == pytest.approx(1.0)


def test_group_stats_closed_forms():
    N, G = 12, 3
    f = np.full(N, 1.0 / N)
    assert oracle.group_load_stats(f, f, G)["L_dev"] == pytest.approx(1.0, abs=1e-15)
    # all assignments and all score mass on group 1
    f = np.zeros(N)
    f[4:8] = 0.25
    P = np.zeros(N)
    P[4:8] = [0.1, 0.2, 0.3, 0.4]
    assert oracle.group_load_stats(f, P, G)["L_dev"] == pytest.approx(G, abs=1e-15)
