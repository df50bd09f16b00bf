"""Pins for the oracle's fp32 softmax (the v1/v2 gate's score and the order
device-level dropping follows, [EVO] §ST-MoE p_i(x) and §DeepSeek-v2).

The definition fixes every rounding step so that the GPU reproduces it bit
for bit; these tests tie it to facts outside that definition:
  * the fp64 softmax, within the error bound of the fp32 steps;
  * the pinned fp32 sigmoid: for two logits (l, 0) with l <= 0 the second
    score is 1 / (1 + e^l) formed by the same steps, i.e. sigmoid32(-l)
    exactly;
  * exact values: equal logits over a power-of-two count give exactly 1/N;
    a logit more than 64 above all others gets exactly 1 and the rest 0;
  * shift invariance when the shift is exact.
"""
import numpy as np
import pytest

import oracle


def _softmax64(l: np.ndarray) -> np.ndarray:
    l = l.astype(np.float64)
    e = np.exp(l - l.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("N", [2, 16, 64, 160, 256])
def test_softmax32_within_bound_of_fp64(N):
    rng = np.random.default_rng(N)
    l = (rng.standard_normal((400, N)) * rng.choice([0.5, 3.0, 12.0], size=(400, 1))).astype(np.float32)
    got = oracle.softmax32(l).astype(np.float64)
    ref = _softmax64(l)
    # per score: the rounded shift x = fl(l - m) (half an ulp of x, i.e. a
    # relative error of up to |x| u in e^x), the exponential (<= 2 ulp, as
    # the pinned sigmoid's), the pairwise sum over 256 slots (8 levels) and
    # the divide
    u = 2.0 ** -24
    x = np.abs(l.astype(np.float64) - l.max(axis=1, keepdims=True))
    big = ref > 1e-20  # terms the definition may set to 0 are below e^-64
    rel = np.abs(got[big] - ref[big]) / ref[big]
    bound = (x[big] + 2 + 8 + 1 + 1) * u
    assert np.all(rel <= bound), np.max(rel / bound)
    assert np.all(got[~big] <= 1e-20)
    np.testing.assert_allclose(got.sum(axis=1), 1.0, rtol=0, atol=(8 + 4) * u)


def test_softmax32_two_logits_is_the_pinned_sigmoid():
    # logits (l, 0), l <= 0: m = 0, E = (e^l, 1), S = fl(e^l + 1) (the other
    # 254 slots add zeros), s_1 = 1 / fl(1 + e^l) = sigmoid32(-l)
    l = -np.concatenate([np.linspace(0, 64, 20001, dtype=np.float32),
                         np.arange(0, 0x42800000, 9973, dtype=np.uint32).view(np.float32)])
    l = l[l >= -64]
    pair = np.stack([l, np.zeros_like(l)], axis=1)
    got = oracle.softmax32(pair)
    np.testing.assert_array_equal(got[:, 1], oracle.sigmoid32(-l))
    # s_0 = e^l / (1 + e^l) is then the complement within rounding
    assert np.max(np.abs(got[:, 0].astype(np.float64) + got[:, 1] - 1.0)) <= 2 ** -23


@pytest.mark.parametrize("N", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_softmax32_equal_logits_power_of_two_is_exact(N):
    for c in (0.0, -3.25, 7.5, 1e4):
        s = oracle.softmax32(np.full((1, N), c, np.float32))
        assert np.all(s == np.float32(1.0 / N)), (N, c, s[0, :4])


def test_softmax32_far_below_the_maximum_is_zero():
    l = np.array([[0.0, -64.5, -100.0, -1e30, 5.0]], np.float32)  # gaps > 64 from 5.0
    l[0, 0] = 5.0 - 64.25
    s = oracle.softmax32(l)[0]
    assert s[4] == 1.0 and np.all(s[:4] == 0.0)
    # a term exactly 64 below the maximum is kept
    s2 = oracle.softmax32(np.array([[0.0, -64.0]], np.float32))[0]
    assert s2[1] > 0 and s2[0] == 1.0  # 1 + 1.6e-28 rounds to 1


def test_softmax32_exact_shift_invariance():
    rng = np.random.default_rng(7)
    # logits on a 2^-8 grid and integer shifts: l + c is exact, so l - m is
    # unchanged and every score must be bit-identical
    l = (np.round(rng.standard_normal((200, 64)) * 256) / 256).astype(np.float32)
    for c in (1.0, -37.0, 1024.0):
        np.testing.assert_array_equal(oracle.softmax32(l + np.float32(c)), oracle.softmax32(l))


def test_softmax32_rejects_more_than_256_experts():
    with pytest.raises(ValueError):
        oracle.softmax32(np.zeros((1, 257), np.float32))
