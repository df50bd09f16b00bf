"""Pins for the oracle's fp32 sigmoid and router logits.

The sigmoid is pinned against the fp64 definition 1/(1+e^-l) (ulp error on a
dense sweep), against exact special values, and by monotonicity; the logits
against numpy's fp64 matmul (the step is a plain matrix product).
"""
import numpy as np
import pytest

import oracle


def _ulp_dist(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in units of the last place between fp32 arrays (same sign)."""
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def _sweep():
    # every 37th fp32 bit pattern with |l| <= 87, plus a dense grid near 0
    pos = np.arange(0, 0x42AE0000, 37, dtype=np.uint32).view(np.float32)
    pos = pos[np.isfinite(pos)]
    grid = np.linspace(-12, 12, 200001, dtype=np.float32)
    return np.concatenate([pos, -pos, grid])


def test_sigmoid32_within_2ulp_of_fp64_definition():
    l = _sweep()
    got = oracle.sigmoid32(l)
    ref = (1.0 / (1.0 + np.exp(-l.astype(np.float64)))).astype(np.float32)
    # below fp32's normal range the comparison is meaningless: restrict to
    # results that are normal numbers
    ok = ref >= np.float32(1.2e-38)
    d = _ulp_dist(got[ok], ref[ok])
    assert d.max() <= 2, f"max ulp error {d.max()} at l={l[ok][d.argmax()]}"


def test_sigmoid32_special_values():
    s = oracle.sigmoid32(np.array([0.0, -0.0, 87.0, 200.0, 1e30], np.float32))
    assert s[0] == np.float32(0.5) and s[1] == np.float32(0.5)
    assert s[2] == 1.0 and s[3] == 1.0 and s[4] == 1.0
    # saturation below -87 keeps the result a positive normal number
    lo = oracle.sigmoid32(np.array([-87.0, -100.0, -1e30], np.float32))
    assert np.all(lo == lo[0]) and lo[0] > 0 and lo[0] >= np.float32(1.17549435e-38)


def test_sigmoid32_monotone_and_symmetric():
    l = np.sort(_sweep())
    s = oracle.sigmoid32(l)
    assert np.all(np.diff(s) >= 0), "sigmoid must be non-decreasing"
    # sigma(l) + sigma(-l) = 1 up to rounding of the two evaluations
    m = np.abs(l) < 20
    tot = s[m].astype(np.float64) + oracle.sigmoid32(-l[m]).astype(np.float64)
    assert np.max(np.abs(tot - 1.0)) < 2.5e-7


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (test-side helper)."""
    u = a.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_router_logits_match_numpy_matmul(dt):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((37, 96)).astype(np.float32)
    wg = (0.02 * rng.standard_normal((20, 96))).astype(np.float32)
    if dt == "bf16":
        xb, wb = _bf16_bits(x), _bf16_bits(wg)
        got = oracle.router_logits(xb, wb)
        ref = _bf16_to_f64(xb) @ _bf16_to_f64(wb).T
    else:
        got = oracle.router_logits(x, wg)
        ref = x.astype(np.float64) @ wg.astype(np.float64).T
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
