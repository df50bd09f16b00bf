"""Host-side logic that the GPU tests and the benchmark rely on, checked on
the CPU: the stratified sample of tokens used for full-size parity, and the
digest of the gfx950 code object that keys the committed counter records."""
import os

import numpy as np
import pytest

import oracle
from routing_expert_ffn_sigmoid_amd import workloads

import gpu_common

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _skewed_dispatch(T, N, k, capacity, seed):
    """A routing with very uneven expert loads (some experts over 512 rows),
    dispatched by the oracle."""
    rng = np.random.default_rng(seed)
    pop = rng.zipf(1.3, size=N).astype(np.float64)
    pop /= pop.sum()
    idx = np.stack([rng.choice(N, size=k, replace=False, p=pop) for _ in range(T)]).astype(np.int32)
    score = rng.random((T, k)).astype(np.float32)
    return oracle.dispatch(idx, score, N, capacity)


@pytest.mark.parametrize("capacity", [0, 700])
def test_stratified_sample_reaches_every_tile(capacity):
    wl = workloads.V3_PREFILL.with_(T=4000, N=32, k=4, n_groups=4, topk_groups=2,
                                    capacity=capacity)
    d = _skewed_dispatch(wl.T, wl.N, wl.k, capacity, seed=3)
    toks = gpu_common.stratified_tokens(wl, d, min_count=300)
    tset = set(toks)
    assert toks == sorted(tset) and len(toks) >= 300
    off, rt = d["offsets"], d["row_token"]
    split = 0
    for e in range(wl.N):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        mtc = -(-(b - a) // 256)
        split += mtc > 1
        rpt = (-(-(b - a) // mtc) + 15) & ~15
        for m in range(mtc):
            r0 = a + m * rpt
            if r0 < b:
                # the first and the last row of every balanced row tile
                assert int(rt[r0]) in tset and int(rt[min(r0 + rpt, b) - 1]) in tset
    assert split > 0  # the routing does split experts over several tiles
    for r0 in range(0, wl.T, 256):  # shared expert: rows are tokens in order
        assert r0 in tset and min(r0 + 255, wl.T - 1) in tset
    dropped = np.nonzero((d["inv_row"] < 0).any(axis=1))[0]
    assert (d["n_dropped"] > 0) == (capacity > 0)
    assert set(dropped[:64].tolist()) <= tset


def test_code_object_digest_of_the_built_library():
    bench = pytest.importorskip("bench")
    if not os.path.exists(bench.LIB_PATH):
        pytest.skip("libmoe.so not built")
    d = bench.code_object_digest("ffn_pp_kernel")
    assert isinstance(d, str) and len(d) == 16 and int(d, 16) >= 0
    # another translation unit's code object has its own digest
    r = bench.code_object_digest("route_kernel")
    assert r is not None and r != d
    assert bench.code_object_digest("no_such_kernel_name") is None


def test_row_rel_l2_flags_one_bad_row_and_nonzero_zero_rows():
    from gpu_common import normwise, row_rel_l2
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((4096, 64))
    got = ref * (1 + 1e-3 * rng.standard_normal(ref.shape))
    got[17] *= 1.05                       # one row 5 % off
    assert normwise(got, ref)[1] < 5e-3   # the block norm does not see it
    rows = row_rel_l2(got, ref)
    assert int(np.argmax(rows)) == 17 and rows[17] > 4e-2
    ref[5] = 0.0
    got[5] = 0.0
    assert row_rel_l2(got, ref)[5] == 0.0
    got[5, 3] = 1e-30
    assert np.isinf(row_rel_l2(got, ref)[5])
