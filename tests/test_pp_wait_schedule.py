"""Model of the ping-pong grouped GEMM's per-wave memory-instruction order
and its vmcnt waits (grouped_ffn.hip, ffn_pp_kernel / pp_tile), checked over
random sequences of tiles: at every wait, the loads of the stage the next
LDS reads need have completed (vector-memory instructions of a wave complete
in issue order, so vmcnt(N) completes all but the newest N), and each wait
constant plus one would leave a needed load in flight.

The order modelled (one wave; NA = ceil(4 * NMBW / 8) activation loads per
pair of k-steps, 2 weight loads per k-step, 1 row_index load, S epilogue
stores: 8 in the gate/up kernel, 16 in the down kernel):
  first tile:  W(0), A(0,1) (4 loads), W(1), W(2); wait vmcnt(2)
  step k:      k + 3 < nk: A(k+2,k+3) if k even, R at k = nk-4, W(k+3)
               otherwise:  W'(0) | A'(0,1) (4 loads), W'(1) | W'(2)
  after a tile: S stores
  waits after step k: 4 + NA + S (k = 0); 4 + NA (even) / 4 (odd) in the
  middle; 4 + NA + 1, 5, 8, 4 in the last four steps; vmcnt(4) before the
  row_index entries are read at the start of step nk - 2.
"""
import random

import pytest

STORES = {"gate_up": 8, "down": 16}


def kernel_wait(k, nk, na, stores):
    """The constant the kernel waits with after step k."""
    if k == 0:
        return 4 + na + stores
    if k < nk - 4:
        return 4 + na if k % 2 == 0 else 4
    return {nk - 4: 4 + na + 1, nk - 3: 5, nk - 2: 8, nk - 1: 4}[k]


def run(tiles, stores, delta=None):
    """tiles: [(nk, nmbw)]; stores: epilogue stores per tile.  delta:
    (tile, k, d) adds d to one wait.  Returns the list of waits that leave a
    needed load in flight."""
    ops = []       # (tag, tile)
    done = 0
    bad = []

    def issue(tag, ti, n):
        ops.extend([(tag, ti)] * n)

    def wait(n, need, where):
        nonlocal done
        done = max(done, len(ops) - n)
        for nd in need:
            idx = [i for i, o in enumerate(ops) if o == nd]
            assert idx, (where, nd)
            if max(idx) >= done:
                bad.append((where, nd))

    def stage(ti, j):
        return {(f"W{j}", ti), (f"A{j - j % 2}", ti)}

    issue("W0", 0, 2); issue("A0", 0, 4); issue("W1", 0, 2); issue("W2", 0, 2)
    wait(2, stage(0, 0) | {("W1", 0)}, "prologue")
    for ti, (nk, nmbw) in enumerate(tiles):
        na = (4 * nmbw + 7) // 8
        for k in range(nk):
            if k + 3 < nk:
                if k % 2 == 0:
                    issue(f"A{k + 2}", ti, na)
                if k == nk - 4:
                    issue("R", ti + 1, 1)
                issue(f"W{k + 3}", ti, 2)
            else:
                j = k + 3 - nk
                if j == 0:
                    issue("W0", ti + 1, 2)
                elif j == 1:
                    issue("A0", ti + 1, 4)
                    issue("W1", ti + 1, 2)
                else:
                    issue("W2", ti + 1, 2)
            n = kernel_wait(k, nk, na, stores)
            if delta and delta[:2] == (ti, k):
                n += delta[2]
            if k + 1 < nk:
                need = stage(ti, k + 1)
            elif ti + 1 < len(tiles):
                need = stage(ti + 1, 0)
            else:
                need = set()
            wait(n, need, (ti, k))
            if k == nk - 3:  # start of step nk - 2: the row_index entries
                wait(4 + (delta[2] if delta and delta[:2] == (ti, "R") else 0),
                     {("R", ti + 1)}, (ti, "R"))
        issue("S", ti, stores)
    return bad


def random_tiles(rng):
    return [(4 * rng.choice([2, 3, 5, 16, 56]), rng.randint(1, 8))
            for _ in range(rng.randint(1, 4))]


@pytest.mark.parametrize("kernel", sorted(STORES))
def test_every_wait_covers_the_next_stage(kernel):
    rng = random.Random(1)
    for _ in range(500):
        tiles = random_tiles(rng)
        assert run(tiles, STORES[kernel]) == [], tiles


@pytest.mark.parametrize("k_of", [lambda nk: 0, lambda nk: 1, lambda nk: 2, lambda nk: nk - 4,
                                  lambda nk: nk - 3, lambda nk: nk - 2, lambda nk: nk - 1])
@pytest.mark.parametrize("kernel", sorted(STORES))
def test_each_wait_is_tight(k_of, kernel):
    """One more allowed in flight at any of the distinct waits leaves a
    needed load outstanding: the constants are exact, not merely safe."""
    tiles = [(64, 8), (224, 6), (32, 3)]
    k = k_of(tiles[1][0])
    assert run(tiles, STORES[kernel], delta=(1, k, +1)) != []


@pytest.mark.parametrize("kernel", sorted(STORES))
def test_row_index_wait_is_tight(kernel):
    tiles = [(64, 8), (224, 6), (32, 3)]
    assert run(tiles, STORES[kernel]) == []
    assert run(tiles, STORES[kernel], delta=(1, "R", +1)) != []
