"""The balanced split-K schedule (host restatement of include/mla.h): every token of every
sequence lands in exactly one segment, slots are distinct and in range, and no unit exceeds
its quota."""

import numpy as np
import pytest

from balanced_ref import SEG_COST, TILE, num_slots, segments


@pytest.mark.parametrize("n_units", [1, 2, 3, 7, 64, 256, 2048])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_partition(n_units, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 5000, size=int(rng.integers(1, 70)))
    lens[rng.random(lens.size) < 0.2] = 0
    segs = segments(lens, n_units)
    slots = [s[4] for s in segs]
    assert len(set(slots)) == len(slots)
    assert all(0 <= s < num_slots(len(lens), n_units) for s in slots)
    for b, L in enumerate(lens):
        mine = sorted((t0, t1) for w, bb, t0, t1, _ in segs if bb == b)
        covered = 0
        for t0, t1 in mine:
            assert t0 == covered and t1 > t0 and t0 % TILE == 0
            covered = t1
        assert covered == L
    tiles = -(-lens // TILE)
    total = int(np.sum(np.where(tiles > 0, tiles + SEG_COST, 0)))
    if total:
        q = -(-total // n_units)
        for w in range(n_units):
            used = sum(-(-(t1 - t0) // TILE) for ww, _, t0, t1, _ in segs if ww == w)
            assert used <= q
        assert max(s[0] for s in segs) < n_units


def test_empty_batch_and_cap():
    assert segments([0, 0], 4) == []
    segs = segments([10_000], 3, cap=4096)
    assert sum(t1 - t0 for _, _, t0, t1, _ in segs) == 4096
