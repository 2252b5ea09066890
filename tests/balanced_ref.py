"""The work-balanced split-K schedule as include/mla.h defines it, restated in Python.

Test infrastructure: it tells the tests which token range of which sequence each partial slot
holds, so that slot contents can be checked exactly.  Constants are the header's.
"""

from __future__ import annotations

import numpy as np

TILE = 32       # MLA_BALANCED_TILE
SEG_COST = 8    # MLA_BALANCED_SEG_COST


def segments(lens, n_units: int, cap: int | None = None):
    """List of (unit, sequence, t0, t1, slot) for every non-empty segment, in slot order per unit."""
    lens = [int(x) for x in np.asarray(lens).reshape(-1)]
    if cap is not None:
        lens = [min(max(x, 0), cap) for x in lens]
    tiles = [-(-x // TILE) for x in lens]
    cost = [t + SEG_COST if t > 0 else 0 for t in tiles]
    total = sum(cost)
    if total == 0:
        return []
    q = -(-total // n_units)
    out = []
    cb = 0
    for b, (L, t) in enumerate(zip(lens, tiles)):
        if t > 0:
            s = cb + SEG_COST
            for w in range(s // q, (s + t - 1) // q + 1):
                k0 = max(w * q, s) - s
                k1 = min((w + 1) * q, s + t) - s
                out.append((w, b, k0 * TILE, min(k1 * TILE, L), w + b))
        cb += cost[b]
    return out


def num_slots(batch: int, n_units: int) -> int:
    return 0 if batch == 0 else n_units + batch - 1

