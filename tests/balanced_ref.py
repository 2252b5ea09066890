"""The work-balanced split-K schedule as include/mla.h defines it, restated in Python.

Test infrastructure: it tells the tests which token range of which sequence each partial slot
holds, so that slot contents can be checked exactly.  Constants are the header's.
"""

from __future__ import annotations

import numpy as np

TILE = 32       # MLA_BALANCED_TILE
SEG_COST = 8    # MLA_BALANCED_SEG_COST


def segments(lens, n_units: int, cap: int | None = None, group: int = 1):
    """List of (unit, row, t0, t1, slot) for every non-empty segment, in slot order per unit.

    With group G > 1 the rows form len / G groups of G consecutive rows; a group costs like its
    longest row, the split runs over groups with n_units / G group-units, and unit G*w + i runs
    row i of group g's segment in group-unit w, clamped to the row's own length, into slot
    G*(w + g) + i."""
    lens = [int(x) for x in np.asarray(lens).reshape(-1)]
    if cap is not None:
        lens = [min(max(x, 0), cap) for x in lens]
    G = int(group)
    assert G >= 1 and len(lens) % G == 0 and n_units % G == 0
    glens = [max(lens[g * G:(g + 1) * G]) for g in range(len(lens) // G)]
    tiles = [-(-x // TILE) for x in glens]
    cost = [t + SEG_COST if t > 0 else 0 for t in tiles]
    total = sum(cost)
    if total == 0:
        return []
    q = -(-total // (n_units // G))
    out = []
    cb = 0
    for g, t in enumerate(tiles):
        if t > 0:
            s = cb + SEG_COST
            for w in range(s // q, (s + t - 1) // q + 1):
                k0 = max(w * q, s) - s
                k1 = min((w + 1) * q, s + t) - s
                for i in range(G):
                    r = g * G + i
                    r1 = min(k1, -(-lens[r] // TILE))
                    if r1 > k0:
                        out.append((G * w + i, r, k0 * TILE, min(r1 * TILE, lens[r]), G * (w + g) + i))
        cb += cost[g]
    return out


def num_slots(batch: int, n_units: int) -> int:
    return 0 if batch == 0 else n_units + batch - 1

