"""Query-group geometry on the (t, h, w) token grid.

DSV summaries, zh §2.2 "Query Grouping" / ko §2나 (Observation 5): tokens that are adjacent
in the 3-D spatio-temporal grid share most of their critical KV pairs, so adjacent queries
are grouped and share one index list. Reading used here: a group is a gt x gh x gw box of the
row-major token grid (token n = (t*Hh + y)*W + x); boxes tile the grid; boxes are numbered
row-major over (box_t, box_y, box_x) and members row-major over (dt, dy, dx).
"""
from __future__ import annotations

import numpy as np


def token_index(t, y, x, Hh, W):
    return (t * Hh + y) * W + x


def group_members(T: int, Hh: int, W: int, gt: int, gh: int, gw: int) -> np.ndarray:
    """int64 [NG, G]: token indices of each group's members, in member order."""
    if T % gt or Hh % gh or W % gw:
        raise ValueError("group extents must divide the token grid")
    groups = []
    for a in range(T // gt):
        for b in range(Hh // gh):
            for c in range(W // gw):
                mem = []
                for dt in range(gt):
                    for dy in range(gh):
                        for dx in range(gw):
                            mem.append(token_index(a * gt + dt, b * gh + dy, c * gw + dx, Hh, W))
                groups.append(mem)
    return np.asarray(groups, dtype=np.int64)


def group_of_token(members: np.ndarray, S: int) -> np.ndarray:
    """int64 [S]: the group each token belongs to."""
    g = np.full(S, -1, dtype=np.int64)
    for gi, mem in enumerate(members):
        g[mem] = gi
    return g
