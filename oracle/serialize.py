"""Token serialisation orders of a 2D patch grid, and re-permutation between them.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "Semantic Head Specialization ..." (the SHS slides), the slides on
Factor 2 (token serialisation) and the Ariadne design: a Gh x Gw patch grid is
flattened to a 1D token sequence, and local attention acts on that sequence.
Orders (Gh, Gw even for the block orders; 2 x 2 patches form a block, the
minimal unit):

  raster      row by row:                      position = r * Gw + c
  block_row   (c) blocks left to right, then top to bottom; inside a block
              its 4 patches row by row (reading: the slides draw the block as
              the unit without numbering its inside; row-major is the plain
              choice and matches raster inside a block)
  block_col   (d) blocks top to bottom, then left to right; reading: the
              block_row order of the transposed grid, so inside a block the
              4 patches go column by column

Ariadne alternates block_row and block_col layers and re-permutes the tokens
where the order changes (a memory-bound gather).  The mapping is written out
with explicit loops over the grid.
"""

from __future__ import annotations

import numpy as np

ORDERS = ("raster", "block_row", "block_col")


def positions(order: str, gh: int, gw: int) -> np.ndarray:
    """pos[r, c]: the sequence position of patch (r, c) in `order`."""
    pos = np.full((gh, gw), -1, dtype=np.int64)
    if order == "raster":
        for r in range(gh):
            for c in range(gw):
                pos[r, c] = r * gw + c
    elif order == "block_row":
        if gh % 2 or gw % 2:
            raise ValueError("block orders need an even grid")
        t = 0
        for br in range(gh // 2):            # blocks top to bottom ...
            for bc in range(gw // 2):        # ... each row of blocks left to right
                for dr in range(2):
                    for dc in range(2):
                        pos[2 * br + dr, 2 * bc + dc] = t
                        t += 1
    elif order == "block_col":
        if gh % 2 or gw % 2:
            raise ValueError("block orders need an even grid")
        t = 0
        for bc in range(gw // 2):            # blocks left to right ...
            for br in range(gh // 2):        # ... each column of blocks top to bottom
                for dc in range(2):
                    for dr in range(2):
                        pos[2 * br + dr, 2 * bc + dc] = t
                        t += 1
    else:
        raise ValueError(order)
    return pos


def reorder(x: np.ndarray, src: str, dst: str, gh: int, gw: int, axis: int = 1) -> np.ndarray:
    """Tokens of x (sequence along `axis`, in `src` order) rearranged into `dst` order."""
    ps, pd = positions(src, gh, gw).ravel(), positions(dst, gh, gw).ravel()
    gather = np.empty(gh * gw, dtype=np.int64)
    gather[pd] = ps                          # the token at dst position pd[p] is patch p, at ps[p] in x
    return np.take(x, gather, axis=axis)
