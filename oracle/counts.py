"""Unmasked (query, key) pair counts by enumerating the explicit mask.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The effective-throughput metric counts 4*d flops per allowed pair per head
(2d for the score, 2d for the value mix), the n^2 * d cost model of
"Vision transformers and hybrid architectures", section 3.  This module only
counts pairs, by summing the boolean mask row slab by row slab; closed forms
live in the tests as pins.
"""

from __future__ import annotations

import numpy as np

from .attention import allowed_rows


def pair_count(mask: dict, H: int, L: int, slab: int = 1024) -> np.ndarray:
    """Allowed pairs per head, int64 [H]."""
    out = np.zeros(H, dtype=np.int64)
    for h in range(H):
        for r0 in range(0, L, slab):
            out[h] += int(allowed_rows(mask, h, np.arange(r0, min(L, r0 + slab)), L).sum())
    return out
