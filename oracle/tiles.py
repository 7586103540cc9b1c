"""Canonical per-query-tile KV tile lists, derived from the explicit mask.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is listed: the token mask (see ``attention.py``) is cut into BM x BN
tiles.  For every (head, query tile), in that row-major order, the list holds
the ascending indices of the key tiles that contain at least one allowed
pair; a tile is flagged FULL (1) when its whole BM x BN rectangle lies inside
the sequence and every pair in it is allowed, else PARTIAL (0).  Tiles with
no allowed pair are left out.  This is the block partition of the
block-sparse page ("RRAttention", section 2.1: contiguous blocks,
N_b = ceil(L/B)) applied to any of the masks.

Two independent derivations:
* dense:  reshape the explicit L x L mask into [nq, BM, nk, BN] and use any/all;
* block:  for a block matrix whose block size equals BM and BN, by index
          arithmetic on B (a kept block strictly below the diagonal is FULL,
          the diagonal block is PARTIAL because of j <= i, Eq. 2).
"""

from __future__ import annotations

import math

import numpy as np

from .attention import allowed_rows


def _csr(present: np.ndarray, full: np.ndarray):
    """present/full: bool [R, nk] -> (row_ptr int32 [R+1], kv_tile int32, flag uint8)."""
    counts = present.sum(axis=1)
    row_ptr = np.zeros(present.shape[0] + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    r, c = np.nonzero(present)              # row-major order, ascending columns
    return row_ptr.astype(np.int32), c.astype(np.int32), full[r, c].astype(np.uint8)


def tile_lists_dense(mask: dict, H: int, L: int, bm: int, bn: int, heads=None):
    """Derivation from the dense mask, one query tile (BM rows x L) at a time."""
    nq, nk = math.ceil(L / bm), math.ceil(L / bn)
    heads = range(H) if heads is None else heads
    pres, full = [], []
    kv_in_range = np.array([(t + 1) * bn <= L for t in range(nk)])
    for h in heads:
        for qt in range(nq):
            rows = np.arange(qt * bm, min(L, (qt + 1) * bm))
            m = allowed_rows(mask, h, rows, L)
            pad = np.zeros((bm, nk * bn), dtype=bool)
            pad[: len(rows), :L] = m
            t = pad.reshape(bm, nk, bn)
            p = t.any(axis=(0, 2))
            f = t.all(axis=(0, 2)) & kv_in_range & ((qt + 1) * bm <= L)
            pres.append(p)
            full.append(f)
    return _csr(np.array(pres), np.array(full))


def tile_lists_block(mask: dict, H: int, L: int, bm: int, bn: int):
    """Index-arithmetic derivation for block masks when BM == BN == block size."""
    bs = int(mask["block"])
    if not (bm == bn == bs):
        raise ValueError("block derivation needs BM == BN == block size")
    bmat = np.asarray(mask["block_mask"]) != 0
    nb = math.ceil(L / bs)
    pres, full = [], []
    n_idx = np.arange(nb)
    for h in range(H):
        bh = bmat[h] if bmat.shape[0] > 1 else bmat[0]
        for m in range(nb):
            p = bh[m] & (n_idx <= m)
            f = p & (n_idx < m) & ((n_idx + 1) * bs <= L) & ((m + 1) * bs <= L)
            pres.append(p)
            full.append(f)
    return _csr(np.array(pres), np.array(full))


def tile_lists(mask: dict, H: int, L: int, bm: int, bn: int):
    if mask["kind"] == "block" and bm == bn == int(mask["block"]) and L > 16384:
        return tile_lists_block(mask, H, L, bm, bn)
    return tile_lists_dense(mask, H, L, bm, bn)
