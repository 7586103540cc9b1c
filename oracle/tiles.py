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
* block:  for a block matrix whose block size is a multiple of BM and BN, by
          index arithmetic on B (each tile sits inside one block; Eq. 2's
          j <= i decides PARTIAL against FULL).
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
    """Index-arithmetic derivation for block masks whose block size is a multiple of BM and BN.

    Each tile then lies inside one block (m, n) = (i0 // Bs, j0 // Bs).  It holds
    an allowed pair iff B[m][n] = 1 and some key is not after some query
    (j0 <= i1 - 1, Eq. 2's j <= i); it is FULL iff in addition every key is at or
    before every query (j1 - 1 <= i0) and the rectangle lies inside the sequence.
    """
    bs = int(mask["block"])
    if bs % bm or bs % bn:
        raise ValueError("block derivation needs the block size to be a multiple of BM and BN")
    bmat = np.asarray(mask["block_mask"]) != 0
    nq, nk = math.ceil(L / bm), math.ceil(L / bn)
    i0 = np.arange(nq)[:, None] * bm
    i1 = np.minimum(L, i0 + bm)
    j0 = np.arange(nk)[None, :] * bn
    j1 = j0 + bn
    causal_some = j0 <= i1 - 1
    causal_all = (j1 - 1 <= i0) & (j1 <= L) & (i0 + bm <= L)
    pres, full = [], []
    for h in range(H):
        bh = bmat[h] if bmat.shape[0] > 1 else bmat[0]
        kept = bh[(i0 // bs), (j0 // bs)]                      # [nq, nk]
        p = kept & causal_some
        pres.append(p)
        full.append(p & causal_all)
    return _csr(np.concatenate(pres), np.concatenate(full))


def tile_lists(mask: dict, H: int, L: int, bm: int, bn: int):
    if mask["kind"] == "block" and int(mask["block"]) % bm == 0 and int(mask["block"]) % bn == 0 and L > 16384:
        return tile_lists_block(mask, H, L, bm, bn)
    return tile_lists_dense(mask, H, L, bm, bn)


def key_block_lists(mask: dict, H: int, Hk: int, L: int, bm: int, bn: int, kb_size: int = 128):
    """Transposed lists for the backward, from the dense mask: for every (K/V head hk, key block of
    kb_size keys), in that row-major order, the entries (g << 24) | (query tile << 1) | full for each
    query head h = hk * (H / Hk) + g in turn and each query tile (of bm rows) whose rectangle with
    the block holds an allowed pair; full = the rectangle (keys clipped to the bn-key tiles that
    exist, i.e. to ceil(L / bn) * bn) lies inside the sequence and every pair is allowed.
    Returns (col_ptr int32 [Hk * nkb + 1], entries int32)."""
    g = H // Hk
    nq, nk = math.ceil(L / bm), math.ceil(L / bn)
    nkb = math.ceil(L / kb_size)
    dense = [np.zeros((nq * bm, nkb * kb_size), dtype=bool) for _ in range(H)]
    for h in range(H):
        dense[h][:L, :L] = allowed_rows(mask, h, np.arange(L), L)
    col_ptr, entries = [0], []
    for hk in range(Hk):
        for kb in range(nkb):
            k0, k1 = kb * kb_size, min((kb + 1) * kb_size, nk * bn)
            for gi in range(g):
                m = dense[hk * g + gi]
                for qt in range(nq):
                    r0, r1 = qt * bm, (qt + 1) * bm
                    rect = m[r0:r1, k0:k1]
                    if rect.any():
                        full = bool(rect.all()) and r1 <= L and k1 <= L
                        entries.append((gi << 24) | (qt << 1) | int(full))
            col_ptr.append(len(entries))
    return np.array(col_ptr, dtype=np.int32), np.array(entries, dtype=np.int32)
