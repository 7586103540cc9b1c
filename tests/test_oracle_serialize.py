"""Pins for the token serialisation orders (oracle/serialize.py).  CPU only."""

import numpy as np
import pytest

from oracle.serialize import ORDERS, positions, reorder


def test_block_row_hand_example():
    # 4 x 4 grid: blocks (0,0), (0,1), (1,0), (1,1), each numbered row by row inside
    want = np.array([[0, 1, 4, 5],
                     [2, 3, 6, 7],
                     [8, 9, 12, 13],
                     [10, 11, 14, 15]])
    assert np.array_equal(positions("block_row", 4, 4), want)


def test_block_col_hand_example():
    # 4 x 4 grid: blocks (0,0), (1,0), (0,1), (1,1), each numbered column by column inside
    want = np.array([[0, 2, 8, 10],
                     [1, 3, 9, 11],
                     [4, 6, 12, 14],
                     [5, 7, 13, 15]])
    assert np.array_equal(positions("block_col", 4, 4), want)


@pytest.mark.parametrize("gh,gw", [(2, 2), (4, 8), (6, 4), (16, 16)])
def test_orders_are_bijections_and_relations(gh, gw):
    for o in ORDERS:
        assert np.array_equal(np.sort(positions(o, gh, gw).ravel()), np.arange(gh * gw))
    # block_col is block_row of the transposed grid
    assert np.array_equal(positions("block_col", gh, gw), positions("block_row", gw, gh).T)
    # a single block: block_row is raster
    if gh == 2 and gw == 2:
        assert np.array_equal(positions("block_row", 2, 2), positions("raster", 2, 2))


def test_reorder_round_trips_and_composes():
    gh, gw = 8, 6
    x = np.random.default_rng(0).standard_normal((2, gh * gw, 3, 4))
    for a in ORDERS:
        for b in ORDERS:
            y = reorder(x, a, b, gh, gw)
            assert np.array_equal(reorder(y, b, a, gh, gw), x)
            for c in ORDERS:
                assert np.array_equal(reorder(y, b, c, gh, gw), reorder(x, a, c, gh, gw))
    # a token carries its patch: tag each raster token with its (r, c) and look it up after the move
    tag = np.array([[r * 100 + c for c in range(gw)] for r in range(gh)]).ravel()
    moved = reorder(tag[None], "raster", "block_col", gh, gw)[0]
    pos = positions("block_col", gh, gw)
    for r in range(gh):
        for c in range(gw):
            assert moved[pos[r, c]] == r * 100 + c


def test_blocks_are_consecutive_positions():
    """In both block orders every aligned run of 4 positions is one 2 x 2 block (the minimal unit)."""
    for o in ("block_row", "block_col"):
        pos = positions(o, 6, 8)
        where = {int(pos[r, c]): (r, c) for r in range(6) for c in range(8)}
        for t in range(0, 48, 4):
            cells = [where[t + u] for u in range(4)]
            rs, cs = {r for r, _ in cells}, {c for _, c in cells}
            assert len(rs) == 2 and len(cs) == 2 and min(rs) % 2 == 0 and min(cs) % 2 == 0


def test_row_major_window_example_of_the_pages():
    """The Factor 2 example of "Semantic Head Specialization ..." (the Factor 2 slides, panel (c) and the
    right-hand example): on the 4 x 8 patch grid with 2 x 2 blocks, the row-major block order puts the
    anchor token 23 so that its sliding window of 8 positions on each side (15 .. 31) lies in the rows
    around it.  Worked by hand from the figure's definition: blocks are numbered left to right, then top to
    bottom, four positions each; token 23 is the last position of block 5, which is block (1, 1), so it sits
    at patch (3, 3); position 15 closes block 3 = block (0, 3) at patch (1, 7); positions 16 .. 31 fill
    blocks (1, 0) .. (1, 3), i.e. exactly patch rows 2 and 3."""
    pos = positions("block_row", 4, 8)
    where = {int(pos[r, c]): (r, c) for r in range(4) for c in range(8)}
    assert where[23] == (3, 3)
    assert where[15] == (1, 7)
    assert {where[t] for t in range(16, 32)} == {(r, c) for r in (2, 3) for c in range(8)}
