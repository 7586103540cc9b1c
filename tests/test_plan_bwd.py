"""Host-side checks of the backward's transposed tile lists and dK/dV schedule against the oracle's
derivation from the dense mask (bit for bit), and of the backward entry points' argument validation.
No GPU needed: nothing here launches a kernel."""

import ctypes

import numpy as np
import pytest

from block_sparse_softmax_amd import _lib
from block_sparse_softmax_amd.inputs import block_matrix_top_half
from oracle.tiles import key_block_lists

MASKS = [
    (dict(kind="full"), 300, 2, 2),
    (dict(kind="full", causal=True), 520, 4, 2),
    (dict(kind="chunk", chunk=64), 256, 2, 2),
    (dict(kind="chunk", chunk=100), 333, 1, 1),
    (dict(kind="chunk", chunk=256), 1024, 2, 1),
    (dict(kind="window", left=17, right=3), 500, 2, 2),
    (dict(kind="window", left=128, right=128), 1000, 1, 1),
    (dict(kind="window", left=0, right=0, causal=True, head_left=[0, 63, 64, 1000]), 777, 4, 2),
    (dict(kind="window", left=6, right=0, causal=True, prefix=3), 450, 2, 1),
    (dict(kind="chunk", chunk=90, prefix=70), 600, 3, 1),
    (dict(kind="window", left=200, right=200), 192, 2, 2),    # L of one full key tile past the block
]


def _check(mask, L, H, Hk):
    plan = _lib.Plan(mask, L, H, 64)
    bm, bn, _, _, _ = plan.tiles()
    nkb, col_ptr, entries, items = plan.bwd_lists(Hk)
    ref_ptr, ref_ent = key_block_lists(mask, H, Hk, L, bm, bn)
    assert nkb == -(-L // 128)
    assert np.array_equal(col_ptr, ref_ptr), mask
    assert np.array_equal(entries, ref_ent), mask
    # the schedule: 8 equal queues, every (kv head, key block) once with its list range
    assert items.shape[0] % 8 == 0
    real = items[items[:, 0] >= 0]
    assert len(real) == Hk * nkb
    keys = sorted((int(a), int(b)) for a, b in real[:, :2])
    assert keys == [(hk, kb) for hk in range(Hk) for kb in range(nkb)]
    for hk, kb, b0, b1, *_ in real:
        r = hk * nkb + kb
        assert (b0, b1) == (col_ptr[r], col_ptr[r + 1])


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_key_block_lists_match_oracle(mi):
    _check(*MASKS[mi])


@pytest.mark.parametrize("bs,nb,L", [(128, 8, 1024), (128, 8, 1000), (256, 6, 1536)])
def test_key_block_lists_block_masks(bs, nb, L):
    H = 2
    bm = block_matrix_top_half(3, 9, H, nb)
    bm[1, nb // 2, :] = 0
    _check(dict(kind="block", block=bs, block_mask=bm), L, H, 1)
    _check(dict(kind="block", block=bs, block_mask=bm), L, H, 2)


def test_random_descriptors_key_block_lists():
    rng = np.random.default_rng(5)
    for trial in range(25):
        L = int(rng.integers(1, 600))
        Hk = int(rng.integers(1, 3))
        H = Hk * int(rng.integers(1, 4))
        kind = rng.choice(["full", "chunk", "window"])
        causal = bool(rng.integers(0, 2))
        if kind == "full":
            mask = dict(kind="full", causal=causal)
        elif kind == "chunk":
            mask = dict(kind="chunk", chunk=int(rng.integers(1, 300)), causal=causal)
        else:
            mask = dict(kind="window", left=int(rng.integers(0, 300)), right=int(rng.integers(0, 300)),
                        causal=causal, head_left=rng.integers(0, 500, H))
        if trial % 3 == 0:
            mask["prefix"] = int(rng.integers(1, 150))
        _check(mask, L, H, Hk)


def test_bwd_workspace_and_argument_errors_without_gpu():
    """Validation of the backward entry points runs before any HIP call."""
    lib = _lib.load_library()
    plan = _lib.Plan(dict(kind="full"), 256, 4, 64)
    n = ctypes.c_size_t()
    assert lib.attn_bwd_workspace_bytes(plan.handle, 1, 3, ctypes.byref(n)) == _lib.ATTN_E_INVAL   # 3 does not divide 4
    assert lib.attn_bwd_workspace_bytes(plan.handle, 0, 2, ctypes.byref(n)) == _lib.ATTN_E_INVAL
    assert lib.attn_bwd_workspace_bytes(plan.handle, 2, 2, ctypes.byref(n)) == _lib.ATTN_OK
    n2 = ctypes.c_size_t()
    assert lib.attn_bwd_workspace_bytes(plan.handle, 1, 2, ctypes.byref(n2)) == _lib.ATTN_OK
    assert n.value > n2.value >= plan.workspace_bytes()
    fake = 1 << 20

    def t(H=4, data=fake):
        a = _lib.AttnTensor()
        a.data, a.B, a.L, a.H, a.D = data, 1, 256, H, 64
        a.stride_b, a.stride_l, a.stride_h = 256 * 256, 256, 64
        return a

    ln = _lib.Launch()
    ln.workspace, ln.workspace_bytes = fake * 64, n2.value
    q, k, v, o, do = t(), t(2, fake * 2), t(2, fake * 3), t(data=fake * 4), t(data=fake * 5)
    dq, dk, dv = t(data=fake * 6), t(2, fake * 7), t(2, fake * 8)
    lse = ctypes.c_void_p(fake * 9)
    B = ctypes.byref

    def bwd(q=q, k=k, v=v, dq=dq, dk=dk, dv=dv, lse=lse, ws_bytes=n2.value):
        ln.workspace_bytes = ws_bytes
        return lib.attn_masked_bwd(plan.handle, B(q), B(k), B(v), B(o), B(do), lse, None, B(dq), B(dk), B(dv),
                                   None, B(ln))

    # a workspace that attn_bwd_upload never prepared
    assert bwd() == _lib.ATTN_E_INVAL and "attn_bwd_upload" in lib.attn_last_error().decode()
    assert bwd(ws_bytes=16) == _lib.ATTN_E_WORKSPACE
    assert bwd(lse=None) == _lib.ATTN_E_INVAL
    assert bwd(dq=t(data=fake)) == _lib.ATTN_E_INVAL              # dq aliases q
    assert bwd(dk=t(2, fake * 6)) == _lib.ATTN_E_INVAL            # dk aliases dq
    assert bwd(dk=t(4, fake * 7)) == _lib.ATTN_E_INVAL            # dk with q's head count
    assert bwd(k=t(3, fake * 2)) == _lib.ATTN_E_INVAL             # 3 K/V heads for 4 query heads
