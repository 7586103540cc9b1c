"""Host-side checks of the C-ABI library: it loads, exports what the header
declares, and its mask-descriptor compiler (tile lists, pair counts, schedule,
error handling) matches the oracle's independent derivation bit for bit.
No GPU needed: nothing here launches a kernel."""

import ctypes
import os
import re

import numpy as np
import pytest

from block_sparse_softmax_amd import _lib
from block_sparse_softmax_amd.inputs import block_matrix_top_half, head_windows, workload
from oracle.counts import pair_count
from oracle.tiles import tile_lists, tile_lists_dense

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bss_attn.h")


@pytest.fixture(scope="module")
def lib():
    return _lib.load_library()


def test_library_exports_every_declared_symbol(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(attn_[a-z_]+)\s*\(", text, re.M))
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.attn_version().decode().startswith("bss_attn")


def test_checked_library_exports_the_same_symbols():
    """The checked build (range checks in the forward kernels) loads and exports every declared symbol
    too; its attn_checks reports the checks enabled (no GPU call: only the flag is asked for)."""
    import ctypes
    from block_sparse_softmax_amd.build import LIB_CHECKED
    if not os.path.exists(LIB_CHECKED):
        pytest.skip("checked build missing")
    chk = ctypes.CDLL(LIB_CHECKED)
    for name in _lib.EXPORTS:
        assert hasattr(chk, name), name
    en = ctypes.c_int32(-1)
    assert chk.attn_checks(ctypes.byref(en), None, 0) == 0 and en.value == 1
    en.value = -1
    assert _lib.load_library().attn_checks(ctypes.byref(en), None, 0) == 0 and en.value == 0


def _compare(mask, L, H, D=64):
    plan = _lib.Plan(mask, L, H, D)
    bm, bn, rp, kv, fl = plan.tiles()
    ref = tile_lists(mask, H, L, bm, bn)
    assert rp.dtype == ref[0].dtype and np.array_equal(rp, ref[0])
    assert kv.dtype == ref[1].dtype and np.array_equal(kv, ref[1])
    assert fl.dtype == ref[2].dtype and np.array_equal(fl, ref[2])
    return plan, (bm, bn, rp, kv, fl)


SMALL_MASKS = [
    (dict(kind="full"), 300, 2),
    (dict(kind="full", causal=True), 300, 2),
    (dict(kind="chunk", chunk=64), 256, 2),
    (dict(kind="chunk", chunk=100), 333, 1),
    (dict(kind="chunk", chunk=1), 130, 1),
    (dict(kind="chunk", chunk=50, causal=True), 250, 1),
    (dict(kind="window", left=0, right=0), 200, 1),
    (dict(kind="window", left=17, right=3), 500, 2),
    (dict(kind="window", left=128, right=128), 1000, 1),
    (dict(kind="window", left=5000, right=5000), 700, 1),
    (dict(kind="window", left=0, right=0, causal=True, head_left=[0, 63, 64, 1000]), 777, 4),
    (dict(kind="window", left=40, right=9, causal=True), 411, 1),
]


@pytest.mark.parametrize("mi", range(len(SMALL_MASKS)))
def test_tile_lists_match_oracle_small(lib, mi):
    mask, L, H = SMALL_MASKS[mi]
    _compare(mask, L, H)


@pytest.mark.parametrize("bs,nb,L", [(128, 8, 1024), (128, 8, 1000), (256, 6, 1536), (64, 20, 1280),
                                     (100, 10, 1000), (48, 25, 1190), (384, 3, 1100)])
def test_tile_lists_match_oracle_block(lib, bs, nb, L):
    H = 2
    bm = block_matrix_top_half(7, 5, H, nb)
    bm[1, nb // 2, :] = 0          # an empty block row
    mask = dict(kind="block", block=bs, block_mask=bm)
    plan = _lib.Plan(mask, L, H, 128)
    bmt, bnt, rp, kv, fl = plan.tiles()
    ref = tile_lists_dense(mask, H, L, bmt, bnt)
    for a, b in zip((rp, kv, fl), ref):
        assert np.array_equal(a, b)


def test_random_descriptors_match_oracle(lib):
    rng = np.random.default_rng(11)
    for trial in range(40):
        L = int(rng.integers(1, 700))
        H = int(rng.integers(1, 3))
        kind = rng.choice(["full", "chunk", "window", "block"])
        causal = bool(rng.integers(0, 2))
        if kind == "full":
            mask = dict(kind="full", causal=causal)
        elif kind == "chunk":
            mask = dict(kind="chunk", chunk=int(rng.integers(1, 300)), causal=causal)
        elif kind == "window":
            mask = dict(kind="window", left=int(rng.integers(0, 400)), right=int(rng.integers(0, 400)),
                        causal=causal)
            if rng.integers(0, 2):
                mask["head_left"] = rng.integers(0, 800, H)
        else:
            bs = int(rng.integers(1, 200))
            nb = -(-L // bs)
            b = np.tril(rng.integers(0, 2, (H, nb, nb))).astype(np.uint8)
            mask = dict(kind="block", block=bs, block_mask=b)
        if kind != "block" and trial % 2:
            mask["prefix"] = int(rng.integers(1, 200))    # StreamingLLM prefix tokens
        plan = _lib.Plan(mask, L, H, 80)
        bm, bn, rp, kv, fl = plan.tiles()
        ref = tile_lists_dense(mask, H, L, bm, bn)
        for a, b in zip((rp, kv, fl), ref):
            assert np.array_equal(a, b), mask
        per, tot = plan.pairs()
        assert np.array_equal(per, pair_count(mask, H, L)), mask
        assert tot == per.sum()


@pytest.mark.parametrize("name", ["tiny_chunk", "vit896", "vit1792", "lm_headwin"])
def test_workload_tile_lists_and_pairs(lib, name):
    w = workload(name)
    for label, mask in w["masks"].items():
        plan, _ = _compare(mask, w["L"], w["H"], w["D"])
        per, tot = plan.pairs()
        if w["L"] <= 4096:
            assert np.array_equal(per, pair_count(mask, w["H"], w["L"]))
        else:  # closed forms at 16K tokens
            L = w["L"]
            exp = L * L if mask["kind"] == "full" else L * (2 * mask["left"] + 1) - mask["left"] * (mask["left"] + 1)
            assert np.all(per == exp)


def test_blocksparse_128k_tile_lists(lib):
    w = workload("blocksparse128k")
    mask = w["masks"]["block50"]
    plan = _lib.Plan(mask, w["L"], w["H"], w["D"])
    bm, bn, rp, kv, fl = plan.tiles()
    assert mask["block"] % bm == 0 and mask["block"] % bn == 0
    ref = tile_lists(mask, w["H"], w["L"], bm, bn)   # index-arithmetic derivation at 128K
    for a, b in zip((rp, kv, fl), ref):
        assert np.array_equal(a, b)
    per, tot = plan.pairs()
    nb = w["L"] // mask["block"]
    bsz = mask["block"]
    kept = mask["block_mask"].reshape(w["H"], -1).sum(axis=1).astype(np.int64)
    assert np.array_equal(per, nb * bsz * (bsz + 1) // 2 + (kept - nb) * bsz * bsz)
    assert int(kept[0]) == 263679


def _schedule_cost(flags, b, e):
    return float(np.sum(np.where(flags[b:e] == 1, 1.0, 1.25)))


def test_schedule_covers_every_row_once(lib):
    """The batch-1 schedule: 8 equal-length XCD queues (padding items have head -1); every (head, query
    tile) row's list is covered exactly once, by one item or by pieces that cut it into contiguous ranges
    in piece order; split rows own distinct partial slots and split-row indices (their merge-list entry);
    the queues carry equal cost: within twice the largest item's, or, where whole heads were given to
    XCDs (each head's items in one queue), every queue within 5 % of the mean."""
    split_seen = {}
    for name in ("vit896", "vit1792", "lm_headwin"):
        w = workload(name)
        for label, mask in w["masks"].items():
            plan = _lib.Plan(mask, w["L"], w["H"], w["D"])
            bm, bn, rp, kv, fl = plan.tiles()
            items = plan.schedule()
            nq = -(-w["L"] // bm)
            assert items.shape[1] == 8 and items.shape[0] % 8 == 0
            real = items[items[:, 0] >= 0]
            assert np.all(items[items[:, 0] < 0][:, 3] == items[items[:, 0] < 0][:, 2])
            rows = real[:, 0] * nq + real[:, 1]
            assert np.array_equal(np.unique(rows), np.arange(w["H"] * nq))
            slots, split_rows = [], []
            for r in np.unique(rows):
                its = real[rows == r]
                its = its[np.argsort(its[:, 5])]
                npc = its[0, 6]
                assert len(its) == npc and np.all(its[:, 6] == npc) and np.array_equal(its[:, 5], np.arange(npc))
                assert its[0, 2] == rp[r] and its[-1, 3] == rp[r + 1]
                assert np.all(its[1:, 2] == its[:-1, 3]) and np.all(its[:, 3] > its[:, 2] - (npc == 1))
                if npc > 1:
                    assert np.all(its[:, 4] == its[0, 4]) and np.all(its[:, 7] == its[0, 7])
                    slots.extend(its[0, 4] + np.arange(npc))
                    split_rows.append(its[0, 7])
            assert len(set(slots)) == len(slots) and len(set(split_rows)) == len(split_rows)
            if slots:
                assert sorted(slots) == list(range(len(slots))) and sorted(split_rows) == list(range(len(split_rows)))
            split_seen[(name, label)] = len(split_rows)
            # per-XCD queues of equal total cost
            q = items.reshape(8, -1, 8)
            cost = np.array([[0.0 if it[0] < 0 else 0.5 + _schedule_cost(fl, it[2], it[3]) + (2.0 if it[6] > 1 else 0.0)
                              for it in qq] for qq in q])
            tot = cost.sum(axis=1)
            heads_per_queue = [set(qq[qq[:, 0] >= 0][:, 0].tolist()) for qq in q]
            whole_heads = all(not (a & b) for i, a in enumerate(heads_per_queue) for b in heads_per_queue[i + 1:])
            if whole_heads and name == "lm_headwin":
                assert tot.max() <= 1.05 * tot.mean() + 1e-9, (name, label, tot)
            else:
                assert tot.max() - tot.min() <= 2 * cost.max() + 1e-9, (name, label, tot)
    # the per-head windows (uneven rows, one round of work-groups) keep each head on one XCD
    lw = workload("lm_headwin")
    its = _lib.Plan(lw["masks"]["headwin"], lw["L"], lw["H"], lw["D"]).schedule().reshape(8, -1, 8)
    owner = {}
    for x in range(8):
        for h in set(its[x][its[x][:, 0] >= 0][:, 0].tolist()):
            assert owner.setdefault(h, x) == x, ("head on two XCDs", h)
    # uniform ViT masks are never split; the causal per-head windows are
    assert split_seen[("vit896", "full")] == 0 and split_seen[("vit1792", "full")] == 0
    assert split_seen[("vit1792", "swa512")] == 0
    assert split_seen[("lm_headwin", "headwin")] > 0


def _status(lib, mask, L, H, D):
    desc, keep = _lib.build_desc(mask, H)
    h = ctypes.c_void_p()
    st = lib.attn_plan_create(ctypes.byref(desc), L, H, D, ctypes.byref(h))
    if st == 0:
        lib.attn_plan_destroy(h)
    return st, lib.attn_last_error().decode()


def test_descriptor_errors(lib):
    ok, _ = _status(lib, dict(kind="full"), 64, 1, 64)
    assert ok == _lib.ATTN_OK
    st, msg = _status(lib, dict(kind="full"), 64, 1, 96)
    assert st == _lib.ATTN_E_UNSUPPORTED and "96" in msg
    assert _status(lib, dict(kind="window", left=575, right=0, causal=True, prefix=4), 4096, 16, 256)[0] == \
        _lib.ATTN_OK
    assert _status(lib, dict(kind="chunk", chunk=0), 64, 1, 64)[0] == _lib.ATTN_E_INVAL
    assert _status(lib, dict(kind="window", left=-1, right=0), 64, 1, 64)[0] == _lib.ATTN_E_INVAL
    assert _status(lib, dict(kind="window", left=0, right=0, head_left=[3, -2]), 64, 2, 64)[0] == _lib.ATTN_E_INVAL
    upper = np.tril(np.ones((1, 4, 4), np.uint8))
    upper[0, 1, 3] = 1
    st, msg = _status(lib, dict(kind="block", block=16, block_mask=upper), 64, 1, 64)
    assert st == _lib.ATTN_E_INVAL and "diagonal" in msg
    st, _ = _status(lib, dict(kind="block", block=16, block_mask=np.ones((3, 4, 4), np.uint8)), 64, 2, 64)
    assert st == _lib.ATTN_E_INVAL
    assert _status(lib, dict(kind="full"), 0, 1, 64)[0] == _lib.ATTN_E_INVAL
    assert _status(lib, dict(kind="window", left=3, right=0, prefix=-1), 64, 1, 64)[0] == _lib.ATTN_E_INVAL
    st, msg = _status(lib, dict(kind="block", block=16, block_mask=np.tril(np.ones((1, 4, 4), np.uint8)), prefix=4),
                      64, 1, 64)
    assert st == _lib.ATTN_E_INVAL and "prefix" in msg
    d = _lib.MaskDesc()
    d.kind = 9
    h = ctypes.c_void_p()
    assert lib.attn_plan_create(ctypes.byref(d), 64, 1, 64, ctypes.byref(h)) == _lib.ATTN_E_INVAL
    assert lib.attn_plan_create(None, 64, 1, 64, ctypes.byref(h)) == _lib.ATTN_E_INVAL


def test_launch_argument_errors_without_gpu(lib):
    """Validation runs before any HIP call: bad shapes and a short workspace are rejected."""
    plan = _lib.Plan(dict(kind="full"), 256, 2, 64)
    fake = 1 << 20  # never dereferenced: validation fails first

    def t(L=256, H=2, D=64, stride_l=128, data=fake):
        a = _lib.AttnTensor()
        a.data, a.B, a.L, a.H, a.D = data, 1, L, H, D
        a.stride_b, a.stride_l, a.stride_h = L * stride_l, stride_l, 64
        return a

    ln = _lib.Launch()
    ln.workspace = fake
    ln.workspace_bytes = 16
    q, k, v, o = t(), t(), t(), t(data=fake * 2)
    st = lib.attn_masked_fwd_plan(plan.handle, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None,
                                  ctypes.byref(o), ctypes.byref(ln))
    assert st == _lib.ATTN_E_WORKSPACE
    k_bad = t(L=128)
    ln.workspace_bytes = plan.workspace_bytes()
    st = lib.attn_masked_fwd_plan(plan.handle, ctypes.byref(q), ctypes.byref(k_bad), ctypes.byref(v), None,
                                  ctypes.byref(o), ctypes.byref(ln))
    assert st == _lib.ATTN_E_INVAL
    q_mis = t(stride_l=130)
    st = lib.attn_masked_fwd_plan(plan.handle, ctypes.byref(q_mis), ctypes.byref(k), ctypes.byref(v), None,
                                  ctypes.byref(o), ctypes.byref(ln))
    assert st == _lib.ATTN_E_INVAL and "16-byte" in lib.attn_last_error().decode()
    o_alias = t()
    st = lib.attn_masked_fwd_plan(plan.handle, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None,
                                  ctypes.byref(o_alias), ctypes.byref(ln))
    assert st == _lib.ATTN_E_INVAL


def test_group_argument_errors_without_gpu(lib):
    """The grouped entry point validates before any HIP call."""
    plan = _lib.Plan(dict(kind="full"), 256, 2, 64)
    plan2 = _lib.Plan(dict(kind="full"), 256, 2, 80)
    fake = 1 << 20

    def t(data=fake, D=64):
        a = _lib.AttnTensor()
        a.data, a.B, a.L, a.H, a.D = data, 1, 256, 2, D
        a.stride_b, a.stride_l, a.stride_h = 256 * 128, 128, 64
        return a

    ln = _lib.Launch()
    P = ctypes.c_void_p

    def call(n, plans, outs, wss, D=64):
        ta = _lib.AttnTensor * max(n, 1)
        q = ta(*[t(D=D) for _ in range(max(n, 1))])
        o = ta(*outs)
        pl = (P * max(n, 1))(*plans)
        ws = (P * max(n, 1))(*wss)
        wb = (ctypes.c_size_t * max(n, 1))(*[plan.workspace_bytes()] * max(n, 1))
        return lib.attn_masked_fwd_group(n, pl, q, q, q, None, o, ws, wb, ctypes.byref(ln))

    h = plan.handle.value
    assert call(0, [h], [t(fake * 2)], [fake * 4]) == _lib.ATTN_E_INVAL
    assert call(9, [h] * 9, [t(fake * (2 + j)) for j in range(9)], [fake * (20 + j) for j in range(9)]) == \
        _lib.ATTN_E_UNSUPPORTED
    # shared workspace, shared output
    assert call(2, [h, h], [t(fake * 2), t(fake * 3)], [fake * 4, fake * 4]) == _lib.ATTN_E_INVAL
    assert call(2, [h, h], [t(fake * 2), t(fake * 2)], [fake * 4, fake * 5]) == _lib.ATTN_E_INVAL
    # differing head dims
    assert call(2, [h, plan2.handle.value], [t(fake * 2), t(fake * 3)], [fake * 4, fake * 5]) == _lib.ATTN_E_INVAL
    assert "same head dim" in lib.attn_last_error().decode()


def test_reorder_argument_errors_without_gpu(lib):
    fake = 1 << 20

    def t(L, data=fake):
        a = _lib.AttnTensor()
        a.data, a.B, a.L, a.H, a.D = data, 1, L, 2, 64
        a.stride_b, a.stride_l, a.stride_h = L * 128, 128, 64
        return a

    ln = _lib.Launch()
    i, o = t(48), t(48, fake * 2)
    f = lib.attn_reorder_tokens
    assert f(ctypes.byref(i), 0, ctypes.byref(o), 1, 6, 7, ctypes.byref(ln)) == _lib.ATTN_E_INVAL   # 6*7 != 48
    assert f(ctypes.byref(i), 0, ctypes.byref(o), 1, 3, 16, ctypes.byref(ln)) == _lib.ATTN_E_INVAL  # odd side
    assert f(ctypes.byref(i), 0, ctypes.byref(o), 3, 6, 8, ctypes.byref(ln)) == _lib.ATTN_E_INVAL   # bad order
    assert f(ctypes.byref(i), 0, ctypes.byref(i), 1, 6, 8, ctypes.byref(ln)) == _lib.ATTN_E_INVAL   # aliasing


def test_decode_argument_errors_without_gpu(lib):
    """Decode validation runs on the host before any device call."""
    import ctypes
    from block_sparse_softmax_amd._lib import AttnTensor, DecodeDesc, Launch

    def view(B, L, H, D, ptr=16):
        t = AttnTensor()
        t.data, t.B, t.L, t.H, t.D = ptr, B, L, H, D
        t.stride_b, t.stride_l, t.stride_h = L * H * D, H * D, D
        return t

    desc = DecodeDesc(576, 0)
    nbytes = ctypes.c_size_t()
    q, k = view(64, 1, 32, 128), view(64, 131072, 8, 128, 4096)
    assert lib.attn_decode_workspace_bytes(ctypes.byref(q), ctypes.byref(k), 131072, ctypes.byref(desc),
                                           ctypes.byref(nbytes)) == 0
    assert nbytes.value == 0                      # 512 work-groups: one split per sequence and head
    q1, k1 = view(1, 1, 32, 128), view(1, 131072, 8, 128, 4096)
    full = DecodeDesc(0, 0)
    assert lib.attn_decode_workspace_bytes(ctypes.byref(q1), ctypes.byref(k1), 131072, ctypes.byref(full),
                                           ctypes.byref(nbytes)) == 0
    assert nbytes.value == 32 * 64 * 130 * 4      # 64 splits of 2048 keys, (D + 2) floats each
    bad_d = view(1, 1, 32, 80)
    assert lib.attn_decode_workspace_bytes(ctypes.byref(bad_d), ctypes.byref(k1), 10, ctypes.byref(desc),
                                           ctypes.byref(nbytes)) == -2
    ln = Launch()
    o = view(1, 1, 32, 128, 8192)
    v1 = view(1, 131072, 8, 128, 4096 + 1024)
    seq = ctypes.c_void_p(64)
    assert lib.attn_decode_fwd(ctypes.byref(q1), ctypes.byref(k1), ctypes.byref(v1), None, 10,
                               ctypes.byref(desc), None, ctypes.byref(o), ctypes.byref(ln)) == -1   # no seq_lens
    assert lib.attn_decode_fwd(ctypes.byref(q1), ctypes.byref(k1), ctypes.byref(v1), seq, 131073,
                               ctypes.byref(desc), None, ctypes.byref(o), ctypes.byref(ln)) == -1   # max_len > Lmax
    g17 = view(1, 1, 17 * 8, 128)
    assert lib.attn_decode_fwd(ctypes.byref(g17), ctypes.byref(k1), ctypes.byref(v1), seq, 10,
                               ctypes.byref(desc), None, ctypes.byref(view(1, 1, 17 * 8, 128, 8192)),
                               ctypes.byref(ln)) == -2                                                # 17 heads per cache head
    neg = DecodeDesc(576, -1)
    assert lib.attn_decode_fwd(ctypes.byref(q1), ctypes.byref(k1), ctypes.byref(v1), seq, 10,
                               ctypes.byref(neg), None, ctypes.byref(o), ctypes.byref(ln)) == -1    # negative prefix
    assert lib.attn_decode_fwd(ctypes.byref(q1), ctypes.byref(k1), ctypes.byref(v1), seq, 131072,
                               ctypes.byref(full), None, ctypes.byref(o), ctypes.byref(ln)) == -3   # no workspace


def test_rr_workspace_and_argument_errors_without_gpu(lib):
    """Pattern-search validation and workspace size on the host.  The workspace holds, each part
    256-byte aligned: the sampled queries (rows of d bf16), the stride-summed keys (rows of 2 d bf16,
    the hi and lo halves, plus 16 pad bytes), one float per key row (its squared norm),
    one float per (batch, head) (the largest key-aggregate
    norm), one int per 128-row query tile (recompute flag) and one float
    per (key block, row) (the single pass's per-block sums); one row per stride of every block (nb R >= floor(L / S)) padded to a multiple of 256."""
    import ctypes
    from block_sparse_softmax_amd._lib import AttnTensor, RrParams

    def view(B, L, H, D, ptr=16):
        t = AttnTensor()
        t.data, t.B, t.L, t.H, t.D = ptr, B, L, H, D
        t.stride_b, t.stride_l, t.stride_h = L * H * D, H * D, D
        return t

    def ws(q, prm):
        n = ctypes.c_size_t()
        st = lib.attn_rr_workspace_bytes(ctypes.byref(q), ctypes.byref(prm), ctypes.byref(n))
        return st, n.value

    def expect(B, H, rows, D, nb):
        up = lambda x: -(-x // 256) * 256
        bh = B * H
        return (up(bh * rows * 2 * D) + up(bh * rows * (4 * D + 16)) + up(bh * rows * 4)
                + up(bh * 4)
                + up(bh * (rows // 128) * 4) + up(bh * rows * nb * 4))

    assert ws(view(1, 131072, 32, 128), RrParams(8, 128, 0.9, 1)) == (0, expect(1, 32, 16384, 128, 1024))
    assert expect(1, 32, 16384, 128, 1024) > 2 * 2 ** 30      # the single pass's block sums: 2 GiB at 128K
    # 9 key blocks of 32 strides -> 288 rows -> 512 (a multiple of 256)
    assert ws(view(2, 1030, 3, 80), RrParams(4, 128, 0.5, 0)) == (0, expect(2, 3, 512, 80, 9))
    # 16388 // 8 = 2048 strides, a whole number of 256-row tiles, but 129 blocks of 16 strides need 2064 rows
    assert ws(view(1, 16388, 1, 64), RrParams(8, 128, 0.9, 1)) == (0, expect(1, 1, 2304, 64, 129))
    assert ws(view(1, 4096, 2, 96), RrParams(8, 128, 0.9, 1))[0] == _lib.ATTN_E_UNSUPPORTED   # head dim
    assert ws(view(1, 4096, 2, 64), RrParams(8, 100, 0.9, 1))[0] == _lib.ATTN_E_INVAL         # Bs % S != 0
    assert ws(view(1, 4096, 2, 64), RrParams(8, 512, 0.9, 1))[0] == _lib.ATTN_E_UNSUPPORTED   # Bs / S = 64
    assert ws(view(1, 4096, 2, 64), RrParams(8, 128, 0.0, 1))[0] == _lib.ATTN_E_INVAL         # tau
    assert ws(view(1, 4096, 2, 64), RrParams(8, 128, 1.5, 1))[0] == _lib.ATTN_E_INVAL
    assert ws(view(1, 4096, 2, 64), RrParams(8, 128, 0.9, 2))[0] == _lib.ATTN_E_INVAL         # protect_last
    assert ws(view(1, 4, 2, 64), RrParams(8, 64, 0.9, 1))[0] == _lib.ATTN_E_INVAL              # L < S
    assert ws(view(1, 4096 * 64 + 64, 1, 64), RrParams(8, 64, 0.9, 1))[0] == _lib.ATTN_E_UNSUPPORTED  # > 4096 blocks


def test_head_dim_256_is_forward_only(lib):
    """Plans of head dim 256 compile (the forward runs them); every backward entry point refuses them."""
    plan = _lib.Plan(dict(kind="window", left=575, right=0, causal=True), 2048, 16, 256)
    assert plan.workspace_bytes() > 0
    nbytes = ctypes.c_size_t(0)
    st = lib.attn_bwd_workspace_bytes(plan.handle, 1, 4, ctypes.byref(nbytes))
    assert st == _lib.ATTN_E_UNSUPPORTED and "256" in lib.attn_last_error().decode()
    nb, ne, ni = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    cp, en, it = (ctypes.POINTER(ctypes.c_int32)(), ctypes.POINTER(ctypes.c_int32)(), ctypes.POINTER(ctypes.c_int32)())
    assert lib.attn_bwd_lists(plan.handle, 4, ctypes.byref(nb), ctypes.byref(cp), ctypes.byref(ne), ctypes.byref(en),
                              ctypes.byref(ni), ctypes.byref(it)) == _lib.ATTN_E_UNSUPPORTED
    assert lib.attn_bwd_upload(plan.handle, 4, None, 0, None) == _lib.ATTN_E_UNSUPPORTED


def test_swa576_d256_workload_pairs(lib):
    """The 128K-token causal window of 576 keys (head dim 256): every head holds
    sum_i min(i + 1, 576) = 576 * 577 / 2 + (L - 576) * 576 allowed pairs."""
    w = workload("swa576_d256")
    assert (w["H"], w["Hkv"], w["D"]) == (16, 4, 256)
    mask = w["masks"]["swa576"]
    plan = _lib.Plan(mask, w["L"], w["H"], w["D"])
    per, tot = plan.pairs()
    W, L = mask["left"] + 1, w["L"]
    assert np.all(per == W * (W + 1) // 2 + (L - W) * W) and tot == per.sum()
    # every query tile lists the key tiles its window touches: 10 or 11 of 64 keys, the diagonal PARTIAL
    bm, bn, rp, kv, fl = plan.tiles()
    n = np.diff(rp)
    assert n.max() <= -(-(bm + W - 1) // bn) + 1 and n[w["H"] * 8 - 1] >= 10


def test_forward_kernel_choice(lib):
    """Head dims 64 and 80 run the swizzled kernel, 256 the single-group one; at 128 the plan picks
    the ping-pong kernel when its rows hold 32 tiles or more on average (schedule cost)."""
    assert _lib.Plan(dict(kind="full"), 1024, 2, 64).kernel() == "swizzled"
    assert _lib.Plan(dict(kind="full"), 1024, 2, 80).kernel() == "swizzled"
    assert _lib.Plan(dict(kind="full"), 4096, 2, 256).kernel() == "single"
    assert _lib.Plan(dict(kind="full"), 2048, 2, 128).kernel() == "pingpong"      # 32 tiles per row
    assert _lib.Plan(dict(kind="full"), 1984, 2, 128).kernel() == "single"        # 31
    assert _lib.Plan(dict(kind="window", left=575, right=0, causal=True), 131072, 4, 128).kernel() == "single"
    w = workload("blocksparse128k")
    assert _lib.Plan(w["masks"]["block50"], w["L"], w["H"], w["D"]).kernel() == "pingpong"
