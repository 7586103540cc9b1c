"""Pins for the float64 oracle: brute force, closed forms, library special cases,
invariants and the numbers printed on the pages.  CPU only."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import allowed_rows, attention, dense_mask
from oracle.counts import pair_count
from oracle.tiles import tile_lists_block, tile_lists_dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# brute force: plain Python loops, predicates written as explicit key sets
# ---------------------------------------------------------------------------

def _keys_brute(mask, h, i, L):
    kind = mask["kind"]
    if kind == "full":
        ks = list(range(L))
    elif kind == "chunk":
        c = mask["chunk"]
        start = (i // c) * c
        ks = list(range(start, min(L, start + c)))
    elif kind == "window":
        left = mask["head_left"][h] if mask.get("head_left") is not None else mask.get("left", 0)
        ks = [j for j in range(max(0, i - left), min(L, i + mask.get("right", 0) + 1))]
    elif kind == "block":
        bs = mask["block"]
        bm = mask["block_mask"]
        bh = bm[h] if len(bm) > 1 else bm[0]
        ks = []
        for n in range(len(bh[i // bs])):
            if bh[i // bs][n]:
                ks.extend(j for j in range(n * bs, min(L, (n + 1) * bs)) if j <= i)
        ks.sort()
    prefix = mask.get("prefix", 0) or 0
    if prefix:
        ks = sorted(set(ks) | set(range(min(prefix, L))))
    if mask.get("causal", False):
        ks = [j for j in ks if j <= i]
    return ks


def _brute(q, k, v, mask, sink):
    """q: [H, L, D], k, v: [Hk, L, D] nested lists (query head h reads K/V head h // (H/Hk));
    returns [H, L, D]."""
    H, L, D = len(q), len(q[0]), len(q[0][0])
    g = H // len(k)
    out = []
    for h in range(H):
        kh, vh = k[h // g], v[h // g]
        oh = []
        for i in range(L):
            ks = _keys_brute(mask, h, i, L)
            w = [math.exp(sum(q[h][i][t] * kh[j][t] for t in range(D)) / math.sqrt(D)) for j in ks]
            z = sum(w) + (math.exp(sink[h]) if sink is not None else 0.0)
            if z == 0.0:
                oh.append([0.0] * D)
                continue
            oh.append([sum(w[a] * vh[ks[a]][t] for a in range(len(ks))) / z for t in range(D)])
        out.append(oh)
    return np.array(out)


BRUTE_MASKS = [
    dict(kind="full"),
    dict(kind="full", causal=True),
    dict(kind="chunk", chunk=8),
    dict(kind="chunk", chunk=7),                      # ragged last chunk
    dict(kind="window", left=3, right=3),
    dict(kind="window", left=5, right=2),
    dict(kind="window", left=0, right=0, causal=True, head_left=[2, 30]),
    dict(kind="window", left=6, right=0, causal=True, prefix=3),   # StreamingLLM prefix + causal window
    dict(kind="window", left=2, right=4, prefix=5),                # prefix + symmetric window
    dict(kind="chunk", chunk=8, prefix=2),
    dict(kind="block", block=8, block_mask=np.array([np.tril(np.ones((4, 4), np.uint8)),
                                                     np.array([[1, 0, 0, 0], [1, 1, 0, 0],
                                                               [0, 1, 0, 0], [1, 0, 1, 1]], np.uint8)])),
    dict(kind="block", block=5, block_mask=np.array([[[1, 0, 0, 0, 0, 0, 0],
                                                      [0, 1, 0, 0, 0, 0, 0],
                                                      [1, 1, 1, 0, 0, 0, 0],
                                                      [0, 0, 0, 0, 0, 0, 0],   # an empty block row
                                                      [1, 0, 0, 1, 1, 0, 0],
                                                      [0, 0, 1, 0, 0, 1, 0],
                                                      [1, 1, 1, 1, 1, 1, 1]]], np.uint8)),
]


@pytest.mark.parametrize("mi", range(len(BRUTE_MASKS)))
@pytest.mark.parametrize("with_sink", [False, True])
def test_brute_force_tiny(mi, with_sink):
    mask = BRUTE_MASKS[mi]
    H, L, D = 2, 32, 8
    q, k, v = (_rand((1, H, L, D), s) for s in (1, 2, 3))
    sink = np.array([0.7, -1.3]) if with_sink else None
    got = attention(q, k, v, mask, sink=sink)["out"][0]
    ref = _brute(q[0].tolist(), k[0].tolist(), v[0].tolist(), mask, None if sink is None else sink.tolist())
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_grouped_query_heads():
    """Grouped-query attention is multi-head attention with each K/V head repeated for its run of
    consecutive query heads; brute force agrees on a tiny case."""
    H, Hk, L, D = 6, 2, 24, 8
    q = _rand((1, H, L, D), 31)
    k, v = _rand((1, Hk, L, D), 32), _rand((1, Hk, L, D), 33)
    for mask in (dict(kind="full", causal=True), dict(kind="window", left=4, right=1, prefix=2)):
        got = attention(q, k, v, mask)["out"]
        rep = attention(q, np.repeat(k, H // Hk, axis=1), np.repeat(v, H // Hk, axis=1), mask)["out"]
        assert np.array_equal(got, rep)
        ref = _brute(q[0].tolist(), k[0].tolist(), v[0].tolist(), mask, None)
        assert np.max(np.abs(got[0] - ref)) <= 1e-12
    with pytest.raises(ValueError):
        attention(q, _rand((1, 4, L, D), 1), _rand((1, 4, L, D), 2), dict(kind="full"))


def test_prefix_tokens_hand_example():
    """Causal window of 3 keys plus 2 prefix tokens: row 6 sees {0, 1, 4, 5, 6}; row 1 sees {0, 1}."""
    from oracle.attention import allowed_rows
    m = allowed_rows(dict(kind="window", left=2, right=0, causal=True, prefix=2), 0, np.array([6, 1]), 10)
    assert np.flatnonzero(m[0]).tolist() == [0, 1, 4, 5, 6]
    assert np.flatnonzero(m[1]).tolist() == [0, 1]


def test_brute_force_sampled_rows():
    mask = BRUTE_MASKS[5]
    H, L, D = 2, 32, 8
    q, k, v = (_rand((1, H, L, D), s) for s in (4, 5, 6))
    rows = np.array([[0, 5, 17, 31], [3, 4, 9, 30]])
    got = attention(q, k, v, mask, rows=rows)["out"][0]
    ref = _brute(q[0].tolist(), k[0].tolist(), v[0].tolist(), mask, None)
    for h in range(H):
        assert np.max(np.abs(got[h] - ref[h][rows[h]])) <= 1e-12


# ---------------------------------------------------------------------------
# special cases that reduce to a library routine (torch SDPA, float64, CPU)
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, causal=False, attn_mask=None):
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=attn_mask, is_causal=causal).numpy()


def test_v1_wide_window_equals_full():
    H, L, D = 3, 96, 16
    q, k, v = (_rand((2, H, L, D), s) for s in (7, 8, 9))
    ref = _sdpa(q, k, v)
    got = attention(q, k, v, dict(kind="window", left=L - 1, right=L - 1))["out"]
    assert np.max(np.abs(got - ref)) <= 1e-12
    got_full = attention(q, k, v, dict(kind="full"))["out"]
    assert np.max(np.abs(got_full - ref)) <= 1e-12
    # causal window of W = L keys equals causal full attention
    refc = _sdpa(q, k, v, causal=True)
    gotc = attention(q, k, v, dict(kind="window", left=L - 1, right=0, causal=True))["out"]
    assert np.max(np.abs(gotc - refc)) <= 1e-12
    gotw = attention(q, k, v, dict(kind="window", left=0, right=0, causal=True,
                                   head_left=[L - 1] * H))["out"]
    assert np.max(np.abs(gotw - refc)) <= 1e-12


def test_v2_chunk_equals_independent_chunks():
    H, L, D, C = 2, 100, 8, 32      # last chunk is ragged (4 tokens)
    q, k, v = (_rand((1, H, L, D), s) for s in (10, 11, 12))
    got = attention(q, k, v, dict(kind="chunk", chunk=C))["out"]
    for s in range(0, L, C):
        e = min(L, s + C)
        ref = _sdpa(q[:, :, s:e], k[:, :, s:e], v[:, :, s:e])
        assert np.max(np.abs(got[:, :, s:e] - ref)) <= 1e-12


def test_v5_lower_triangular_block_matrix_is_causal():
    H, L, D, bs = 2, 64, 8, 16
    q, k, v = (_rand((1, H, L, D), s) for s in (13, 14, 15))
    bm = np.tril(np.ones((1, L // bs, L // bs), np.uint8))
    got = attention(q, k, v, dict(kind="block", block=bs, block_mask=bm))["out"]
    assert np.max(np.abs(got - _sdpa(q, k, v, causal=True))) <= 1e-12
    # ragged: L not a multiple of the block size
    L2 = 60
    q2, k2, v2 = q[:, :, :L2], k[:, :, :L2], v[:, :, :L2]
    bm2 = np.tril(np.ones((1, 4, 4), np.uint8))
    got2 = attention(q2, k2, v2, dict(kind="block", block=bs, block_mask=bm2))["out"]
    assert np.max(np.abs(got2 - _sdpa(q2, k2, v2, causal=True))) <= 1e-12


def test_sink_equals_extra_zero_value_key():
    """A sink is a key with logit s_aux and a zero value: append it and use SDPA."""
    H, L, D = 2, 40, 8
    q, k, v = (_rand((1, H, L, D), s) for s in (16, 17, 18))
    sink = np.array([0.4, 2.5])
    got = attention(q, k, v, dict(kind="full"), sink=sink)
    # extra key column with score exactly s_aux: additive float mask of -inf/sink on a zero key
    kx = np.concatenate([k, np.zeros((1, H, 1, D))], axis=2)
    vx = np.concatenate([v, np.zeros((1, H, 1, D))], axis=2)
    am = np.zeros((1, H, L, L + 1))
    am[0, :, :, L] = sink[:, None]
    ref = _sdpa(q, kx, vx, attn_mask=torch.from_numpy(am))
    assert np.max(np.abs(got["out"] - ref)) <= 1e-12


# ---------------------------------------------------------------------------
# closed forms and invariants
# ---------------------------------------------------------------------------

MASKS_MED = [
    dict(kind="full"),
    dict(kind="chunk", chunk=16),
    dict(kind="window", left=9, right=9),
    dict(kind="window", left=0, right=0, causal=True, head_left=[5, 17, 63]),
    dict(kind="block", block=16, block_mask=np.array([np.tril(np.random.default_rng(3).integers(0, 2, (4, 4))).astype(np.uint8) | np.eye(4, dtype=np.uint8)])),
]


@pytest.mark.parametrize("mi", range(len(MASKS_MED)))
def test_v3_rows_sum_to_one_minus_sink(mi):
    H, L, D = 3, 64, 16
    q, k, v = (_rand((1, H, L, D), s) for s in (19, 20, 21))
    r0 = attention(q, k, v, MASKS_MED[mi])
    assert np.max(np.abs(r0["rowsum"] - 1.0)) <= 1e-12
    sink = np.array([-0.5, 0.0, 1.5])
    r1 = attention(q, k, v, MASKS_MED[mi], sink=sink)
    assert np.max(np.abs(r1["rowsum"] + r1["sink_mass"] - 1.0)) <= 1e-12
    assert np.all(r1["sink_mass"] > 0)


@pytest.mark.parametrize("mi", range(len(MASKS_MED)))
def test_closed_form_v_ones(mi):
    """V = 1 gives o_i = 1 - pi_i in every component."""
    H, L, D = 3, 64, 16
    q, k = _rand((1, H, L, D), 22), _rand((1, H, L, D), 23)
    v = np.ones((1, H, L, D))
    sink = np.array([0.3, -2.0, 1.0])
    r = attention(q, k, v, MASKS_MED[mi], sink=sink)
    assert np.max(np.abs(r["out"] - (1.0 - r["sink_mass"])[..., None])) <= 1e-12


@pytest.mark.parametrize("mi", range(len(MASKS_MED)))
def test_closed_form_equal_keys(mi):
    """All keys equal: weights are uniform over N(i); pi_i = e^{s_aux}/(e^{s_aux} + n_i e^{s_i})."""
    H, L, D = 3, 64, 16
    q, v = _rand((1, H, L, D), 24), _rand((1, H, L, D), 25)
    k = np.broadcast_to(_rand((1, H, 1, D), 26), (1, H, L, D)).copy()
    sink = np.array([0.9, -0.1, 0.0])
    got = attention(q, k, v, MASKS_MED[mi], sink=sink)["out"]
    mask = MASKS_MED[mi]
    for h in range(H):
        for i in range(L):
            ks = _keys_brute(mask, h, i, L)
            s = float(q[0, h, i] @ k[0, h, 0]) / math.sqrt(D)
            n = len(ks)
            pi = math.exp(sink[h]) / (math.exp(sink[h]) + n * math.exp(s))
            exp_o = (1.0 - pi) * v[0, h, ks].mean(axis=0)
            assert np.max(np.abs(got[0, h, i] - exp_o)) <= 1e-12


@pytest.mark.parametrize("mask", [dict(kind="window", left=0, right=0),
                                  dict(kind="chunk", chunk=1),
                                  dict(kind="window", left=0, right=0, causal=True, head_left=[0, 0])])
def test_closed_form_self_only(mask):
    """r = 0, C = 1 or W = 1: o_i = (1 - pi_i) v_i with pi_i = e^{s_aux}/(e^{s_aux} + e^{s_ii})."""
    H, L, D = 2, 24, 8
    q, k, v = (_rand((1, H, L, D), s) for s in (27, 28, 29))
    sink = np.array([0.5, -1.0])
    got = attention(q, k, v, mask, sink=sink)["out"]
    s = np.einsum("bhld,bhld->bhl", q, k) / math.sqrt(D)
    pi = np.exp(sink)[None, :, None] / (np.exp(sink)[None, :, None] + np.exp(s))
    assert np.max(np.abs(got - (1 - pi)[..., None] * v)) <= 1e-12


def test_full_mask_permutation_equivariant():
    """Without a mask, permuting tokens permutes outputs (lesson page, section 4)."""
    H, L, D = 2, 50, 8
    q, k, v = (_rand((1, H, L, D), s) for s in (30, 31, 32))
    perm = np.random.default_rng(33).permutation(L)
    a = attention(q, k, v, dict(kind="full"))["out"]
    b = attention(q[:, :, perm], k[:, :, perm], v[:, :, perm], dict(kind="full"))["out"]
    assert np.max(np.abs(a[:, :, perm] - b)) <= 1e-12


def test_neg_inf_sink_is_no_sink():
    H, L, D = 2, 40, 8
    q, k, v = (_rand((1, H, L, D), s) for s in (34, 35, 36))
    m = dict(kind="window", left=4, right=7)
    a = attention(q, k, v, m)["out"]
    b = attention(q, k, v, m, sink=np.array([-np.inf, -np.inf]))["out"]
    assert np.array_equal(a, b)


def test_empty_rows_give_zero():
    """A block row with no kept block has no allowed key: o_i = 0, also with a sink."""
    mask = BRUTE_MASKS[-1]           # block row 3 is empty
    H, L, D = 1, 32, 8
    q, k, v = (_rand((1, H, L, D), s) for s in (37, 38, 39))
    for sink in (None, np.array([0.2])):
        out = attention(q, k, v, mask, sink=sink)["out"]
        assert np.all(out[0, 0, 15:20] == 0.0)
        assert np.all(np.isfinite(out))


def test_bf16_decode_exact():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4049, 0x7F80, 0x0001], dtype=np.uint16)
    vals = oracle.bf16_to_f64(bits)
    assert vals[0] == 0.0 and vals[2] == 1.0 and vals[3] == -1.0
    assert vals[4] == 3.140625 and np.isinf(vals[5])
    assert vals[6] == 2.0 ** -133


# ---------------------------------------------------------------------------
# mask predicates against the pages' worked example, and pair counts
# ---------------------------------------------------------------------------

def test_swa_worked_example_from_pages():
    g = json.load(open(GOLDEN))["swa_worked_example"]
    L = 64
    mask = dict(kind="window", left=g["per_side"], right=g["per_side"])
    for case in g["cases"]:
        row = allowed_rows(mask, 0, np.array([case["anchor"]]), L)[0]
        keys = np.nonzero(row)[0]
        assert keys[0] == case["first"] and keys[-1] == case["last"]
        assert len(keys) == case["last"] - case["first"] + 1


def _closed_pairs(mask, L):
    kind = mask["kind"]
    if kind == "full":
        return L * L if not mask.get("causal") else L * (L + 1) // 2
    if kind == "chunk":
        c = mask["chunk"]
        full, rem = divmod(L, c)
        return full * c * c + rem * rem
    if kind == "window" and not mask.get("causal"):
        r = mask["left"]
        assert mask["right"] == r
        return L * (2 * r + 1) - r * (r + 1)
    if kind == "window":
        w = mask["left"] + 1
        return w * L - w * (w - 1) // 2
    raise ValueError


@pytest.mark.parametrize("mask,L", [
    (dict(kind="full"), 300), (dict(kind="full", causal=True), 300),
    (dict(kind="chunk", chunk=64), 256), (dict(kind="chunk", chunk=48), 300),
    (dict(kind="window", left=17, right=17), 300), (dict(kind="window", left=128, right=128), 4096),
    (dict(kind="window", left=511, right=0, causal=True), 4096),
    (dict(kind="window", left=4095, right=0, causal=True), 4096),
])
def test_pair_count_closed_forms(mask, L):
    assert pair_count(mask, 1, L)[0] == _closed_pairs(mask, L)


def test_pair_count_block_closed_form():
    # block matrix with the structure used at 128K (diagonal + first block + half of the rest),
    # at a smaller size: pairs = nb * bs(bs+1)/2 + (kept off-diagonal blocks) * bs^2
    from block_sparse_softmax_amd.inputs import block_matrix_top_half
    bs, nb = 16, 24
    bm = block_matrix_top_half(0, 5, 1, nb)
    mask = dict(kind="block", block=bs, block_mask=bm)
    off = int(bm[0].sum()) - nb
    assert pair_count(mask, 1, nb * bs)[0] == nb * bs * (bs + 1) // 2 + off * bs * bs


def test_page_token_counts_and_flops():
    g = json.load(open(GOLDEN))
    for c in g["vit_token_counts"]["cases"]:
        assert (c["px"] // g["vit_token_counts"]["patch_px"]) ** 2 == c["tokens"]
    f = g["vit_attention_tflops"]
    for c in f["cases"]:
        L = c["tokens"]
        pairs = int(pair_count(dict(kind="full"), 1, L)[0])
        tflops = 16 * pairs * f["heads"] * f["head_dim"] * f["layers"] / 1e12
        assert round(tflops, c["decimals"]) == c["tflops"]
    a = g["ariadne_tflops"]
    L = a["tokens"]
    full = int(pair_count(dict(kind="full"), 1, L)[0])
    swa = int(pair_count(dict(kind="window", left=a["per_side"], right=a["per_side"]), 1, L)[0])
    t = 16 * f["heads"] * f["head_dim"] * (a["local_layers"] * swa + a["full_layers"] * full) / 1e12
    assert round(t, 2) == a["tflops"]
    # the other reading (a 128-key window, 64 left and 63 right) would print 1.67T
    swa_excl = int(pair_count(dict(kind="window", left=64, right=63), 1, L)[0])
    t2 = 16 * f["heads"] * f["head_dim"] * (a["local_layers"] * swa_excl + a["full_layers"] * full) / 1e12
    assert round(t2, 2) != a["tflops"]
    s = g["scores_per_head"]
    assert round(pair_count(dict(kind="full"), 1, s["tokens"])[0] / 1e6, 1) == s["millions"]
    for c in g["vit_lesson_pairs"]["cases"]:
        n = (c["px"] // c["patch"]) ** 2
        assert n == c["tokens"]
        pairs = int(pair_count(dict(kind="full"), 1, n)[0])
        assert abs(pairs - c["approx_entries"]) <= c["rel_tol"] * c["approx_entries"]


# ---------------------------------------------------------------------------
# tile lists
# ---------------------------------------------------------------------------

def _tiles_brute(mask, H, L, bm, bn):
    rp, kv, fl = [0], [], []
    M = [dense_mask(mask, h, L) for h in range(H)]
    nq, nk = -(-L // bm), -(-L // bn)
    for h in range(H):
        for qt in range(nq):
            for kt in range(nk):
                cnt, tot = 0, 0
                for i in range(qt * bm, (qt + 1) * bm):
                    for j in range(kt * bn, (kt + 1) * bn):
                        tot += 1
                        if i < L and j < L and M[h][i, j]:
                            cnt += 1
                if cnt:
                    kv.append(kt)
                    fl.append(1 if cnt == tot else 0)
            rp.append(len(kv))
    return np.array(rp, np.int32), np.array(kv, np.int32), np.array(fl, np.uint8)


@pytest.mark.parametrize("mi", range(len(BRUTE_MASKS)))
@pytest.mark.parametrize("bm,bn", [(8, 8), (16, 8), (8, 16), (12, 20)])
def test_tile_lists_dense_vs_brute(mi, bm, bn):
    mask = BRUTE_MASKS[mi]
    H = 2 if (mask["kind"] != "block" or len(mask["block_mask"]) > 1) else 1
    L = 32 if mask["kind"] != "block" or mask["block"] == 8 else 35
    a = tile_lists_dense(mask, H, L, bm, bn)
    b = _tiles_brute(mask, H, L, bm, bn)
    for x, y in zip(a, b):
        assert x.dtype == y.dtype and np.array_equal(x, y)


def test_tile_lists_block_vs_dense():
    from block_sparse_softmax_amd.inputs import block_matrix_top_half
    bs, nb, H = 16, 20, 3
    mask = dict(kind="block", block=bs, block_mask=block_matrix_top_half(0, 5, H, nb))
    for L in (nb * bs, nb * bs - 5):
        for bm, bn in ((16, 16), (16, 8), (8, 16), (4, 2), (2, 8)):
            a = tile_lists_block(mask, H, L, bm, bn)
            b = tile_lists_dense(mask, H, L, bm, bn)
            for x, y in zip(a, b):
                assert np.array_equal(x, y)


def test_block_matrix_generator_shape():
    from block_sparse_softmax_amd.inputs import block_matrix_top_half
    bm = block_matrix_top_half(0, 5, 2, 1024)
    assert bm.shape == (2, 1024, 1024)
    assert np.all(np.triu(bm[0], 1) == 0)
    assert np.all(bm[:, :, 0] == 1) and np.all(bm[:, np.arange(1024), np.arange(1024)] == 1)
    # 263,679 kept causal blocks per head: nb diagonal + first-column + ceil((m-1)/2) per row
    exp = 1 + 2 + sum(2 + (m) // 2 for m in range(2, 1024))
    assert int(bm[0].sum()) == exp == 263679
