"""Pins for the float64 gradient oracle (oracle/backward.py): central finite differences of the
forward definition, the autograd of a library attention on the full mask, closed-form invariants
of the softmax's shift and scale symmetries, and the log-sum-exp against scipy.  CPU only."""

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle.attention import attention, dense_mask
from oracle.backward import attention_backward

MASKS = [
    dict(kind="full"),
    dict(kind="full", causal=True),
    dict(kind="chunk", chunk=5),                                     # ragged last chunk
    dict(kind="window", left=3, right=1, head_left=[1, 4]),         # per-head left extents
    dict(kind="window", left=4, right=0, causal=True, prefix=2),    # StreamingLLM prefix + window
    dict(kind="block", block=4, block_mask=np.array([[[1, 0, 0, 0], [0, 0, 0, 0],   # an empty block row
                                                      [1, 0, 1, 0], [0, 1, 1, 1]]], np.uint8)),
]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, dout, mask, sink):
    """The scalar whose gradients the oracle returns: sum over all outputs of dO * O."""
    return float((attention(q, k, v, mask, sink=sink)["out"] * dout).sum())


def _fd(f, x, eps=1e-5):
    """Central differences of f with respect to every element of x (modified in place, restored)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        x0 = x[idx]
        x[idx] = x0 + eps
        fp = f()
        x[idx] = x0 - eps
        fm = f()
        x[idx] = x0
        g[idx] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("mi", range(len(MASKS)))
@pytest.mark.parametrize("with_sink", [False, True])
def test_finite_differences(mi, with_sink):
    mask = MASKS[mi]
    H, L, D = 2, 16, 4
    q, k, v, do = (_rand((1, H, L, D), s) for s in (11, 12, 13, 14))
    sink = np.array([0.4, -0.9]) if with_sink else None
    g = attention_backward(q, k, v, do, mask, sink=sink)
    f = lambda: _loss(q, k, v, do, mask, sink)
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        np.testing.assert_allclose(g[name], _fd(f, x), rtol=0, atol=2e-8, err_msg=name)
    if with_sink:
        np.testing.assert_allclose(g["dsink"], _fd(f, sink), rtol=0, atol=2e-8)
    else:
        assert g["dsink"] is None
    np.testing.assert_allclose(g["out"], attention(q, k, v, mask, sink=sink)["out"], rtol=0, atol=1e-13)


def test_finite_differences_grouped_heads():
    """Query heads 0-2 share K/V head 0 and 3-5 share head 1: their K/V gradients add up."""
    H, Hk, L, D = 6, 2, 12, 4
    mask = dict(kind="window", left=3, right=2, prefix=1)
    q, do = _rand((1, H, L, D), 21), _rand((1, H, L, D), 22)
    k, v = _rand((1, Hk, L, D), 23), _rand((1, Hk, L, D), 24)
    sink = np.linspace(-1.0, 1.0, H)
    g = attention_backward(q, k, v, do, mask, sink=sink)
    f = lambda: _loss(q, k, v, do, mask, sink)
    for name, x in (("dq", q), ("dk", k), ("dv", v), ("dsink", sink)):
        np.testing.assert_allclose(g[name], _fd(f, x), rtol=0, atol=2e-8, err_msg=name)


def test_explicit_scale():
    mask = dict(kind="chunk", chunk=4)
    q, k, v, do = (_rand((1, 1, 8, 4), s) for s in (31, 32, 33, 34))
    g = attention_backward(q, k, v, do, mask, scale=0.3)
    f = lambda: float((attention(q, k, v, mask, scale=0.3)["out"] * do).sum())
    np.testing.assert_allclose(g["dq"], _fd(f, q), rtol=0, atol=2e-8)
    np.testing.assert_allclose(g["dk"], _fd(f, k), rtol=0, atol=2e-8)


def test_library_autograd_full_mask():
    """On the full (and causal) mask without a sink the op is PyTorch's scaled dot-product
    attention; its autograd in float64 gives the same gradients."""
    B, H, L, D = 2, 3, 24, 8
    q, k, v, do = (_rand((B, H, L, D), s) for s in (41, 42, 43, 44))
    for causal in (False, True):
        g = attention_backward(q, k, v, do, dict(kind="full", causal=causal))
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
        o.backward(torch.tensor(do))
        for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
            np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=0, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_symmetry_invariants(mi):
    """Adding c to every key adds sigma q_i.c to each logit of row i; only the sink's share of the
    row moves, so sum_j dK_j = sigma sum_i pi_i D_i q_i (0 without a sink).  Scaling q by t and k by
    1/t changes nothing: sum_i q_i.dQ_i = sum_j k_j.dK_j.  Summing dV over keys gives
    sum_i (1 - pi_i) dO_i."""
    mask = MASKS[mi]
    H, L, D = 2, 16, 6
    q, k, v, do = (_rand((1, H, L, D), s) for s in (51, 52, 53, 54))
    for sink in (None, np.array([1.5, -0.5])):
        g = attention_backward(q, k, v, do, mask, sink=sink)
        fw = attention(q, k, v, mask, sink=sink)
        pi, Di = fw["sink_mass"][0], (fw["out"][0] * do[0]).sum(axis=-1)
        sigma = 1 / np.sqrt(D)
        for h in range(H):
            lhs = g["dk"][0, h].sum(axis=0)
            np.testing.assert_allclose(lhs, sigma * ((pi[h] * Di[h])[:, None] * q[0, h]).sum(axis=0),
                                       rtol=0, atol=1e-12)
            np.testing.assert_allclose((q[0, h] * g["dq"][0, h]).sum(), (k[0, h] * g["dk"][0, h]).sum(),
                                       rtol=0, atol=1e-12)
            has_key = dense_mask(mask, h, L).any(axis=1)
            w = np.where(has_key, 1 - pi[h], 0.0)
            np.testing.assert_allclose(g["dv"][0, h].sum(axis=0), (w[:, None] * do[0, h]).sum(axis=0),
                                       rtol=0, atol=1e-12)
        if sink is None:
            assert np.abs(g["dk"].sum(axis=2)).max() <= 1e-12


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_lse(mi):
    """The log-sum-exp of each row over its allowed logits and the sink, against scipy."""
    mask = MASKS[mi]
    H, L, D = 2, 16, 4
    q, k, v, do = (_rand((1, H, L, D), s) for s in (61, 62, 63, 64))
    sink = np.array([0.2, 3.0])
    for sk in (None, sink):
        g = attention_backward(q, k, v, do, mask, sink=sk)
        for h in range(H):
            s = (q[0, h] @ k[0, h].T) / np.sqrt(D)
            s = np.where(dense_mask(mask, h, L), s, -np.inf)
            if sk is not None:
                s = np.concatenate([s, np.full((L, 1), sk[h])], axis=1)
            with np.errstate(divide="ignore"):
                ref = logsumexp(s, axis=1)
            np.testing.assert_allclose(g["lse"][0, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mi", range(len(MASKS)))
def test_sampled_rows_and_columns(mi):
    """The row-sampled dQ and column-sampled dK/dV (for long sequences) equal the full gradients'
    rows and columns, with and without a sink and with grouped heads."""
    from oracle.backward import dkdv_cols, dq_rows, lse_rows
    mask = MASKS[mi]
    H, Hk, L, D = 2, 1, 16, 4
    q, do = _rand((2, H, L, D), 71), _rand((2, H, L, D), 72)
    for hk_n, sink in ((H, None), (Hk, np.array([0.3, -1.2]))):
        k, v = _rand((2, hk_n, L, D), 73), _rand((2, hk_n, L, D), 74)
        g = attention_backward(q, k, v, do, mask, sink=sink)
        rows = np.array([[0, 5, 15], [3, 4, 9]])
        np.testing.assert_allclose(dq_rows(q, k, v, do, mask, rows, sink=sink),
                                   np.take_along_axis(g["dq"], rows[None, :, :, None], axis=2), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse_rows(q, k, mask, rows, sink=sink), np.take_along_axis(g["lse"], rows[None], axis=2),
                                   rtol=0, atol=1e-12)
        cols = np.array([[1, 8, 14], [0, 7, 15]])[:hk_n]
        dk, dv = dkdv_cols(q, k, v, do, mask, cols, sink=sink, row_chunk=5)
        np.testing.assert_allclose(dk, np.take_along_axis(g["dk"], cols[None, :, :, None], axis=2), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, np.take_along_axis(g["dv"], cols[None, :, :, None], axis=2), rtol=0, atol=1e-12)
        if mask.get("causal"):   # rows before the first key cannot see it
            dk2, dv2 = dkdv_cols(q, k, v, do, mask, cols, sink=sink, first_row=int(cols.min()))
            np.testing.assert_allclose(dk2, dk, rtol=0, atol=1e-12)
            np.testing.assert_allclose(dv2, dv, rtol=0, atol=1e-12)
