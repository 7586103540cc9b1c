"""GPU re-permutation of tokens between serialisation orders (attn_reorder_tokens) against the
oracle's explicit-loop orders: a copy, so bit-exact."""

import numpy as np
import pytest
import torch

from oracle.serialize import ORDERS, reorder

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gh,gw,H,D", [(8, 6, 3, 64), (64, 64, 16, 80), (10, 4, 2, 128), (128, 128, 2, 8)])
def test_reorder_bit_exact(gh, gw, H, D):
    from block_sparse_softmax_amd import reorder_tokens
    L = gh * gw
    x = np.random.default_rng(gh + gw).integers(0, 1 << 16, (2, L, H, D)).astype(np.uint16)
    xt = torch.from_numpy(x.view(np.int16)).cuda()
    for a in ORDERS:
        for b in ORDERS:
            got = reorder_tokens(xt.view(torch.bfloat16), a, b, gh, gw)
            torch.cuda.synchronize()
            want = reorder(x, a, b, gh, gw, axis=1)
            assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), want), (a, b)


def test_reorder_bhld_views_and_round_trip():
    from block_sparse_softmax_amd import reorder_tokens
    gh, gw, H, D = 16, 12, 4, 80
    L = gh * gw
    x = torch.randn(1, H, L, D, device="cuda").to(torch.bfloat16)
    y = reorder_tokens(x, "block_row", "block_col", gh, gw, layout="bhld")
    z = reorder_tokens(y, "block_col", "block_row", gh, gw, layout="bhld")
    torch.cuda.synchronize()
    assert torch.equal(z, x)
    want = reorder(x.view(torch.int16).cpu().numpy(), "block_row", "block_col", gh, gw, axis=2)
    assert np.array_equal(y.view(torch.int16).cpu().numpy(), want)
