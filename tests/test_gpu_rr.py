"""GPU parity of RRAttention's block-pattern search (attn_rr_search) against the float64 oracle.

Block scores: compared with the plain float64 oracle of Eq. 6-10 (stride sums of the keys in
float64), each within the bound that tests/rr_tolerance.py derives from the kernel's stated
precision (fp32 stride sums carried as a bf16 hi + lo pair, bf16 products, fp32 accumulation and
softmax).  Block matrix: a floating-point decision (a sort and a threshold), so each row is checked
to be a valid top-tau selection of the oracle's scores within the row's summed bound (the mass
reaches tau, no selected block is superfluous, no unselected block is clearly larger), and must
equal the oracle's row wherever no decision lies within the bound.  The last query block is
protected exactly."""

import numpy as np
import pytest
import torch

from block_sparse_softmax_amd import inputs as gen
from oracle.rr_search import rr_search as rr_oracle

from rr_tolerance import score_tolerance

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _random(seed, B, H, L, D):
    rng = np.random.default_rng(seed)
    return tuple(gen.f32_to_bf16_bits(rng.standard_normal((B, H, L, D), dtype=np.float32)) for _ in range(2))


def _planted(seed, H, L, D, Bs):
    """Queries share a direction u; the keys of a few chosen blocks per head point along it."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((1, H, L, D)) + 3.0 * u
    k = rng.standard_normal((1, H, L, D))
    nb = -(-L // Bs)
    for h in range(H):
        for n in rng.choice(max(1, nb - 1), size=min(3, max(1, nb - 1)), replace=False):
            k[0, h, n * Bs:(n + 1) * Bs] += 6.0 * u
    return tuple(gen.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k))


def _check_row(sel, s, tau, eps):
    """sel: GPU row (0/1 over n <= m); s: oracle scores (n <= m).  Returns True if the decision is
    clear (then sel must equal the oracle's own selection)."""
    T = s.sum()
    G = np.flatnonzero(sel)
    if T <= 0:
        assert G.size == 0
        return True
    mass = s[G].sum()
    assert G.size > 0 and mass >= tau * T - eps, (mass, tau * T)
    assert mass - s[G].min() < tau * T + eps, "a selected block is superfluous"
    rest = np.setdiff1d(np.arange(s.size), G)
    if rest.size:
        assert s[rest].max() <= s[G].min() + eps, "a larger block was left out"
    # clear decision: the sorted prefix sums stay away from the threshold and no near-ties cross it
    order = np.argsort(-s, kind="stable")
    cs = np.cumsum(s[order])
    k = int(np.searchsorted(cs, tau * T))
    k = min(k, s.size - 1)
    clear = (cs[k] - tau * T > eps) and (k == 0 or tau * T - cs[k - 1] > eps)
    if k + 1 < s.size:
        clear = clear and (s[order[k]] - s[order[k + 1]] > eps)
    return clear


CASES = [
    # (L, H, D, S, Bs, tau, kind)
    (2048, 3, 128, 8, 128, 0.9, "random"),
    (2000, 2, 64, 8, 128, 0.5, "random"),      # ragged last block
    (1030, 2, 80, 4, 128, 0.9, "random"),      # ragged last stride, 32 strides per block
    (1024, 2, 128, 16, 128, 0.95, "random"),   # 8 strides per block
    (4096, 4, 128, 8, 128, 0.5, "planted"),
    (2048, 2, 64, 8, 128, 1.0, "random"),      # tau = 1: every block with mass
    (8200, 1, 64, 1, 8, 0.5, "planted"),       # 1025 blocks per row (the select kernel's wide variant)
    (2052, 2, 64, 8, 128, 0.9, "random"),      # 256 strides; the 17th block holds no sampled query
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_rr_search_parity(ci):
    from block_sparse_softmax_amd import rr_search
    L, H, D, S, Bs, tau, kind = CASES[ci]
    print(f"[case] rr search L={L} H={H} D={D} S={S} Bs={Bs} tau={tau} {kind}", flush=True)
    q, k = _random(50 + ci, 1, H, L, D) if kind == "random" else _planted(60 + ci, H, L, D, Bs)
    bm, sc = rr_search(_dev(q), _dev(k), S, Bs, tau, layout="bhld")
    torch.cuda.synchronize()
    bm, sc = bm.cpu().numpy(), sc.cpu().numpy().astype(np.float64)
    nb = -(-L // Bs)
    worst, clear_rows, rows = 0.0, 0, 0
    for h in range(H):
        s_ref, b_ref = rr_oracle(q, k, S, Bs, tau, h=h)
        tol = score_tolerance(q, k, S, Bs, h)
        err = np.abs(sc[0, h] - s_ref)
        worst = max(worst, float((err / np.maximum(tol, 1e-300)).max()))
        assert np.all(np.triu(sc[0, h], 1) == 0) and np.all(np.triu(bm[0, h], 1) == 0)
        assert np.all(err <= tol), (h, float((err - tol).max()))
        for m in range(nb - 1):
            eps = float(tol[m].sum())
            if tau == 1.0:
                # the whole mass: exactly the blocks with a positive score (here every causal block);
                # no row has a clear decision in the sense of _check_row, whose band is the threshold
                assert np.array_equal(bm[0, h, m, : m + 1], (s_ref[m, : m + 1] > 0).astype(np.uint8)), (h, m)
                continue
            clear = _check_row(bm[0, h, m, : m + 1], s_ref[m, : m + 1], tau, eps)
            rows += 1
            if clear:
                clear_rows += 1
                assert np.array_equal(bm[0, h, m], b_ref[m]), (h, m)
        assert np.all(bm[0, h, nb - 1] == 1)
    print(f"[rr] max |dS| / bound = {worst:.2e}; {clear_rows}/{rows} rows with a clear decision, all equal",
          flush=True)
    # every row passed the validity checks; rows of about a thousand blocks hold many scores within the
    # decision band of each other, so fewer of them are clear (a few percent here, most at nb <= 64)
    assert clear_rows >= (0.5 if nb <= 64 else 0.02) * rows


def test_rr_search_128k_sampled_blocks():
    """The 128K-token shape (32 heads, d = 128, stride 8, block 128, tau 0.9): GPU search over every
    head; the oracle on 8 seeded query blocks of 4 heads."""
    from block_sparse_softmax_amd import RrSearch
    L, H, D, S, Bs, tau = 131072, 32, 128, 8, 128, 0.9
    print("[case] rr search 128k: generating inputs", flush=True)
    q = np.stack([gen.gaussian_bf16(0, 5, gen.Q_ID, h, (1, L, D)) for h in range(H)], axis=1)
    k = np.stack([gen.gaussian_bf16(0, 5, gen.K_ID, h, (1, L, D)) for h in range(H)], axis=1)
    qt, kt = _dev(q), _dev(k)
    srch = RrSearch(qt, S, Bs, tau, layout="bhld")
    bm, sc = srch(qt, kt)
    torch.cuda.synchronize()
    nb = L // Bs
    rng = np.random.default_rng(7)
    for h in (0, 9, 18, 31):
        blocks = np.sort(rng.choice(nb - 1, size=8, replace=False))
        s_ref, b_ref = rr_oracle(q, k, S, Bs, tau, h=h, query_blocks=blocks)
        tol = score_tolerance(q, k, S, Bs, h, query_blocks=blocks)
        s_gpu = sc[0, h].cpu().numpy().astype(np.float64)
        b_gpu = bm[0, h].cpu().numpy()
        for m in blocks:
            err = np.abs(s_gpu[m] - s_ref[m])
            assert np.all(err <= tol[m]), (h, m, float((err - tol[m]).max()))
            if _check_row(b_gpu[m, : m + 1], s_ref[m, : m + 1], tau, float(tol[m].sum())):
                assert np.array_equal(b_gpu[m], b_ref[m]), (h, m)
        assert np.all(b_gpu[nb - 1] == 1)
    print(f"[rr] 128k: density of the selected blocks {bm.float().mean().item() * 2:.3f} of the causal half", flush=True)


def test_rr_search_grouped_keys():
    """Grouped-query attention: 4 query heads on 2 key heads (query head h reads key head h // 2)."""
    from block_sparse_softmax_amd import rr_search
    L, H, Hk, D, S, Bs, tau = 2048, 4, 2, 128, 8, 128, 0.9
    rng = np.random.default_rng(77)
    q = gen.f32_to_bf16_bits(rng.standard_normal((1, H, L, D), dtype=np.float32))
    k = gen.f32_to_bf16_bits(rng.standard_normal((1, Hk, L, D), dtype=np.float32))
    bm, sc = rr_search(_dev(q), _dev(k), S, Bs, tau, layout="bhld")
    torch.cuda.synchronize()
    bm, sc = bm.cpu().numpy(), sc.cpu().numpy().astype(np.float64)
    for h in range(H):
        s_ref, b_ref = rr_oracle(q, k, S, Bs, tau, h=h)
        tol = score_tolerance(q, k, S, Bs, h)
        assert np.all(np.abs(sc[0, h] - s_ref) <= tol)
        for m in range(L // Bs - 1):
            if _check_row(bm[0, h, m, : m + 1], s_ref[m, : m + 1], tau, float(tol[m].sum())):
                assert np.array_equal(bm[0, h, m], b_ref[m]), (h, m)


def test_rr_search_batch():
    """Batch 2 with different data per batch element (the single pass's grid walks batch and head in one
    index): every (b, h) against the oracle of its own element, and the rows with a clear decision equal."""
    from block_sparse_softmax_amd import rr_search
    B, L, H, D, S, Bs, tau = 2, 2000, 2, 64, 8, 128, 0.9
    print(f"[case] rr search batch B={B} L={L} H={H} D={D}", flush=True)
    q, k = _random(88, B, H, L, D)
    bm, sc = rr_search(_dev(q), _dev(k), S, Bs, tau, layout="bhld")
    torch.cuda.synchronize()
    bm, sc = bm.cpu().numpy(), sc.cpu().numpy().astype(np.float64)
    nb = -(-L // Bs)
    clear = 0
    for b in range(B):
        for h in range(H):
            s_ref, b_ref = rr_oracle(q, k, S, Bs, tau, b=b, h=h)
            tol = score_tolerance(q, k, S, Bs, h, b=b)
            assert np.all(np.abs(sc[b, h] - s_ref) <= tol), (b, h)
            assert np.all(bm[b, h, nb - 1] == 1)
            for m in range(nb - 1):
                if _check_row(bm[b, h, m, : m + 1], s_ref[m, : m + 1], tau, float(tol[m].sum())):
                    clear += 1
                    assert np.array_equal(bm[b, h, m], b_ref[m]), (b, h, m)
    assert clear >= 0.5 * B * H * (nb - 1)


@pytest.mark.parametrize("L,H,big", [(8192, 1, 20.0), (8192, 1, 25.0), (2048, 2, 400.0)])
def test_rr_search_recompute_path(L, H, big):
    """Queries live in the first half of the head dim; one key of some strides carries a large component
    in the second half, orthogonal to every query.  Those keys put the single pass's fixed reference
    (|q| times the largest key-aggregate norm) far above the rows' maxima: rows whose sum against it
    falls below 2^-40 send their 128-row query tile to the two-pass recompute.  On the CPU these inputs
    flag no tile (big = 20: the reference about 35 log2 units above the maxima), 6 of 8 tiles (25) and
    every tile (400); the scores must match the oracle within the derived bound in all three."""
    from block_sparse_softmax_amd import rr_search
    D, S, Bs, tau = 128, 8, 64, 0.9
    rng = np.random.default_rng(int(big))
    q = rng.standard_normal((1, H, L, D))
    q[..., D // 2:] = 0.0
    k = rng.standard_normal((1, H, L, D))
    hot = rng.choice(L, size=L // 64, replace=False)
    k[:, :, hot, D // 2:] += big * rng.standard_normal((1, H, hot.size, D // 2))
    q, k = (gen.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k))
    print(f"[case] rr search recompute path L={L} big={big}", flush=True)
    bm, sc = rr_search(_dev(q), _dev(k), S, Bs, tau, layout="bhld")
    torch.cuda.synchronize()
    bm, sc = bm.cpu().numpy(), sc.cpu().numpy().astype(np.float64)
    nb = L // Bs
    for h in range(H):
        s_ref, b_ref = rr_oracle(q, k, S, Bs, tau, h=h)
        tol = score_tolerance(q, k, S, Bs, h)
        err = np.abs(sc[0, h] - s_ref)
        assert np.all(err <= tol), (h, float((err - tol).max()))
        np.testing.assert_allclose(sc[0, h].sum(axis=1), Bs // S, rtol=1e-5)   # every row's mass is there
        for m in range(nb - 1):
            if _check_row(bm[0, h, m, : m + 1], s_ref[m, : m + 1], tau, float(tol[m].sum())):
                assert np.array_equal(bm[0, h, m], b_ref[m]), (h, m)
