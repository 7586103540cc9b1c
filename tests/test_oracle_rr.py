"""Pins for the float64 oracle of RRAttention's pattern search (oracle/rr_search.py): the closed
form of Eq. 6, brute-force loops for Eq. 8-10, hand-worked top-tau selections, invariants, the
last-row protection and a planted pattern.  CPU only."""

import math

import numpy as np
import pytest

from oracle.rr_search import block_scores, rr_search, sample_positions, stride_importance, stride_softmax, top_tau


def test_sample_positions_closed_form():
    # S = 4, L = 16: P(i, h) = 4i + 3 - (h mod 4)
    assert sample_positions(16, 4, 0).tolist() == [3, 7, 11, 15]
    assert sample_positions(16, 4, 1).tolist() == [2, 6, 10, 14]
    assert sample_positions(16, 4, 3).tolist() == [0, 4, 8, 12]
    assert sample_positions(16, 4, 5).tolist() == sample_positions(16, 4, 1).tolist()
    # only full strides are sampled
    assert sample_positions(18, 4, 0).tolist() == [3, 7, 11, 15]


@pytest.mark.parametrize("S", [1, 2, 4, 8, 16])
def test_sampling_is_round_robin(S):
    """S consecutive heads sample every position of every stride exactly once."""
    L = 5 * S + 3
    seen = np.sort(np.concatenate([sample_positions(L, S, h) for h in range(7, 7 + S)]))
    assert seen.tolist() == list(range((L // S) * S))


def _brute_pipeline(q, k, S, Bs, h, all_strides=False):
    """Eq. 8-10 with explicit loops (tiny inputs only); all_strides: Eq. 9 over every key stride."""
    L, d = len(q), len(q[0])
    ns = L // S
    I = [[0.0] * ns for _ in range(ns)]
    for i in range(ns):
        p = i * S + (S - 1 - (h % S))
        for j in range(ns):
            acc = 0.0
            for kk in range(j * S, (j + 1) * S):
                for c in range(d):
                    acc += q[p][c] * k[kk][c]
            I[i][j] = acc / (S * math.sqrt(d))
    P = [[0.0] * ns for _ in range(ns)]
    for i in range(ns):
        keys = range(ns) if all_strides else range(i + 1)
        mx = max(I[i][j] for j in keys)
        z = sum(math.exp(I[i][j] - mx) for j in keys)
        for j in keys:
            P[i][j] = math.exp(I[i][j] - mx) / z
    nb = -(-L // Bs)
    B = [[0.0] * nb for _ in range(nb)]
    for i in range(ns):
        for j in range(ns):
            B[(i * S) // Bs][(j * S) // Bs] += P[i][j]
    return np.array(I), np.array(P), np.array(B)


@pytest.mark.parametrize("L,S,Bs,d,h", [(32, 4, 8, 3, 0), (37, 4, 16, 5, 2), (40, 2, 8, 4, 7), (24, 8, 8, 2, 1)])
def test_pipeline_against_brute_force(L, S, Bs, d, h):
    rng = np.random.default_rng(L + S + d)
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    I0, P0, B0 = _brute_pipeline(q.tolist(), k.tolist(), S, Bs, h)
    I = stride_importance(q, k, S, h)
    P = stride_softmax(I)
    nb = -(-L // Bs)
    np.testing.assert_allclose(I, I0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(P, P0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(block_scores(P, S, Bs, nb), B0, rtol=0, atol=1e-12)
    qh = np.zeros((1, h + 1, L, d))
    kh = np.zeros((1, h + 1, L, d))
    qh[0, h], kh[0, h] = q, k
    scores, _ = rr_search(qh, kh, S, Bs, 0.9, h=h)         # head h samples with offset h mod S
    np.testing.assert_allclose(scores, B0, rtol=0, atol=1e-12)


def test_top_tau_hand_examples():
    s = np.array([0.1, 0.5, 0.2, 0.2])
    # descending order 1, 2, 3, 0 (the tie 2/3 goes to the lower index); cumulative 0.5, 0.7, 0.9, 1.0
    assert sorted(top_tau(s, 0.6).tolist()) == [1, 2]
    assert sorted(top_tau(s, 0.5).tolist()) == [1]
    assert sorted(top_tau(s, 0.85).tolist()) == [1, 2, 3]
    assert sorted(top_tau(s, 1.0).tolist()) == [0, 1, 2, 3]
    # relative to the row total
    assert sorted(top_tau(3.0 * s, 0.6).tolist()) == [1, 2]
    assert top_tau(np.zeros(3), 0.9).size == 0


def _rand_bits(shape, seed):
    from block_sparse_softmax_amd import inputs as gen
    return gen.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("L,S,Bs", [(512, 8, 64), (500, 8, 64), (384, 4, 128)])
def test_invariants_and_tau_one(L, S, Bs):
    q, k = _rand_bits((1, 2, L, 16), 1), _rand_bits((1, 2, L, 16), 2)
    nb = -(-L // Bs)
    for h in range(2):
        scores, B = rr_search(q, k, S, Bs, 1.0, h=h, protect_last=False)
        # each sampled stride's softmax sums to 1: a block row holds the number of its sampled strides
        ns = L // S
        per_block = np.bincount((np.arange(ns) * S) // Bs, minlength=nb)
        np.testing.assert_allclose(scores.sum(axis=1), per_block, rtol=1e-12)
        assert np.all(np.triu(scores, 1) == 0)
        # tau = 1 keeps every causal block that holds mass
        want = np.tril(np.ones((nb, nb), dtype=np.uint8)) * (scores > 0)
        assert np.array_equal(B, want.astype(np.uint8))


def test_protection_and_row_subset():
    L, S, Bs = 1024, 8, 128
    q, k = _rand_bits((1, 1, L, 32), 3), _rand_bits((1, 1, L, 32), 4)
    s_all, b_all = rr_search(q, k, S, Bs, 0.5)
    nb = L // Bs
    assert np.all(b_all[nb - 1] == 1)                       # Eq. 12: the last query block keeps every block
    s_no, b_no = rr_search(q, k, S, Bs, 0.5, protect_last=False)
    assert np.array_equal(b_all[: nb - 1], b_no[: nb - 1])
    assert b_no[nb - 1].sum() < nb                          # without protection tau = 0.5 drops some
    s_sub, b_sub = rr_search(q, k, S, Bs, 0.5, query_blocks=[2, 5, nb - 1])
    for m in (2, 5, nb - 1):
        np.testing.assert_array_equal(s_sub[m], s_all[m])
        np.testing.assert_array_equal(b_sub[m], b_all[m])


def test_planted_pattern_is_found():
    """Keys of one early block point along the queries' shared direction: every query block's
    importance concentrates there, and top-tau at 0.5 keeps it."""
    L, S, Bs, d = 1024, 8, 128, 32
    rng = np.random.default_rng(5)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((L, d)) + 3.0 * u
    k = rng.standard_normal((L, d))
    k[128:256] += 6.0 * u                                   # key block 1
    scores, B = rr_search(q[None, None], k[None, None], S, Bs, 0.5, protect_last=False)
    for m in range(1, L // Bs):
        assert B[m, 1] == 1 and B[m].sum() == 1, (m, B[m])
        assert scores[m, 1] > 0.5 * scores[m].sum()


@pytest.mark.parametrize("L,S,Bs,d,h", [(32, 4, 8, 3, 0), (37, 4, 16, 5, 2), (24, 8, 8, 2, 1)])
def test_literal_range_against_brute_force(L, S, Bs, d, h):
    """softmax_range="all" (Eq. 9 as printed: every key stride) against the same loops."""
    rng = np.random.default_rng(3 * L + S + d)
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    I0, P0, B0 = _brute_pipeline(q.tolist(), k.tolist(), S, Bs, h, all_strides=True)
    P = stride_softmax(stride_importance(q, k, S, h), "all")
    np.testing.assert_allclose(P, P0, rtol=0, atol=1e-12)
    qh = np.zeros((1, h + 1, L, d))
    kh = np.zeros((1, h + 1, L, d))
    qh[0, h], kh[0, h] = q, k
    scores, B = rr_search(qh, kh, S, Bs, 1.0, h=h, protect_last=False, softmax_range="all")
    np.testing.assert_allclose(scores, B0, rtol=0, atol=1e-12)
    # tau = 1 over whole rows: every block with mass, above the diagonal too
    assert np.array_equal(B, (B0 > 0).astype(np.uint8))


def test_readings_agree_on_the_last_stride_and_differ_before():
    """The last sampled stride sees every key stride under both readings, so its row of P is the
    same; earlier rows differ (the causal reading gives future strides no mass); both readings give
    each row a total of 1, so block rows hold the number of their sampled strides."""
    rng = np.random.default_rng(21)
    L, S, Bs, d = 256, 8, 64, 16
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    I = stride_importance(q, k, S, 0)
    Pc, Pa = stride_softmax(I), stride_softmax(I, "all")
    np.testing.assert_allclose(Pc[-1], Pa[-1], rtol=0, atol=1e-15)
    upper = np.triu_indices(Pc.shape[0], 1)
    assert np.all(Pc[upper] == 0) and np.all(Pa[upper] > 0)
    assert np.max(np.abs(Pc[:-1] - Pa[:-1])) > 1e-3
    np.testing.assert_allclose(Pa.sum(axis=1), 1.0, rtol=1e-13)
    nb = L // Bs
    for rng_name in ("causal", "all"):
        sc, _ = rr_search(q[None, None], k[None, None], S, Bs, 0.9, softmax_range=rng_name)
        np.testing.assert_allclose(sc.sum(axis=1), Bs // S, rtol=1e-12)
    with pytest.raises(ValueError):
        rr_search(q[None, None], k[None, None], S, Bs, 0.9, softmax_range="future")


def test_literal_range_selects_a_future_block():
    """Keys of the last block point along the queries' direction: as printed, Eq. 9 gives every
    earlier query block its mass there (a block above the diagonal, excluded by Eq. 5 for causal
    attention); the causal reading cannot."""
    L, S, Bs, d = 1024, 8, 128, 32
    rng = np.random.default_rng(6)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((L, d)) + 3.0 * u
    k = rng.standard_normal((L, d))
    k[896:1024] += 6.0 * u                                  # key block 7 (the last)
    _, Ba = rr_search(q[None, None], k[None, None], S, Bs, 0.5, protect_last=False, softmax_range="all")
    _, Bc = rr_search(q[None, None], k[None, None], S, Bs, 0.5, protect_last=False)
    for m in range(L // Bs - 1):
        assert Ba[m, 7] == 1 and Ba[m].sum() == 1, (m, Ba[m])
        assert Bc[m, 7] == 0 and np.all(np.triu(Bc, 1) == 0)
