"""Pins of the decode oracle (oracle/decode.py), CPU only.

The decode query of a sequence with n cached tokens is token n - 1, so its
output must equal row n - 1 of the prefill attention over the first n tokens
with the causal window (+ prefix) mask; a pure-Python brute force with the
window written as plain integer bounds; closed forms (a one-key window gives
the newest value scaled by 1 - sink mass, V = 1 gives 1 - sink mass); cache
rows outside the key set may hold NaN without changing anything.
"""

import math

import numpy as np
import pytest

from block_sparse_softmax_amd import inputs as gen
from oracle.attention import attention, bf16_to_f64
from oracle.decode import decode_attention, decode_mask


def _case(B=3, H=4, Hk=2, L=40, D=8, seed=0, cfg=90):
    rng = np.random.default_rng([seed, cfg])
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, H, D), dtype=np.float32))
    k = gen.f32_to_bf16_bits(rng.standard_normal((B, Hk, L, D), dtype=np.float32))
    v = gen.f32_to_bf16_bits(rng.standard_normal((B, Hk, L, D), dtype=np.float32))
    return q, k, v


@pytest.mark.parametrize("window,prefix,with_sink", [(0, 0, False), (1, 0, False), (7, 0, True), (7, 3, False),
                                                      (16, 2, True), (100, 0, True)])
def test_equals_last_prefill_row(window, prefix, with_sink):
    q, k, v = _case()
    lens = np.array([1, 23, 40], np.int32)
    sink = np.array([0.3, -1.0, 2.0, -np.inf]) if with_sink else None
    got = decode_attention(q, k, v, lens, window, prefix, sink=sink)
    mask = decode_mask(window, prefix)
    for b, n in enumerate(lens):
        # prefill over the first n tokens, the query placed as token n - 1
        qp = np.zeros((1, 4, n, 8), np.uint16)
        qp[0, :, n - 1] = q[b]
        ref = attention(qp, k[b:b + 1, :, :n], v[b:b + 1, :, :n], mask, sink=sink,
                        rows=np.full((4, 1), n - 1))
        np.testing.assert_allclose(got["out"][b], ref["out"][0, :, 0], rtol=0, atol=1e-12)
        assert got["pairs"][b] == ref["pairs"][0]


def test_brute_force():
    B, H, Hk, L, D = 2, 2, 1, 12, 3
    q, k, v = _case(B, H, Hk, L, D, cfg=91)
    lens = [12, 5]
    sink = [0.5, -0.25]
    for window, prefix in [(0, 0), (3, 0), (4, 2), (20, 1)]:
        got = decode_attention(q, k, v, lens, window, prefix, sink=sink)["out"]
        for b in range(B):
            n = lens[b]
            t = n - 1
            for h in range(H):
                ks = [j for j in range(n) if (window <= 0 or t - window + 1 <= j <= t) or j < prefix]
                qv = [float(x) for x in bf16_to_f64(q[b, h])]
                logits = []
                for j in ks:
                    kj = bf16_to_f64(k[b, 0, j])
                    logits.append(sum(qv[d] * kj[d] for d in range(D)) / math.sqrt(D))
                mx = max(logits + [sink[h]])
                den = sum(math.exp(x - mx) for x in logits) + math.exp(sink[h] - mx)
                for d in range(D):
                    num = sum(math.exp(x - mx) * float(bf16_to_f64(v[b, 0, j])[d]) for x, j in zip(logits, ks))
                    assert abs(got[b, h, d] - num / den) < 1e-12


def test_one_key_window_and_unit_values():
    q, k, v = _case(cfg=92)
    lens = np.array([9, 30, 40], np.int32)
    sink = np.array([0.0, 1.0, -2.0, 0.5])
    r = decode_attention(q, k, v, lens, 1, 0, sink=sink)
    for b, n in enumerate(lens):
        for h in range(4):
            expect = (1 - r["sink_mass"][b, h]) * bf16_to_f64(v[b, h // 2, n - 1])
            np.testing.assert_allclose(r["out"][b, h], expect, rtol=0, atol=1e-12)
    ones = np.full_like(v, 0x3F80)      # bf16 1.0
    r1 = decode_attention(q, k, ones, lens, 16, 3, sink=sink)
    np.testing.assert_allclose(r1["out"], np.repeat((1 - r1["sink_mass"])[:, :, None], 8, axis=2), atol=1e-12)


def test_rows_outside_the_key_set_are_never_read():
    q, k, v = _case(cfg=93)
    lens = np.array([40, 33, 17], np.int32)
    ref = decode_attention(q, k, v, lens, 10, 2)
    kn, vn = k.copy(), v.copy()
    for b, n in enumerate(lens):
        keep = np.zeros(40, bool)
        keep[:2] = True
        keep[n - 10:n] = True
        kn[b, :, ~keep] = 0x7FC0        # bf16 NaN
        vn[b, :, ~keep] = 0x7FC0
    got = decode_attention(q, kn, vn, lens, 10, 2)
    np.testing.assert_array_equal(got["out"], ref["out"])
    assert np.all(np.isfinite(got["out"]))
    assert list(got["pairs"]) == [12, 12, 12]


def test_empty_sequence_and_full_window():
    q, k, v = _case(cfg=94)
    lens = np.array([0, 40, 40], np.int32)
    r = decode_attention(q, k, v, lens, 0, 0, sink=np.zeros(4))
    assert np.all(r["out"][0] == 0) and r["pairs"][0] == 0
    wide = decode_attention(q, k, v, lens, 1000, 0, sink=np.zeros(4))
    np.testing.assert_array_equal(wide["out"], r["out"])
    assert list(r["pairs"]) == [0, 40, 40]


def test_cache_row_generator_fills_head_and_tail():
    pos, kk, vv = gen.decode_cache_rows(0, 10, 3, 1000, 2, 8, 4, 576)
    assert list(pos[:4]) == [0, 1, 2, 3] and pos[4] == 1000 - 576 and pos[-1] == 999 and len(pos) == 580
    assert kk.shape == (2, 580, 8) and vv.shape == (2, 580, 8)
    pos2, _, _ = gen.decode_cache_rows(0, 10, 3, 100, 2, 8, 4, 576)
    assert list(pos2) == list(range(100))
