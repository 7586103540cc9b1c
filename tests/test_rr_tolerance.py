"""CPU check of the block-score bound in tests/rr_tolerance.py: scores computed in float64 from key
stride sums perturbed exactly as the stated precision allows (fp32 sums in key order, then the
bf16 hi + lo pair) stay within the bound of the plain float64 oracle, and the bound is tight enough
to decide the top-tau selection of most rows."""

import numpy as np
import pytest

from block_sparse_softmax_amd import inputs as gen
from oracle.attention import _as_f64
from oracle.rr_search import block_scores, rr_search, sample_positions

from rr_tolerance import score_tolerance


def _bf16_round(x32):
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _perturbed_scores(q, k, S, Bs, h):
    qh, kh = _as_f64(q[0, h]), _as_f64(k[0, h])
    L, d = qh.shape
    ns, nb = L // S, -(-L // Bs)
    acc = np.zeros((ns, d), np.float32)
    blocks = kh[: ns * S].reshape(ns, S, d).astype(np.float32)
    for s in range(S):
        acc = acc + blocks[:, s]
    hi = _bf16_round(acc)
    lo = _bf16_round(acc - hi)
    ks = hi.astype(np.float64) + lo.astype(np.float64)
    I = (qh[sample_positions(L, S, h)] @ ks.T) / (S * np.sqrt(d))
    causal = np.tril(np.ones((ns, ns), bool))
    z = np.where(causal, I, -np.inf)
    z -= z.max(axis=1, keepdims=True)
    P = np.where(causal, np.exp(z), 0.0)
    P /= P.sum(axis=1, keepdims=True)
    return block_scores(P, S, Bs, nb)


@pytest.mark.parametrize("L,D,S,Bs,kind", [(1024, 128, 8, 128, "random"), (1030, 80, 4, 128, "random"),
                                           (2048, 64, 16, 128, "planted")])
def test_bound_covers_the_stated_rounding(L, D, S, Bs, kind):
    rng = np.random.default_rng(L + D)
    if kind == "random":
        q, k = (gen.f32_to_bf16_bits(rng.standard_normal((1, 1, L, D), dtype=np.float32)) for _ in range(2))
    else:
        u = rng.standard_normal(D)
        u /= np.linalg.norm(u)
        qf = rng.standard_normal((1, 1, L, D)) + 3.0 * u
        kf = rng.standard_normal((1, 1, L, D))
        kf[0, 0, 256:384] += 6.0 * u
        q, k = (gen.f32_to_bf16_bits(x.astype(np.float32)) for x in (qf, kf))
    s_ref, _ = rr_search(q, k, S, Bs, 0.9)
    tol = score_tolerance(q, k, S, Bs, 0)
    s_pert = _perturbed_scores(q, k, S, Bs, 0)
    err = np.abs(s_pert - s_ref)
    assert np.all(err <= tol), float((err - tol).max())
    # tight: about 1e-4 of a score, where bf16-rounded sums alone would need about 2e-2
    nz = s_ref > 1e-3
    assert np.median(tol[nz] / s_ref[nz]) < 5e-4
