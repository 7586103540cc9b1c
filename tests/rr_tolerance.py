"""Error bound of a GPU block-score computation against the float64 oracle of RRAttention's search
(Eq. 8-10), derived from the precision the kernel states.

The kernel forms each stride sum of the keys in fp32 (S additions in key order) and carries it as a
pair of bf16 values hi = bf16(x), lo = bf16(x - hi); the importance GEMM multiplies bf16 queries
(exact inputs) by hi and lo on the matrix cores (bf16 products are exact in fp32) and accumulates
in fp32; the softmax and the block sums run in fp32.  With u = 2^-24 (fp32) and float64 values of
the oracle (ks = stride sums, Q = sampled queries, I = Eq. 8, P = Eq. 9):

* key aggregate:  |ks_kernel - ks| <= 2^-16 |ks| + S u sum_s |k_s|              (per component)
  (|x - hi| <= 2^-8 |x| and |x - hi - lo| <= 2^-8 |x - hi|; the S fp32 additions)
* importance:     |I_kernel - I| <= E_ij = [sum_c |q_c| delta_c + 2.1 D u sum_c |q_c| |ks_c|] / (S sqrt(d))
                                    + 4 u |I_ij|                              (2D fp32 additions, scaling)
* softmax:        with eps_i = max_j E_ij over the row's key strides, every probability moves by a
                  factor in [exp(-2 eps_i), exp(2 eps_i)], so
                  |dS_mn| <= T_mn = sum_{i in m, j in n} P_ij (exp(2 eps_i) - 1)
* fp32 sums:      the kernel sums a row's probabilities per lane over chunks of 32 key strides (16
                  terms of a chunk first, then one running addition per chunk) and combines lanes in
                  a tree, so the longest chain of fp32 additions behind a denominator or a block
                  score is about n_row / 32 + 40 (n_row = the row's key strides); with the
                  exponential's and the normalisation's own rounding the relative error is at most
                  (ceil(n_row / 32) + 64) u.
* flushed terms:  the single pass takes every probability against a fixed reference r_i above the
                  row's max (|q| times the largest key-aggregate norm, Cauchy-Schwarz); a row whose
                  sum against r_i is below 2^-40 is recomputed by the two-pass method, so r_i exceeds
                  the row's max by at most 40 + log2(n_row) <= 57 log2 units, and a term that flushes
                  (2^(I - r) below 2^-126) is a probability below 2^-69; a block sums R^2 <= 2^10 of
                  them: at most 2^-59 per block score, covered by 2^-58 R.

tol_mn = T_mn + (ceil(n_row / 32) + 64) u S_mn + 2^-58 R.
"""

from __future__ import annotations

import numpy as np

from oracle.attention import _as_f64
from oracle.rr_search import sample_positions

U32 = 2.0 ** -24


def score_tolerance(q, k, S: int, Bs: int, h: int, b: int = 0, query_blocks=None) -> np.ndarray:
    """tol [nb, nb] for head h (rows outside query_blocks are 0)."""
    qh = _as_f64(q[b, h])
    kh = _as_f64(k[b, h // (np.shape(q)[1] // np.shape(k)[1])])
    L, d = qh.shape
    ns, nb, R = L // S, -(-L // Bs), Bs // S
    ks = kh[: ns * S].reshape(ns, S, d).sum(axis=1)
    kabs = np.abs(kh[: ns * S]).reshape(ns, S, d).sum(axis=1)
    delta = 2.0 ** -16 * np.abs(ks) + S * U32 * kabs
    Q = qh[sample_positions(L, S, h)]
    tol = np.zeros((nb, nb))
    blocks = np.arange(nb) if query_blocks is None else np.asarray(query_blocks)
    scale = 1.0 / (S * np.sqrt(d))
    for m in blocks:
        rows = np.arange(m * R, min((m + 1) * R, ns))
        if rows.size == 0:
            continue
        Qr = Q[rows]
        I = (Qr @ ks.T) * scale
        E = (np.abs(Qr) @ delta.T + 2.1 * d * U32 * (np.abs(Qr) @ np.abs(ks).T)) * scale + 4 * U32 * np.abs(I)
        causal = np.arange(ns)[None, :] <= rows[:, None]
        z = np.where(causal, I, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        e = np.where(causal, np.exp(z), 0.0)
        P = e / e.sum(axis=1, keepdims=True)
        eps = np.where(causal, E, 0.0).max(axis=1)
        chain = -(-(rows + 1) // 32) + 64
        W = P * (np.expm1(2 * eps) + chain * U32)[:, None]
        kb = (np.arange(ns) * S) // Bs
        tol[m] = np.bincount(kb, weights=W.sum(axis=0), minlength=nb)[:nb] + 2.0 ** -58 * R
    return tol
