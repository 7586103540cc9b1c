"""RRAttention's block-pattern search, step by step in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "RRAttention" (the block-sparse page), section 3, in its order and
notation, for one (batch, head) at a time:

* Eq. 6: head round-robin query sampling.  In stride i (tokens [iS, (i+1)S))
  head h samples the query at P(i, h) = iS + (S - 1 - (h mod S)).
* Eq. 7: the sampled queries are those P(i, h) for every full stride,
  i = 0 .. floor(L/S) - 1 (the printed upper bound floor(L/S) would address a
  stride past the sequence when S divides L; the range of Eq. 9's softmax
  fixes the reading).
* Eq. 8: stride-level importance
      I_ij = (1 / (S sqrt(d))) q_P(i,h) . sum_{k = jS}^{(j+1)S - 1} k_k .
* Eq. 9: softmax of each row of I over key strides j'.  Reading: the softmax
  runs over the causal key strides j' <= i only.  The page's attention is
  causal (Eq. 2: j <= i; Eq. 5: B_mn = 0 for n > m), so importance estimated
  for future strides could never be used; the printed range (all j') is read
  as the causal range of the autoregressive setting it serves.
* Eq. 10: block scores S_mn = sum over the query strides i of block m and the
  key strides j of block n of P_ij, where stride i belongs to block
  floor(iS / Bs) (Bs a multiple of S).
* Eq. 11: top-tau selection per query block m: sort S_m,n (n <= m) in
  descending order (ties: lower n first) and keep the shortest prefix whose
  sum reaches tau.  Reading: tau is a fraction of the row's total mass
  sum_n S_mn (each P row sums to 1, so S_m,* sums to the number of sampled
  strides in block m; a threshold such as 0.9 only makes sense relative to
  it).  A row with no sampled stride selects nothing.
* Eq. 12: B = B_dynamic OR B_static, where B_static keeps every (causal)
  block of the last query block.

Returns the block scores S (float64) and the block matrix B (uint8), both
[Nb, Nb] with Nb = ceil(L / Bs).

softmax_range="all" follows Eq. 9 as printed instead: each row's softmax runs
over every key stride j' = 0 .. floor(L/S) - 1, the block scores of Eq. 10 then
fill whole rows (key blocks above the diagonal too) and Eq. 11 ranks all of a
row's blocks.  Kept as an option so the two readings can be compared; the
block matrix it yields can select blocks above the diagonal, which Eq. 5 rules
out for the causal attention the search feeds.
"""

from __future__ import annotations

import numpy as np

from .attention import _as_f64


def sample_positions(L: int, S: int, h: int) -> np.ndarray:
    """Eq. 6-7: the sampled query position of every full stride for head h."""
    i = np.arange(L // S, dtype=np.int64)
    return i * S + (S - 1 - (h % S))


def stride_importance(q: np.ndarray, k: np.ndarray, S: int, h: int) -> np.ndarray:
    """Eq. 8 for one head: q, k are [L, d] float64; returns I [Ns, Ns] (no mask applied)."""
    L, d = q.shape
    ns = L // S
    qs = q[sample_positions(L, S, h)]                       # sampled queries
    ks = k[: ns * S].reshape(ns, S, d).sum(axis=1)          # keys summed over each stride
    return (qs @ ks.T) / (S * np.sqrt(d))


def stride_softmax(I: np.ndarray, softmax_range: str = "causal") -> np.ndarray:
    """Eq. 9 over the causal key strides j <= i (max-subtracted); softmax_range="all": over every j'."""
    ns = I.shape[0]
    causal = _range_mask(ns, ns, np.arange(ns), softmax_range)
    z = np.where(causal, I, -np.inf)
    z = z - z.max(axis=1, keepdims=True)
    e = np.where(causal, np.exp(z), 0.0)
    return e / e.sum(axis=1, keepdims=True)


def _range_mask(ns_q: int, ns_k: int, rows, softmax_range: str) -> np.ndarray:
    """Key strides each row's softmax runs over: j <= i ("causal", the adopted reading) or all."""
    if softmax_range == "causal":
        return np.arange(ns_k)[None, :] <= np.asarray(rows)[:, None]
    if softmax_range == "all":
        return np.ones((len(rows), ns_k), dtype=bool)
    raise ValueError(softmax_range)


def block_scores(P: np.ndarray, S: int, Bs: int, nb: int, rows=None) -> np.ndarray:
    """Eq. 10: sum P over the strides of each (query block, key block) pair.

    rows: the query strides P holds (default: all, 0 .. Ns-1)."""
    ns_q, ns_k = P.shape
    rows = np.arange(ns_q) if rows is None else np.asarray(rows)
    out = np.zeros((nb, nb))
    qb = (rows * S) // Bs
    kb = (np.arange(ns_k) * S) // Bs
    for r in range(ns_q):
        np.add.at(out[qb[r]], kb, P[r])
    return out


def top_tau(scores_row: np.ndarray, tau: float) -> np.ndarray:
    """Eq. 11 for one query block: indices of the shortest prefix of the descending order (ties to
    the lower index) whose sum reaches tau times the row's total."""
    total = scores_row.sum()
    if total <= 0.0:
        return np.zeros(0, dtype=np.int64)
    order = np.argsort(-scores_row, kind="stable")
    csum = np.cumsum(scores_row[order])
    k = int(np.searchsorted(csum, tau * total, side="left"))   # first prefix reaching the threshold
    return order[: min(k + 1, len(order))]


def stride_key_sums(kh: np.ndarray, S: int) -> np.ndarray:
    """sum_{k = jS}^{(j+1)S - 1} k_k for every full stride j (Eq. 8's key aggregate)."""
    L, d = kh.shape
    ns = L // S
    return kh[: ns * S].reshape(ns, S, d).sum(axis=1)


def rr_search(q, k, S: int, Bs: int, tau: float, protect_last: bool = True, b: int = 0, h: int = 0,
              query_blocks=None, softmax_range: str = "causal"):
    """Block scores and block matrix for (batch b, head h) of bf16 bit arrays (or floats) q, k of
    shape [B, H, L, d].

    query_blocks: evaluate only these query blocks (the rows of S and B for other blocks are left
    zero), for long sequences.
    softmax_range: "causal" (Eq. 9 over j' <= i, the adopted reading) or "all" (Eq. 9 as printed,
    with Eq. 10-11 over the whole row)."""
    if Bs % S != 0:
        raise ValueError("the block size must be a multiple of the stride")
    qh = _as_f64(q[b, h])
    kh = _as_f64(k[b, h // (np.shape(q)[1] // np.shape(k)[1])])   # grouped-query: K head of query head h
    L, d = qh.shape
    nb = -(-L // Bs)
    ns = L // S
    R = Bs // S
    blocks = np.arange(nb) if query_blocks is None else np.asarray(query_blocks)
    scores = np.zeros((nb, nb))
    bmat = np.zeros((nb, nb), dtype=np.uint8)
    pos = sample_positions(L, S, h)
    ks = stride_key_sums(kh, S)
    causal_rows = softmax_range == "causal"
    _range_mask(1, 1, [0], softmax_range)                                      # validates the option
    for m in blocks:
        rows = np.arange(m * R, min((m + 1) * R, ns))
        if rows.size:
            I = (qh[pos[rows]] @ ks.T) / (S * np.sqrt(d))                      # Eq. 8
            causal = _range_mask(len(rows), ns, rows, softmax_range)
            z = np.where(causal, I, -np.inf)
            z = z - z.max(axis=1, keepdims=True)
            e = np.where(causal, np.exp(z), 0.0)
            P = e / e.sum(axis=1, keepdims=True)                                # Eq. 9
            scores[m] = block_scores(P, S, Bs, nb, rows=rows)[m]                # Eq. 10
        width = m + 1 if causal_rows else nb
        sel = top_tau(scores[m, :width], tau)                                   # Eq. 11
        bmat[m, sel] = 1
    if protect_last and (nb - 1) in set(blocks.tolist()):
        bmat[nb - 1, :nb] = 1                                                   # Eq. 12
    return scores, bmat
