"""Structured-mask softmax attention, written out as its definition, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed
-------------------
* Scores: s_ij = q_i . k_j / sqrt(d)  ("Vision transformers and hybrid
  architectures", section 2, the score and softmax equations; "RRAttention",
  section 2.1, Eq. 1).
* The softmax of query i runs only over its allowed key set N(i), so each
  row's weights sum to 1 ("Semantic Head Specialization ...", the mask slide
  that defines N(i) for full / chunk / sliding window).  Disallowed pairs are
  excluded (weight exactly 0), not multiplied by a 0/1 mask inside the
  exponent: the block-sparse page says a zero entry of B skips the pair
  (section 2.1, text around Eq. 1).
* Mask families (0-based token and block indices):
    full    every key (optionally j <= i)
    chunk   floor(i/C) == floor(j/C)  (non-overlapping chunks; SHS slides,
            the "window interaction" factor)
    window  i - left_h <= j <= i + right, both ends inclusive; the SHS
            serialisation slide's example (anchor 15 with 8 per side covers
            7..23) fixes the inclusive reading.  A causal window of W keys
            ("Asymmetric Attention Heads", Table 2 candidate windows) is
            left = W-1, right = 0.
    block   B_h[floor(i/Bs), floor(j/Bs)] == 1 and j <= i  ("RRAttention",
            Eq. 2).
* Sink: a per-head logit s_aux added to the softmax denominator only, a key
  with no value; s_aux = -inf is plain softmax (SHS slides, the sink-bias
  slide, "Eq. 1").
* Prefix tokens: mask["prefix"] = P adds keys 0..P-1 to every query's set
  before the causal cut (the StreamingLLM sink tokens that the
  sliding-window-vs-linear-attention article, sections "forget or compress"
  and "comparison at equal memory", keeps beside a window: 572 + 4).
* Grouped-query attention: K and V may have fewer heads Hk (H a multiple of
  Hk); query head h uses K/V head h // (H / Hk), so each run of H/Hk
  consecutive query heads shares one (the same article: 32 query heads
  sharing 8 key-value heads).
* Output: o_i = sum_j a_ij v_j ("Vision transformers ...", section 2).
* Numerically stable form: subtract the row maximum before exponentiating
  (the same page's interactive softmax example).
A row with no allowed key gives o_i = 0 (the pages do not cover it).
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) exactly into float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _as_f64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return x.astype(np.float64)


def allowed_rows(mask: dict, h: int, rows: np.ndarray, L: int) -> np.ndarray:
    """Boolean [len(rows), L]: entry (r, j) is True iff key j is in N(rows[r]) for head h."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(L, dtype=np.int64)[None, :]
    kind = mask["kind"]
    if kind == "full":
        m = np.ones((i.shape[0], L), dtype=bool)
    elif kind == "chunk":
        c = int(mask["chunk"])
        m = (i // c) == (j // c)
    elif kind == "window":
        hl = mask.get("head_left")
        left = int(hl[h]) if hl is not None else int(mask.get("left", 0))
        right = int(mask.get("right", 0))
        m = (j >= i - left) & (j <= i + right)
    elif kind == "block":
        bs = int(mask["block"])
        bm = np.asarray(mask["block_mask"])
        bh = bm[h] if bm.shape[0] > 1 else bm[0]
        m = (bh[i // bs, j // bs] != 0) & (j <= i)
    else:
        raise ValueError(f"unknown mask kind {kind!r}")
    prefix = int(mask.get("prefix", 0) or 0)
    if prefix > 0:
        m = m | (j < prefix)
    if mask.get("causal", False):
        m = m & (j <= i)
    return m


def dense_mask(mask: dict, h: int, L: int) -> np.ndarray:
    """The explicit L x L mask of head h (use for L up to ~16K only)."""
    return allowed_rows(mask, h, np.arange(L), L)


def attention(q, k, v, mask: dict, sink=None, rows=None, scale=None, row_chunk: int = 256) -> dict:
    """Masked softmax attention in float64.

    q       : [B, H, L, D] arrays (bf16 bit patterns as uint16, or any float dtype).
    k, v    : [B, Hk, L, D] with H a multiple of Hk (grouped-query attention when Hk < H).
    mask    : mask dict (see module docstring).
    sink    : None or [H] per-head logits (on the scale of s_ij; -inf = no sink).
    rows    : None for every query row, or int [H, n] of query rows per head.
    scale   : softmax scale; default 1/sqrt(D).

    Returns dict with
      out      [B, H, n, D] float64 outputs of the evaluated rows,
      rowsum   [B, H, n] sum of the attention weights over keys,
      sink_mass[B, H, n] weight taken by the sink (0 without sink),
      pairs    [H] number of allowed (i, j) pairs over the evaluated rows,
      rows     [H, n] the evaluated rows.
    """
    B, H, L, D = np.shape(q)
    Hk = np.shape(k)[1]
    if H % Hk != 0 or np.shape(v)[1] != Hk:
        raise ValueError("K and V need the same number of heads, a divisor of Q's")
    group = H // Hk
    sigma = (1.0 / np.sqrt(D)) if scale is None else float(scale)
    if rows is None:
        rows = np.tile(np.arange(L, dtype=np.int64), (H, 1))
    rows = np.asarray(rows, dtype=np.int64)
    n = rows.shape[1]
    s_aux = None if sink is None else np.asarray(sink, dtype=np.float64)

    out = np.zeros((B, H, n, D))
    rowsum = np.zeros((B, H, n))
    sink_mass = np.zeros((B, H, n))
    pairs = np.zeros(H, dtype=np.int64)
    for h in range(H):
        sa = -np.inf if s_aux is None else s_aux[h]
        for b in range(B):
            kf, vf = _as_f64(k[b, h // group]), _as_f64(v[b, h // group])
            for r0 in range(0, n, row_chunk):
                rr = rows[h, r0:r0 + row_chunk]
                allowed = allowed_rows(mask, h, rr, L)
                if b == 0:
                    pairs[h] += int(allowed.sum())
                s = sigma * (_as_f64(q[b, h, rr]) @ kf.T)        # [r, L]
                s = np.where(allowed, s, -np.inf)
                m = np.maximum(s.max(axis=1), sa)                  # row max incl. the sink logit
                empty = ~np.isfinite(m)                            # no allowed key and no sink
                m = np.where(empty, 0.0, m)
                e = np.exp(s - m[:, None])                         # exp(-inf) = 0 on masked pairs
                z = e.sum(axis=1) + np.exp(sa - m)
                zsafe = np.where(z > 0, z, 1.0)
                p = e / zsafe[:, None]
                out[b, h, r0:r0 + len(rr)] = p @ vf
                rowsum[b, h, r0:r0 + len(rr)] = p.sum(axis=1)
                sink_mass[b, h, r0:r0 + len(rr)] = np.where(z > 0, np.exp(sa - m) / zsafe, 0.0)
    return dict(out=out, rowsum=rowsum, sink_mass=sink_mass, pairs=pairs, rows=rows)
