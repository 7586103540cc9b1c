"""One-query (decode) attention over a key/value cache, written out as its definition, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Generation appends one token at a time: sequence b holds n_b cached tokens and
its new query is token t = n_b - 1.  The sliding-window vs linear-attention
article decodes with a causal window of the last W tokens, with a learned
per-head sink logit or with the first P tokens kept as StreamingLLM sink
tokens ("comparison at equal memory": 576, or 572 + 4), on grouped-query
heads.  The query's allowed keys are therefore row t of the prefill masks of
attention.py restricted to the n_b cached tokens:
    W >= 1 : the causal window of W keys (left reach W - 1) plus the prefix,
    W <= 0 : every cached key (causal full attention).
Scores, the sink term and the empty-row convention are those of
attention.attention; only the allowed keys of each row are gathered, so cache
rows outside that set (which may hold anything) are never read.
"""

from __future__ import annotations

import numpy as np

from .attention import _as_f64, allowed_rows


def decode_mask(window: int, prefix: int = 0) -> dict:
    """The prefill mask whose row t is the decode query's key set."""
    if window <= 0:
        return dict(kind="full", causal=True, prefix=int(prefix))
    return dict(kind="window", left=int(window) - 1, right=0, causal=True, prefix=int(prefix))


def decode_attention(q, k, v, seq_lens, window: int, prefix: int = 0, sink=None, scale=None, batches=None) -> dict:
    """q: [B, H, D]; k, v: indexable by sequence b, each [Hk, >= n_b, D] (H a multiple of Hk;
    bf16 bits as uint16 or floats); seq_lens: [B] cached tokens n_b.
    Returns dict(out [B, H, D] float64 (rows of sequences not evaluated or with n_b <= 0 are 0),
    pairs [B] allowed keys per sequence, sink_mass [B, H])."""
    q = np.asarray(q)
    B, H, D = q.shape
    sigma = (1.0 / np.sqrt(D)) if scale is None else float(scale)
    s_aux = None if sink is None else np.asarray(sink, dtype=np.float64)
    mask = decode_mask(window, prefix)
    out = np.zeros((B, H, D))
    sink_mass = np.zeros((B, H))
    pairs = np.zeros(B, dtype=np.int64)
    for b in (range(B) if batches is None else batches):
        n = int(seq_lens[b])
        if n <= 0:
            continue
        idx = np.nonzero(allowed_rows(mask, 0, np.array([n - 1]), n)[0])[0]
        pairs[b] = len(idx)
        kb, vb = k[b], v[b]
        g = H // np.shape(kb)[0]
        for h in range(H):
            sa = -np.inf if s_aux is None else s_aux[h]
            kf = _as_f64(kb[h // g][idx])
            vf = _as_f64(vb[h // g][idx])
            s = sigma * (kf @ _as_f64(q[b, h]))
            m = max(s.max(), sa)
            e = np.exp(s - m)
            z = e.sum() + np.exp(sa - m)
            out[b, h] = (e / z) @ vf
            sink_mass[b, h] = np.exp(sa - m) / z
    return dict(out=out, pairs=pairs, sink_mass=sink_mass)
