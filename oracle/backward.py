"""Gradients of structured-mask softmax attention, written out in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The forward is the definition in attention.py (the pages' masked softmax
attention with an optional per-head sink logit in the denominator).  For a
loss with upstream gradient dO (the pages train models with these masks: the
SHS slides' ViT variants, the per-head windows of "Asymmetric Attention
Heads"), the chain rule through o_i = sum_j p_ij v_j and the row softmax
gives, per (batch, head), with s_ij = sigma q_i . k_j on allowed pairs:

  D_i     = sum_d dO_id O_id          (= sum_j p_ij (dO_i . v_j))
  dV_j    = sum_i p_ij dO_i
  dP_ij   = dO_i . v_j
  dS_ij   = p_ij (dP_ij - D_i)        (zero on disallowed pairs)
  dQ_i    = sigma sum_j dS_ij k_j
  dK_j    = sigma sum_i dS_ij q_i
  ds_aux  = - sum_i pi_i D_i          (the sink is a key with logit s_aux and
                                       no value: its "dP" is 0; pi_i is the
                                       mass it takes)

With grouped-query heads the K/V gradients of a shared head are summed over
its query heads.  The log-sum-exp of row i (natural log, sink included) is
returned as well: p_ij = exp(s_ij - lse_i).
"""

from __future__ import annotations

import numpy as np

from .attention import _as_f64, allowed_rows


def attention_backward(q, k, v, dout, mask: dict, sink=None, scale=None):
    """Returns dict(dq [B,H,L,D], dk [B,Hk,L,D], dv [B,Hk,L,D], dsink [H] or None, lse [B,H,L],
    out [B,H,L,D]), all float64."""
    B, H, L, D = np.shape(q)
    Hk = np.shape(k)[1]
    g = H // Hk
    sigma = (1.0 / np.sqrt(D)) if scale is None else float(scale)
    s_aux = None if sink is None else np.asarray(sink, dtype=np.float64)
    dq = np.zeros((B, H, L, D))
    dk = np.zeros((B, Hk, L, D))
    dv = np.zeros((B, Hk, L, D))
    lse = np.full((B, H, L), -np.inf)
    out = np.zeros((B, H, L, D))
    dsink = None if s_aux is None else np.zeros(H)
    rows = np.arange(L)
    for h in range(H):
        allowed = allowed_rows(mask, h, rows, L)
        sa = -np.inf if s_aux is None else s_aux[h]
        for b in range(B):
            qf, kf, vf = _as_f64(q[b, h]), _as_f64(k[b, h // g]), _as_f64(v[b, h // g])
            do = _as_f64(dout[b, h])
            s = np.where(allowed, sigma * (qf @ kf.T), -np.inf)
            m = np.maximum(s.max(axis=1), sa)
            empty = ~np.isfinite(m)
            m = np.where(empty, 0.0, m)
            e = np.exp(s - m[:, None])
            z = e.sum(axis=1) + np.exp(sa - m)
            zs = np.where(z > 0, z, 1.0)
            p = e / zs[:, None]
            pi = np.where(z > 0, np.exp(sa - m) / zs, 0.0)
            o = p @ vf
            Di = (do * o).sum(axis=1)
            dP = do @ vf.T
            dS = p * (dP - Di[:, None])
            dq[b, h] = sigma * (dS @ kf)
            dk[b, h // g] += sigma * (dS.T @ qf)
            dv[b, h // g] += p.T @ do
            lse[b, h] = np.where(z > 0, m + np.log(zs), -np.inf)
            out[b, h] = o
            if dsink is not None:
                dsink[h] += -(pi * Di).sum()
    return dict(dq=dq, dk=dk, dv=dv, dsink=dsink, lse=lse, out=out)


def _row_stats(qf, kf, vf, do, allowed, sa, sigma):
    """For query rows with their allowed keys: probabilities p [r, L], row sink mass, D_i, lse."""
    s = np.where(allowed, sigma * (qf @ kf.T), -np.inf)
    m = np.maximum(s.max(axis=1), sa)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m[:, None])
    z = e.sum(axis=1) + np.exp(sa - m)
    zs = np.where(z > 0, z, 1.0)
    p = e / zs[:, None]
    Di = (do * (p @ vf)).sum(axis=1)
    return p, Di


def dq_rows(q, k, v, dout, mask: dict, rows, sink=None, scale=None):
    """dQ of the query rows rows[h] (int [H, n]) only, by the same formulas as attention_backward
    restricted to those rows (each row needs only its own scores): returns [B, H, n, D]."""
    B, H, L, D = np.shape(q)
    g = H // np.shape(k)[1]
    sigma = (1.0 / np.sqrt(D)) if scale is None else float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, H, rows.shape[1], D))
    for h in range(H):
        sa = -np.inf if sink is None else float(sink[h])
        allowed = allowed_rows(mask, h, rows[h], L)
        for b in range(B):
            kf, vf = _as_f64(k[b, h // g]), _as_f64(v[b, h // g])
            qf, do = _as_f64(q[b, h, rows[h]]), _as_f64(dout[b, h, rows[h]])
            p, Di = _row_stats(qf, kf, vf, do, allowed, sa, sigma)
            dS = p * (do @ vf.T - Di[:, None])
            out[b, h] = sigma * (dS @ kf)
    return out


def dkdv_cols(q, k, v, dout, mask: dict, cols, sink=None, scale=None, row_chunk: int = 512, first_row: int = 0):
    """dK and dV of the keys cols[hk] (int [Hk, n]) only: every query row that may see one of those
    keys, of every query head sharing K/V head hk, is evaluated in full (its softmax needs all of its
    keys); returns (dk, dv), each [B, Hk, n, D].  first_row: rows before it are skipped (the caller
    guarantees that they see none of the keys, e.g. a causal mask and first_row <= min(cols))."""
    B, H, L, D = np.shape(q)
    Hk = np.shape(k)[1]
    g = H // Hk
    sigma = (1.0 / np.sqrt(D)) if scale is None else float(scale)
    cols = np.asarray(cols, dtype=np.int64)
    dk = np.zeros((B, Hk, cols.shape[1], D))
    dv = np.zeros((B, Hk, cols.shape[1], D))
    for hk in range(Hk):
        c = cols[hk]
        for h in range(hk * g, (hk + 1) * g):
            sa = -np.inf if sink is None else float(sink[h])
            for r0 in range(first_row, L, row_chunk):
                rr = np.arange(r0, min(L, r0 + row_chunk))
                allowed = allowed_rows(mask, h, rr, L)
                sees = allowed[:, c].any(axis=1)
                if not sees.any():
                    continue
                rr, allowed = rr[sees], allowed[sees]
                for b in range(B):
                    kf, vf = _as_f64(k[b, hk]), _as_f64(v[b, hk])
                    qf, do = _as_f64(q[b, h, rr]), _as_f64(dout[b, h, rr])
                    p, Di = _row_stats(qf, kf, vf, do, allowed, sa, sigma)
                    pc = p[:, c]
                    dSc = pc * (do @ vf[c].T - Di[:, None])
                    dv[b, hk] += pc.T @ do
                    dk[b, hk] += sigma * (dSc.T @ qf)
    return dk, dv


def lse_rows(q, k, mask: dict, rows, sink=None, scale=None):
    """The log-sum-exp (natural log, sink included; -inf for a row with neither keys nor sink) of the
    query rows rows[h] (int [H, n]) only: returns [B, H, n]."""
    B, H, L, D = np.shape(q)
    g = H // np.shape(k)[1]
    sigma = (1.0 / np.sqrt(D)) if scale is None else float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, H, rows.shape[1]))
    for h in range(H):
        sa = -np.inf if sink is None else float(sink[h])
        allowed = allowed_rows(mask, h, rows[h], L)
        for b in range(B):
            s = np.where(allowed, sigma * (_as_f64(q[b, h, rows[h]]) @ _as_f64(k[b, h // g]).T), -np.inf)
            m = np.maximum(s.max(axis=1), sa)
            fin = np.isfinite(m)
            m0 = np.where(fin, m, 0.0)
            z = np.exp(s - m0[:, None]).sum(axis=1) + np.exp(sa - m0)
            with np.errstate(divide="ignore"):
                out[b, h] = np.where(fin, m0 + np.log(z), -np.inf)
    return out
