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
