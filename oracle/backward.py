"""Float64 attention backward — TEST INFRASTRUCTURE ONLY (see package doc).

The FlashAttention interview canvas says the forward keeps only the output and
one statistic per row, and the backward recomputes the local scores and
probabilities from them instead of storing the attention matrix (panel 1,
v1 card; panel 3, Q3).  What the backward computes is fixed by the forward: the
gradients of O = softmax(tau Q K^T) V with respect to Q, K and V, given the
gradient dO of a loss with respect to O.  This module writes that definition
out with the softmax Jacobian, per (batch, query head), in float64 and without
any tiling or recomputation trick:

    P   = softmax over the visible keys of each row (zero elsewhere)
    dV  = P^T dO
    dP  = dO V^T
    dS  = P * (dP - rowsum(P * dP))          (the softmax Jacobian applied to dP)
    dQ  = tau dS K
    dK  = tau dS^T Q

Grouped-query heads: a key/value head's gradient is the sum over the query
heads that read it.  A row with no visible key contributes nothing.  The loss
gradient reaches the forward only through O (no gradient through the LSE).
"""

from __future__ import annotations

import math

import numpy as np

from .attention import _f64, visible_keys


def attention_bwd_fp64(q, k, v, do, causal: bool = False, scale: float | None = None, heads=None):
    """(dQ [B,Hq,Sq,d], dK [B,Hkv,Sk,d], dV [B,Hkv,Sk,dv]) in float64.

    ``heads``: optional iterable of (b, h) query heads; only their
    contributions are computed (dQ of the other heads stays 0, and dK/dV hold
    the selected heads' part of the group sum) — for sampled checks."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    n_vis = np.array([visible_keys(i, Sq, Sk, causal) for i in range(Sq)])
    vis = np.arange(Sk)[None, :] < n_vis[:, None]  # [Sq, Sk]
    has = n_vis > 0
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    work = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in work:
        kvh = h // G
        kk, vv = k[b, kvh], v[b, kvh]
        s = np.where(vis, (q[b, h] @ kk.T) * tau, -np.inf)
        m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
        e = np.where(vis, np.exp(s - m[:, None]), 0.0)
        p = e / np.where(has, e.sum(axis=1), 1.0)[:, None]
        dv[b, kvh] += p.T @ do[b, h]
        dp = do[b, h] @ vv.T
        ds = p * (dp - (p * dp).sum(axis=1)[:, None])
        dq[b, h] = tau * (ds @ kk)
        dk[b, kvh] += tau * (ds.T @ q[b, h])
    return dq, dk, dv
