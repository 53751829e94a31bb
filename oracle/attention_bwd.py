"""Plain float64 oracle for the reverse-mode derivative of the JVP attention forward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP library and imports nothing from it.

What is computed, and where it comes from
-----------------------------------------
The "JVP Flash Attention" README (section "Description") says the kernel
supports Hessian-vector products as well as JVPs. An HVP of a loss through
attention is taken reverse-over-forward: the forward-mode pass returns the
pair (O, dO) from (Q, K, V) and tangents (dQ, dK, dV), and the reverse pass
pulls cotangents (gO, gdO) of that pair back to all six inputs. This module
is that reverse pass, for the map

    (Q, K, V, dQ, dK, dV)  ->  (O, dO)

of ``attention.oracle_fwd_head``, given cotangents gO and gdO. It runs the
forward's own steps backwards, one at a time, with the chain rule (no
algebraic shortcuts, no blocking):

    S  = scale Q K^T + M          P = softmax_j(S)          O  = P V
    dS = scale (dQ K^T + Q dK^T)  t = rowsum(P * dS)        dP = P * (dS - t)
    dO = dP V + P dV

The additive mask M is a constant (no gradient). Rows whose every score is
-inf have P = 0 and contribute nothing. With grouped key/value heads several
query heads read one K/V head, so that head's cotangents are the sum of what
each of its query heads pulls back to it (the chain rule for a shared input).
"""
from __future__ import annotations

import math

import numpy as np

from .attention import MASK_NONE, _f64, _head_bias, kv_head


def oracle_bwd_head(q, k, v, tq, tk, tv, go, gto, bias, scale, tbias=None):
    """One head. Returns the cotangents (gq, gk, gv, gtq, gtk, gtv) in float64.
    tbias: tangent of an additive mask (a constant of the map, like the mask), or None."""
    # forward, keeping the intermediates
    S = scale * (q @ k.T) + bias
    dS = scale * (tq @ k.T + q @ tk.T)
    if tbias is not None:
        dS = dS + tbias
    live = ~np.all(np.isneginf(S), axis=1)
    P = np.zeros_like(S)
    if np.any(live):
        Sl = S[live]
        e = np.exp(Sl - np.max(Sl, axis=1, keepdims=True))
        P[live] = e / np.sum(e, axis=1, keepdims=True)
    t = np.sum(P * dS, axis=1, keepdims=True)
    dP = P * (dS - t)
    # reverse of dO = dP V + P dV
    g_dP = gto @ v.T
    g_v = dP.T @ gto
    g_P = gto @ tv.T
    g_tv = P.T @ gto
    # reverse of O = P V
    g_P = g_P + go @ v.T
    g_v = g_v + P.T @ go
    # reverse of dP = P * (dS - t)
    g_P = g_P + g_dP * (dS - t)
    g_dS = g_dP * P
    g_t = -np.sum(g_dP * P, axis=1, keepdims=True)
    # reverse of t = rowsum(P * dS)
    g_P = g_P + g_t * dS
    g_dS = g_dS + g_t * P
    # reverse of dS = scale (dQ K^T + Q dK^T)
    g_tq = scale * (g_dS @ k)
    g_k = scale * (g_dS.T @ tq)
    g_q = scale * (g_dS @ tk)
    g_tk = scale * (g_dS.T @ q)
    # reverse of P = softmax(S) (rows of P sum to one where live, are zero elsewhere)
    g_S = P * (g_P - np.sum(g_P * P, axis=1, keepdims=True))
    # reverse of S = scale Q K^T + M
    g_q = g_q + scale * (g_S @ k)
    g_k = g_k + scale * (g_S.T @ q)
    return g_q, g_k, g_v, g_tq, g_tk, g_tv


def oracle_bwd(q, k, v, tq, tk, tv, go, gto, mask=None, mask_kind=MASK_NONE, causal=False, scale=None,
               tmask=None):
    """Cotangents of (Q, K, V, dQ, dK, dV) for cotangents (go, gto) of (O, dO).

    Shapes as in ``oracle_fwd``: q, tq, go, gto [B,H,Nq,d]; k, v, tk, tv
    [B,Hkv,Nk,d] (Hkv divides H); mask [Bm,Hm,Nq,Nk]. A tangent given as None
    is zero. tmask: tangent of an additive mask, laid out as ``mask``: the
    forward it differentiates then carries dS + dM (no cotangent of the mask
    or its tangent is returned).
    Returns (gq, gk, gv, gtq, gtk, gtv) float64, shaped like the inputs.
    """
    q, k, v, go, gto = _f64(q), _f64(k), _f64(v), _f64(go), _f64(gto)
    tq = np.zeros_like(q) if tq is None else _f64(tq)
    tk = np.zeros_like(k) if tk is None else _f64(tk)
    tv = np.zeros_like(v) if tv is None else _f64(tv)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if mask is not None:
        mask = np.asarray(mask)
    if (mask is None) != (mask_kind == MASK_NONE):
        raise ValueError("mask must be given exactly when mask_kind is not 'none'")
    gq, gtq = np.empty_like(q), np.empty_like(q)
    gk, gv, gtk, gtv = np.zeros_like(k), np.zeros_like(v), np.zeros_like(k), np.zeros_like(v)
    q_pos = np.arange(Nq)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            bias = _head_bias(mask, mask_kind, b, h, Nq, Nk, causal, q_pos)
            tbias = None if tmask is None else _head_bias(np.asarray(tmask), "additive", b, h, Nq, Nk, False, q_pos)
            r = oracle_bwd_head(q[b, h], k[b, g], v[b, g], tq[b, h], tk[b, g], tv[b, g], go[b, h], gto[b, h],
                                bias, scale, tbias)
            gq[b, h], gtq[b, h] = r[0], r[3]
            gk[b, g] += r[1]
            gv[b, g] += r[2]
            gtk[b, g] += r[4]
            gtv[b, g] += r[5]
    return gq, gk, gv, gtq, gtk, gtv

