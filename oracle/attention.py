"""Plain float64 oracle: scaled-dot-product attention and its forward-mode derivative.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP library and imports nothing from it.

What is computed, and where it comes from
-----------------------------------------
* The primal is PyTorch's ``scaled_dot_product_attention`` without dropout:
  the "JVP Flash Attention" README (section "Usage") presents the method as a
  drop-in replacement for that call, taking ``q, k, v`` and ``attn_mask``,
  with dropout unsupported.
* Per head it is the plain textbook computation shown in the naive MHSA script
  of the equinox issue "Flash Attention" (#732): scores are q.k divided by the
  square root of the key depth, a softmax over the key axis, then the weights
  applied to V. The data generator in that script fixes the tensor layout as
  (batch, heads, seq, dim).
* The derivative: the README's "Description" says the kernel supports
  Jacobian-vector products. A JVP is the directional derivative
  d/dt O(Q + t*dQ, K + t*dK, V + t*dV) at t = 0, written out here with the
  product rule and the derivative of softmax:

      S   = scale * Q K^T + M            M: mask bias
      P   = softmax_j(S)
      O   = P V
      dS  = scale * (dQ K^T + Q dK^T) + dM   dM: tangent of an additive mask (else 0)
      dP  = P * (dS - rowsum(P * dS))    derivative of softmax
      dO  = dP V + P dV                  product rule

  ``tlse = rowsum(P * dS)`` is also the derivative of ``lse = logsumexp_j(S)``,
  so every returned quantity is a value/tangent pair.

Readings taken where the pages say nothing (each is listed in the design notes):
  * boolean mask: nonzero/True = the key takes part (SDPA's convention);
  * additive mask: added after scaling; constant unless a tangent dM of it
    is given (then it enters dS as the derivative of S = scale QK^T + M);
  * causal: key j is visible to query i iff j <= i (top-left aligned, as
    SDPA's ``is_causal``); with an explicit mask both restrictions apply;
  * a row whose every score is -inf ("fully masked") gives O = dO = 0,
    lse = -inf, tlse = 0;
  * lse uses the natural logarithm;
  * grouped key/value heads (fewer K/V heads than query heads, as SDPA's
    ``enable_gqa``): query head h attends with key/value head h // (H // Hkv).
No blocking, no online softmax and no fusion: the softmax is the two-pass
definition (max, exponentials, normalise).
"""
from __future__ import annotations

import math

import numpy as np

MASK_NONE = "none"
MASK_BOOL = "bool"
MASK_ADDITIVE = "additive"
MASK_BITS = "bits"


def unpack_mask_bits(words, Nk):
    """Boolean [..., Nk] from a bit-packed mask [..., ceil(Nk/32)] of 32-bit words:
    key j is visible iff bit (j mod 32) of word j // 32 is set."""
    w = np.asarray(words).astype(np.uint64)
    j = np.arange(Nk)
    return ((w[..., j // 32] >> (j % 32).astype(np.uint64)) & 1).astype(bool)


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _head_bias(mask, mask_kind, b, h, nq_rows, Nk, causal, q_pos):
    """Additive bias M for one head: 0 where a key is visible, -inf where not.

    ``q_pos`` holds the absolute query index of each row (used by causal and to
    pick mask rows), so a subset of query rows can be evaluated on its own.
    """
    M = np.zeros((nq_rows, Nk), dtype=np.float64)
    if mask_kind != MASK_NONE:
        mb = mask[b if mask.shape[0] > 1 else 0, h if mask.shape[1] > 1 else 0]
        # a mask with one row is shared by every query (a key-padding mask), as in SDPA's broadcasting
        rows = mb[np.zeros_like(q_pos) if mb.shape[0] == 1 else q_pos, :]
        if mask_kind == MASK_BOOL:
            M = np.where(rows != 0, 0.0, -np.inf)
        elif mask_kind == MASK_BITS:
            M = np.where(unpack_mask_bits(rows, Nk), 0.0, -np.inf)
        elif mask_kind == MASK_ADDITIVE:
            M = np.asarray(rows, dtype=np.float64).copy()
        else:
            raise ValueError(f"unknown mask kind {mask_kind!r}")
    if causal:
        j = np.arange(Nk)[None, :]
        M = np.where(j <= q_pos[:, None], M, -np.inf)
    return M


def oracle_fwd_head(q, k, v, tq, tk, tv, bias, scale, tbias=None):
    """One head. q,tq: [n, d]; k,v,tk,tv: [Nk, d]; bias: [n, Nk] (0 / -inf / value);
    tbias: [n, Nk] tangent of an additive mask, or None.

    Returns (o, to, lse, tlse) in float64.
    """
    S = scale * (q @ k.T) + bias
    dS = scale * (tq @ k.T + q @ tk.T)
    if tbias is not None:
        dS = dS + tbias
    n, d = q.shape
    o = np.zeros((n, v.shape[1]))
    to = np.zeros((n, v.shape[1]))
    lse = np.full(n, -np.inf)
    tlse = np.zeros(n)
    live = ~np.all(np.isneginf(S), axis=1)  # rows with at least one visible key
    if not np.any(live):
        return o, to, lse, tlse
    S, dS = S[live], dS[live]
    m = np.max(S, axis=1, keepdims=True)
    e = np.exp(S - m)
    s = np.sum(e, axis=1, keepdims=True)
    P = e / s
    o_l = P @ v
    t_l = np.sum(P * dS, axis=1, keepdims=True)
    dP = P * (dS - t_l)
    o[live] = o_l
    to[live] = dP @ v + P @ tv
    lse[live] = (m + np.log(s))[:, 0]
    tlse[live] = t_l[:, 0]
    return o, to, lse, tlse


def kv_head(h, H, Hkv):
    """Key/value head read by query head h when H query heads share Hkv key/value heads."""
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"{H} query heads cannot be grouped over {Hkv} key/value heads")
    return h // (H // Hkv)


def oracle_fwd(q, k, v, tq=None, tk=None, tv=None, mask=None, mask_kind=MASK_NONE,
               causal=False, scale=None, q_pos=None, tmask=None):
    """Attention output and its JVP for [B, H, Nq, d] queries and [B, Hkv, Nk, d] keys/values.

    Hkv = H is plain multi-head attention; a divisor of H groups the query
    heads, query head h reading key/value head ``kv_head(h, H, Hkv)``.

    q, k, v, tq, tk, tv: array-likes (values already rounded to the working
        dtype; they are widened to float64 here). A tangent given as None is zero.
    mask: [Bm, Hm, Nm, Nk] with Bm in {1, B}, Hm in {1, H}, Nm in {1, Nq_full} (one
        row: shared by every query, e.g. a key-padding mask); uint8/bool for
        ``mask_kind="bool"``, float for ``"additive"``, 32-bit words
        [Bm, Hm, Nm, ceil(Nk/32)] for ``"bits"`` (a boolean mask, one bit per
        key); None for ``"none"``.
    causal: key j visible to query i iff j <= i.
    scale: multiplies Q K^T and the score tangent; default 1/sqrt(d).
    q_pos: optional absolute indices of the given query rows (defaults to
        0..Nq-1); lets a caller evaluate a sample of rows of a large problem.
    tmask: tangent of an additive mask, shaped like ``mask`` (additive only).

    Returns (o, to, lse, tlse): [B,H,Nq,d], [B,H,Nq,d], [B,H,Nq], [B,H,Nq] float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    tq = np.zeros_like(q) if tq is None else _f64(tq)
    tk = np.zeros_like(k) if tk is None else _f64(tk)
    tv = np.zeros_like(v) if tv is None else _f64(tv)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if q_pos is None:
        q_pos = np.arange(Nq)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    if mask is not None:
        mask = np.asarray(mask)
    if (mask is None) != (mask_kind == MASK_NONE):
        raise ValueError("mask must be given exactly when mask_kind is not 'none'")
    if tmask is not None and mask_kind != MASK_ADDITIVE:
        raise ValueError("a mask tangent needs an additive mask")
    dv = v.shape[3]
    o = np.empty((B, H, Nq, dv))
    to = np.empty((B, H, Nq, dv))
    lse = np.empty((B, H, Nq))
    tlse = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            bias = _head_bias(mask, mask_kind, b, h, Nq, Nk, causal, q_pos)
            # the mask's tangent, laid out as the mask; -inf entries of the mask make it irrelevant there
            tbias = None if tmask is None else _head_bias(tmask, MASK_ADDITIVE, b, h, Nq, Nk, False, q_pos)
            g = kv_head(h, H, Hkv)
            o[b, h], to[b, h], lse[b, h], tlse[b, h] = oracle_fwd_head(
                q[b, h], k[b, g], v[b, g], tq[b, h], tk[b, g], tv[b, g], bias, scale, tbias)
    return o, to, lse, tlse
