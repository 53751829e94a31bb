"""Comparison bars for GPU results against the float64 oracle.

Two bars apply to O and dO:
  * the absolute bar the method is specified with: max-abs error <= 2e-3 for
    float32 inputs and <= 1e-2 for bfloat16 / float16 inputs, on inputs with
    the specified N(0,1)/sqrt(d) spread (``spec_spread=True``). At larger
    spreads the outputs grow past 1 and a 16-bit output's own rounding
    (half an ulp: 2^-8 relative for bf16) exceeds any fixed absolute bar, so
    there only the scale-free bar applies;
  * always, a scale-free bar, max-abs error <= rho * max|reference|, with rho = 2^-6
    (bf16), 2^-8 (fp16), 1e-4 (fp32). It is what gives the stress inputs
    (unit and doubled spread) their power: at the 1/sqrt(d) spread every
    output is below 1e-2 and the absolute bar alone would pass an all-zero
    result. rho is 4x the unit roundoff of the working type (bf16: 2^-8, fp16:
    2^-10 for the rounded softmax weights and outputs), covering the
    rounding of P and P*dS to the input type before the value products plus
    the final rounding of O and dO; fp32 has no such rounding step and keeps
    1e-4 for accumulation order.
lse: error <= 1e-3 (16-bit) / 1e-5 (fp32) plus 2^-20 |lse| (16 float32 ulps of
the value: lse is formed in float32 from float32 scores, so its own rounding
grows with its size and passes any fixed bar once scores reach the hundreds),
and -inf exactly where the reference is -inf (fully masked rows). tlse: the
same two bars as dO.
"""
from __future__ import annotations

import numpy as np

ABS_TOL = {"f32": 2e-3, "f16": 1e-2, "bf16": 1e-2}
RHO = {"f32": 1e-4, "f16": 2.0 ** -8, "bf16": 2.0 ** -6}
LSE_TOL = {"f32": 1e-5, "f16": 1e-3, "bf16": 1e-3}
LSE_REL = 2.0 ** -20


def _np(x):
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def errors(got: dict, ref: dict, dtype: str, spec_spread: bool = False) -> dict:
    """Per-output (max-abs error, bar, max|ref|); keys o, to, lse, tlse present in both."""
    out = {}
    for name in ("o", "to", "tlse"):
        if name not in got or got[name] is None:
            continue
        g, r = _np(got[name]), _np(ref[name])
        scale = float(np.max(np.abs(r))) if r.size else 0.0
        if not np.all(np.isfinite(g)):
            out[name] = (float("inf"), 0.0, scale)
            continue
        err = float(np.max(np.abs(g - r))) if g.size else 0.0
        bar = RHO[dtype] * scale
        if spec_spread:
            bar = min(bar, ABS_TOL[dtype])
        out[name] = (err, bar, scale)
    if "lse" in got and got["lse"] is not None:
        g, r = _np(got["lse"]), _np(ref["lse"])
        inf_r = np.isneginf(r)
        if not np.array_equal(np.isneginf(g), inf_r) or not np.all(np.isfinite(g[~inf_r])):
            out["lse"] = (float("inf"), 0.0, 0.0)
        else:
            if (~inf_r).any():
                # worst ratio of error to the row's own bar, reported against the bar of the largest |lse|
                gr, rr = g[~inf_r], r[~inf_r]
                bars = LSE_TOL[dtype] + LSE_REL * np.abs(rr)
                i = int(np.argmax(np.abs(gr - rr) / bars))
                out["lse"] = (float(abs(gr[i] - rr[i])), float(bars[i]), float(np.max(np.abs(rr))))
            else:
                out["lse"] = (0.0, LSE_TOL[dtype], 0.0)
    return out


def failures(got: dict, ref: dict, dtype: str, spec_spread: bool = False) -> list:
    return [f"{k}: err {e:.3e} > bar {b:.3e} (max|ref| {m:.3e})"
            for k, (e, b, m) in errors(got, ref, dtype, spec_spread).items() if not e <= b]


def assert_parity(got: dict, ref: dict, dtype: str, what: str = "", spec_spread: bool = False):
    bad = failures(got, ref, dtype, spec_spread)
    assert not bad, f"{what}: " + "; ".join(bad)


# ---------------------------------------------------------------- reverse pass

BWD_NAMES = ("dq", "dk", "dv", "dtq", "dtk", "dtv")
# Elements whose term magnitude is below this fraction of the output's largest one are held to
# that floor instead (a row with no visible key has M = 0 and must come back as exactly 0 there).
BWD_FLOOR = 2.0 ** -20
# Absolute rounding error of a value rounded to the working type below its normal range: half the
# subnormal spacing (float16: normal values start at 2^-14, subnormals are spaced 2^-24). Relative
# bars cannot cover it -- a float16 weight of 1e-6 carries an error of up to 2^-25, 3% of itself.
SUBNORMAL_HALF_ULP = {"f16": 2.0 ** -25, "bf16": 2.0 ** -134, "f32": 2.0 ** -150}


def bwd_term_magnitudes(q, k, v, tq, tk, tv, go, gto, bias_of, scale, heads=None, tbias_of=None):
    """Per-element term magnitudes M of the six cotangents (float64 arrays shaped like them).

    M is the reverse pass with every factor replaced by its absolute value, so M >= |ref| element by
    element, and it exceeds |ref| where terms cancel -- e.g. the score cotangent P (dP - del), whose
    two parts reach the kernel through different roundings (del from the 16-bit O and dO the forward
    returned). Rounding any factor of a term to a t-bit mantissa moves that element by at most
    2^-t times its share of M, which is what a bar rho * M_ij covers.

    q, tq, go, gto: [B, H, Nq, d]; k, v, tk, tv: [B, Hkv, Nk, d] (float64; zero arrays for absent
    tangents). bias_of(b, h) -> [Nq, Nk] additive bias (0 / -inf / mask values, causal applied);
    tbias_of(b, h) -> the mask tangent's [Nq, Nk] or None. heads: None for every head, or a list of
    query heads of batch 0 (then the outputs cover batch 0 and those heads, and the key-side sums
    cover only them -- callers use it without grouped heads).

    Also returns, under the key "floor", the partner magnitudes of the rounded factors summed over
    the visible (query, key) pairs that reach each element (A: dq <- scale sum_j (|k_j| + |dk_j|),
    dk <- scale sum_i (|q_i| + |dq_i|), dv <- sum_i (|gO_i| + |gdO_i|), and likewise for the
    tangent cotangents): a weight, score cotangent or output below the working type's normal range
    is off by up to half a subnormal spacing, times that partner.
    """
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    grp = H // Hkv
    hl = list(range(H)) if heads is None else list(heads)
    bl = list(range(B)) if heads is None else [0]
    nqh = len(hl) if heads is not None else H
    nkh = len(hl) if heads is not None else Hkv
    M = {n: np.zeros((len(bl), nqh, Nq, d)) for n in ("dq", "dtq")}
    M.update({n: np.zeros((len(bl), nkh, Nk, d)) for n in ("dk", "dtk", "dv", "dtv")})
    F = {n: np.zeros_like(a) for n, a in M.items()}
    for bi, b in enumerate(bl):
        for hi, h in enumerate(hl):
            kh = h // grp
            ko = hi if heads is not None else kh       # where the key-side sums go
            qo = hi if heads is not None else h
            k_, v_, tk_, tv_ = k[b, kh], v[b, kh], tk[b, kh], tv[b, kh]
            S = scale * q[b, h] @ k_.T + bias_of(b, h)
            P = np.zeros_like(S)
            live = ~np.all(np.isneginf(S), axis=1)
            if live.any():
                e = np.exp(S[live] - S[live].max(1, keepdims=True))
                P[live] = e / e.sum(1, keepdims=True)
            Sd = scale * (tq[b, h] @ k_.T + q[b, h] @ tk_.T)
            tb = None if tbias_of is None else tbias_of(b, h)
            if tb is not None:
                Sd = Sd + tb
            t = (P * Sd).sum(1, keepdims=True)
            g, gd = go[b, h], gto[b, h]
            aG, aGd = np.abs(g), np.abs(gd)
            aX = aG @ np.abs(v_).T + aGd @ np.abs(tv_).T
            aD = aGd @ np.abs(v_).T
            o = P @ v_
            to = (P * (Sd - t)) @ v_ + P @ tv_
            r = np.abs((gd * o).sum(1, keepdims=True))
            dl = np.abs((g * o).sum(1, keepdims=True)) + np.abs((gd * to).sum(1, keepdims=True)) + np.abs(t) * r
            aS = P * (aX + aD * np.abs(Sd - t) + r * np.abs(Sd) + dl)
            aSd = P * (aD + r)
            aK, aTK, aQ, aTQ = np.abs(k_), np.abs(tk_), np.abs(q[b, h]), np.abs(tq[b, h])
            M["dq"][bi, qo] = scale * (aS @ aK + aSd @ aTK)
            M["dtq"][bi, qo] = scale * aSd @ aK
            M["dk"][bi, ko] += scale * (aS.T @ aQ + aSd.T @ aTQ)
            M["dtk"][bi, ko] += scale * aSd.T @ aQ
            M["dv"][bi, ko] += P.T @ aG + np.abs(P * (Sd - t)).T @ aGd
            M["dtv"][bi, ko] += P.T @ aGd
            vis = np.isfinite(S).astype(np.float64)    # visible (query, key) pairs
            F["dq"][bi, qo] = scale * vis @ (aK + aTK)
            F["dtq"][bi, qo] = scale * vis @ aK
            F["dk"][bi, ko] += scale * vis.T @ (aQ + aTQ)
            F["dtk"][bi, ko] += scale * vis.T @ aQ
            F["dv"][bi, ko] += vis.T @ (aG + aGd)
            F["dtv"][bi, ko] += vis.T @ aGd
    M["floor"] = F
    return M


def bwd_errors(got: dict, ref: dict, M: dict, dtype: str) -> dict:
    """Per cotangent: (worst err_ij / bar_ij, index, err, bar there, power) with
    bar_ij = rho * max(M_ij, BWD_FLOOR * max M) + eta * (floor_ij + 1), eta = SUBNORMAL_HALF_ULP[dtype]
    (the "+ 1": the output's own rounding). power = True when an all-zero result would fail the bar
    (some |ref_ij| > bar_ij)."""
    out = {}
    for n in BWD_NAMES:
        g, r, m = np.asarray(got[n], np.float64), np.asarray(ref[n], np.float64), M[n]
        if r.size == 0:
            out[n] = (0.0, None, 0.0, 0.0, True)
            continue
        if not np.all(np.isfinite(g)):
            out[n] = (float("inf"), None, float("inf"), 0.0, True)
            continue
        bar = RHO[dtype] * np.maximum(m, BWD_FLOOR * float(m.max()))
        bar = bar + SUBNORMAL_HALF_ULP[dtype] * (M["floor"][n] + 1)
        ratio = np.abs(g - r) / np.where(bar > 0, bar, np.inf)
        ratio = np.where((bar == 0) & (g != r), np.inf, ratio)
        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        power = bool(np.any(np.abs(r) > bar))
        out[n] = (float(ratio[i]), i, float(abs(g[i] - r[i])), float(bar[i]), power)
    return out


def bwd_failures(got: dict, ref: dict, M: dict, dtype: str) -> list:
    return [f"{n}: err {e:.3e} > bar {b:.3e} at {i} (worst ratio {q:.2f})"
            for n, (q, i, e, b, _) in bwd_errors(got, ref, M, dtype).items() if not q <= 1.0]
