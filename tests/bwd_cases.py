"""Reverse-pass parity cases shared by the GPU tests and the CPU proof of the bar's power.

``reference`` runs the float64 oracle (``oracle_bwd``) and ``magnitudes`` the per-element term
magnitudes of the bar (tests/parity.py) on the inputs of a workload, for every head or for a few
query heads of batch 0 (the full-size HVP shape). The GPU tests compare the HIP reverse pass with
these; tests/test_oracle_bwd_mutants.py plants mistakes in the oracle and shows the same bar
rejects each of them on the same cases.
"""
from __future__ import annotations

import numpy as np

from forward_mode_autodiff_amd import inputs as I
from oracle import oracle_bwd
from oracle.attention import _head_bias
from tests.parity import BWD_NAMES, bwd_term_magnitudes


def f64(t):
    return None if t is None else t.double().numpy()


def mask_np(x, w):
    if x["mask"] is None:
        return None
    return f64(x["mask"]) if w.mask_kind == "additive" else x["mask"].numpy()


def _sel(a, heads):
    return a if heads is None or a is None else a[:1, heads]


def reference(x, w, tangents=("tq", "tk", "tv"), scale=None, heads=None, tmask=None):
    """oracle_bwd on the workload's inputs: dict of the six cotangents (batch 0, `heads` only if given)."""
    tv = {n: (f64(x[n]) if n in tangents else None) for n in ("tq", "tk", "tv")}
    mask = mask_np(x, w)
    msel = mask
    if mask is not None and heads is not None:
        msel = mask[:1] if mask.shape[1] == 1 else mask[:1, heads]
    tm = None if tmask is None else np.asarray(tmask, np.float64)
    if tm is not None and heads is not None:
        tm = tm[:1] if tm.shape[1] == 1 else tm[:1, heads]
    ref = oracle_bwd(_sel(f64(x["q"]), heads), _sel(f64(x["k"]), heads), _sel(f64(x["v"]), heads),
                     _sel(tv["tq"], heads), _sel(tv["tk"], heads), _sel(tv["tv"], heads),
                     _sel(f64(x["do"]), heads), _sel(f64(x["dto"]), heads), mask=msel, mask_kind=w.mask_kind,
                     causal=w.causal, scale=scale, tmask=tm)
    return dict(zip(BWD_NAMES, ref))


def magnitudes(x, w, tangents=("tq", "tk", "tv"), scale=None, heads=None, tmask=None):
    """Per-element term magnitudes of the six cotangents, shaped like ``reference``'s results."""
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    z = lambda n, like: f64(x[n]) if n in tangents else np.zeros_like(like)
    tq, tk, tv = z("tq", q), z("tk", k), z("tv", v)
    d = q.shape[-1]
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    mask = mask_np(x, w)
    Nq, Nk = q.shape[2], k.shape[2]
    rows = np.arange(Nq)
    bias_of = lambda b, h: _head_bias(mask, w.mask_kind, b, h, Nq, Nk, w.causal, rows)
    tbias_of = None
    if tmask is not None:
        tm = np.asarray(tmask, np.float64)
        tbias_of = lambda b, h: _head_bias(tm, "additive", b, h, Nq, Nk, False, rows)
    return bwd_term_magnitudes(q, k, v, tq, tk, tv, f64(x["do"]), f64(x["dto"]), bias_of, sc, heads=heads,
                               tbias_of=tbias_of)


def small(name, N=200, dtype="bf16", causal=False, std=1.0, seed=5, **kw):
    return I.Workload(name, B=1, H=2, N=N, d=64, dtype=dtype, causal=causal, std=std, seed=seed, **kw)


# Full-size HVP workload (B=4, H=16, N=2048, d=64, bf16, causal), checked on two query heads of batch 0:
# at the specified 1/sqrt(d) spread and at unit spread, where the terms carried by the score tangent
# and tlse stand out of the rounding noise.
HVP_HEADS = [3, 14]
HVP_UNIT = I.Workload("hvp_s1", B=4, H=16, N=2048, d=64, dtype="bf16", causal=True, std=1.0, seed=8)

# The six small configurations of the GPU test ``test_small`` (seed 41): dtype x causal x spread.
SMALL = [small("small", dtype=dt, causal=c, std=s, seed=41)
         for dt in ("bf16", "f16") for c in (False, True) for s in (None, 1.0, 2.0)]
