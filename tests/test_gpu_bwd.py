"""GPU parity of the reverse pass (jvpattn_bwd) against the float64 oracle.

Each case runs the HIP forward, then the HIP reverse pass on its outputs, and
compares the six cotangents with ``oracle_bwd`` on the same (rounded) inputs,
element by element. The bar per output is rho times its term magnitude M:
the same sums with every factor replaced by its absolute value (M >= |ref|
elementwise; it exceeds |ref| where terms cancel, e.g. the score cotangent
P (dP - del), whose two parts come through different roundings -- del from
the 16-bit O and dO the forward returned). rho is the forward's: 2^-6 (bf16),
2^-8 (fp16), covering the rounding of the recomputed weights, their tangents
and the score cotangents to the input type before the products.
"""
import numpy as np
import pytest
import torch

from forward_mode_autodiff_amd import inputs as I
from forward_mode_autodiff_amd.jvpattn import JvpattnError, jvpattn_bwd, jvpattn_fwd
from oracle import oracle_bwd
from oracle.attention import _head_bias
from tests.parity import RHO

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "dtq", "dtk", "dtv")


def f64(t):
    return None if t is None else t.double().numpy()


def run(w, x=None, tangents=("tq", "tk", "tv"), scale=None, heads=None):
    x = I.make_inputs(w, cotangents=True) if x is None else x
    d = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    t = {n: (d[n] if n in tangents else None) for n in ("tq", "tk", "tv")}
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], t["tq"], t["tk"], t["tv"], mask=d["mask"],
                                   causal=w.causal, scale=scale)
    g = jvpattn_bwd(d["q"], d["k"], d["v"], t["tq"], t["tk"], t["tv"], o, to, lse, tlse, d["do"], d["dto"],
                    mask=d["mask"], causal=w.causal, scale=scale)
    torch.cuda.synchronize()
    got = {n: a.float().cpu().numpy() for n, a in zip(NAMES, g)}
    mask = None
    if x["mask"] is not None:
        mask = f64(x["mask"]) if w.mask_kind == "additive" else x["mask"].numpy()
    tv = {n: (f64(x[n]) if n in tangents else None) for n in ("tq", "tk", "tv")}
    # heads: check only those heads of batch 0
    sel = (lambda a: a) if heads is None else (lambda a: None if a is None else a[:1, heads])
    msel = mask
    if mask is not None and heads is not None:
        msel = mask[:1] if mask.shape[1] == 1 else mask[:1, heads]
    ref = oracle_bwd(sel(f64(x["q"])), sel(f64(x["k"])), sel(f64(x["v"])), sel(tv["tq"]), sel(tv["tk"]),
                     sel(tv["tv"]), sel(f64(x["do"])), sel(f64(x["dto"])), mask=msel, mask_kind=w.mask_kind,
                     causal=w.causal, scale=scale)
    if heads is not None:
        got = {n: a[:1, heads] for n, a in got.items()}
    return got, dict(zip(NAMES, ref))


def term_magnitudes(x, w, tangents, scale, heads=None, tmask=None):
    """Per output, max over elements of the sum of absolute terms (see the module docstring)."""
    A = lambda n: None if x[n] is None else np.abs(f64(x[n]))
    q, k, v, g, gd = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["do"]), f64(x["dto"])
    z = lambda n, like: f64(x[n]) if n in tangents else np.zeros_like(like)
    tq, tk, tv = z("tq", q), z("tk", k), z("tv", v)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    grp = H // Hkv
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    mask = None
    if x["mask"] is not None:
        mask = f64(x["mask"]) if w.mask_kind == "additive" else x["mask"].numpy()
    M = {n: 0.0 for n in NAMES}
    kside = {}   # (b, key/value head) -> summed magnitudes over the query heads that read it
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            kh = h // grp
            k_, v_, tk_, tv_ = k[b, kh], v[b, kh], tk[b, kh], tv[b, kh]
            bias = _head_bias(mask, w.mask_kind, b, h, Nq, Nk, w.causal, np.arange(Nq))
            S = sc * q[b, h] @ k_.T + bias
            P = np.zeros_like(S)
            live = ~np.all(np.isneginf(S), axis=1)
            if live.any():
                e = np.exp(S[live] - S[live].max(1, keepdims=True))
                P[live] = e / e.sum(1, keepdims=True)
            Sd = sc * (tq[b, h] @ k_.T + q[b, h] @ tk_.T)
            if tmask is not None:   # the additive mask's tangent joins the score tangent
                Sd = Sd + _head_bias(tmask, "additive", b, h, Nq, Nk, False, np.arange(Nq))
            t = (P * Sd).sum(1, keepdims=True)
            aG, aGd = np.abs(g[b, h]), np.abs(gd[b, h])
            aX = aG @ np.abs(v_).T + aGd @ np.abs(tv_).T
            aD = aGd @ np.abs(v_).T
            o = P @ v_
            to = (P * (Sd - t)) @ v_ + P @ tv_
            r = np.abs((gd[b, h] * o).sum(1, keepdims=True))
            dl = np.abs((g[b, h] * o).sum(1, keepdims=True)) + np.abs((gd[b, h] * to).sum(1, keepdims=True)) \
                + np.abs(t) * r
            aS = P * (aX + aD * np.abs(Sd - t) + r * np.abs(Sd) + dl)
            aSd = P * (aD + r)
            aK, aTK, aQ, aTQ = np.abs(k_), np.abs(tk_), np.abs(q[b, h]), np.abs(tq[b, h])
            upd = {"dq": sc * (aS @ aK + aSd @ aTK), "dtq": sc * aSd @ aK,
                   "dk": sc * (aS.T @ aQ + aSd.T @ aTQ), "dtk": sc * aSd.T @ aQ,
                   "dv": P.T @ aG + np.abs(P * (Sd - t)).T @ aGd, "dtv": P.T @ aGd}
            for n, a in upd.items():
                if n in ("dk", "dtk", "dv", "dtv"):
                    kside[(b, kh, n)] = kside.get((b, kh, n), 0.0) + a
                elif a.size:
                    M[n] = max(M[n], float(a.max()))
    for (_, _, n), a in kside.items():
        if np.size(a):
            M[n] = max(M[n], float(np.max(a)))
    return M


def check(w, x=None, tangents=("tq", "tk", "tv"), scale=None):
    x = I.make_inputs(w, cotangents=True) if x is None else x
    got, ref = run(w, x=x, tangents=tangents, scale=scale)
    M = term_magnitudes(x, w, tangents, scale)
    bad = []
    for n in NAMES:
        g, r = got[n], ref[n]
        assert np.all(np.isfinite(g)), f"{w.name}: {n} not finite"
        err = float(np.max(np.abs(g - r))) if r.size else 0.0
        top = float(np.max(np.abs(r))) if r.size else 0.0
        print(f"{w.name} {w.dtype} {n}: err {err:.2e}  max|ref| {top:.2e}  M {M[n]:.2e}  err/M {err / max(M[n], 1e-30):.2e}")
        assert M[n] >= top * (1 - 1e-12), (n, M[n], top)
        if not err <= RHO[w.dtype] * M[n]:
            bad.append(f"{n}: err {err:.3e} > {RHO[w.dtype]:.2e} x M {M[n]:.3e} (max|ref| {top:.3e})")
    assert not bad, f"{w.name}: " + "; ".join(bad)
    return got, ref


def W(name, N=200, dtype="bf16", causal=False, std=1.0, seed=5, **kw):
    return I.Workload(name, B=1, H=2, N=N, d=64, dtype=dtype, causal=causal, std=std, seed=seed, **kw)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("std", [None, 1.0, 2.0], ids=["spec", "s1", "s2"])
def test_small(dtype, causal, std):
    check(W("small", dtype=dtype, causal=causal, std=std, seed=41))


@pytest.mark.parametrize("N", [1, 31, 32, 33, 97, 128, 129, 257, 513])
def test_ragged_lengths(N):
    check(W(f"len{N}", N=N, causal=N % 2 == 1, seed=N))


@pytest.mark.parametrize("mask_kind", ["bool", "additive"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_masks(mask_kind, causal, dtype):
    check(W("mask", N=160, dtype=dtype, causal=causal, mask_kind=mask_kind, keep=0.7, seed=42,
            mask_heads=2 if mask_kind == "additive" else 1))


@pytest.mark.parametrize("Nq,Nk", [(64, 200), (200, 64), (1, 300), (130, 1), (33, 257)])
@pytest.mark.parametrize("causal", [False, True])
def test_rectangular(Nq, Nk, causal):
    check(I.Workload("rect", B=1, H=2, N=Nq, Nk=Nk, d=64, dtype="bf16", causal=causal, std=1.0, seed=43))


@pytest.mark.parametrize("tangents", [("tv",), ("tq", "tk"), ()], ids=lambda t: "+".join(t) or "none")
def test_missing_tangents(tangents):
    check(W("tang", N=150, seed=44), tangents=tangents)


def test_custom_scale_fp16():
    check(W("scale", N=150, dtype="f16", seed=45), scale=0.3)


def test_custom_scale_bf16_not_power_of_two():
    check(W("scale2", N=150, dtype="bf16", causal=True, seed=50), scale=0.2)


def test_fully_masked_rows_give_zero_row_gradients():
    w = W("dead", N=96, mask_kind="bool", seed=46)
    x = I.make_inputs(w, cotangents=True)
    x["mask"][:, :, 5, :] = 0
    x["mask"][:, :, 70, :] = 0
    got, ref = check(w, x=x)
    for n in ("dq", "dtq"):
        assert np.all(got[n][:, :, [5, 70]] == 0)


def test_no_query_rows_give_zero_key_gradients():
    w = I.Workload("noq", B=1, H=2, N=0, Nk=70, d=64, dtype="bf16", std=1.0, seed=47)
    x = I.make_inputs(w, cotangents=True)
    d = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    o = torch.empty_like(d["q"])
    lse = torch.empty((1, 2, 0), device=DEV)
    g = jvpattn_bwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], o, o.clone(), lse, lse.clone(),
                    d["do"], d["dto"], out=tuple(torch.full_like(t, 7) for t in (d["q"], d["k"], d["v"], d["q"],
                                                                                  d["k"], d["v"])))
    torch.cuda.synchronize()
    for n, t in zip(NAMES, g):
        if t.numel():
            assert torch.all(t == 0), n


def test_hvp_workload_sampled_heads():
    """B=4, H=16, N=2048, d=64, bf16, causal: every head computed, two heads of batch 0 checked whole."""
    w = I.HVP
    x = I.make_inputs(w, cotangents=True)
    got, ref = run(w, x=x, heads=[3, 14])
    sub = {n: (None if t is None else t[:1]) for n, t in x.items()}
    M = term_magnitudes(sub, w, ("tq", "tk", "tv"), None, heads=[3, 14])
    for n in NAMES:
        err = float(np.max(np.abs(got[n] - ref[n])))
        print(f"hvp {n}: err {err:.2e} M {M[n]:.2e}")
        assert err <= RHO["bf16"] * M[n], (n, err, M[n])


def test_deterministic():
    w = W("det", N=300, causal=True, seed=48)
    a, _ = run(w)
    b, _ = run(w)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


def test_errors_raise():
    x = I.make_inputs(W("err", N=64, dtype="f32" if False else "bf16", seed=49), cotangents=True)
    d = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"])
    with pytest.raises(JvpattnError):   # cotangent aliases an output
        out = tuple(torch.empty_like(t) for t in (d["q"], d["k"], d["v"], d["q"], d["k"], d["v"]))
        jvpattn_bwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], o, to, lse, tlse, d["do"], out[0],
                    out=out)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(JvpattnError):   # workspace too small
        jvpattn_bwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], o, to, lse, tlse, d["do"], d["dto"],
                    workspace=ws)


def test_null_cotangent_and_skipped_outputs():
    """go = NULL is a zero cotangent; NULL dtq/dtk/dtv outputs are skipped, the others unchanged."""
    w = W("nullg", N=130, causal=True, seed=51)
    x = I.make_inputs(w, cotangents=True)
    d = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], causal=True)
    out = (torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]), None, None, None)
    g = jvpattn_bwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], o, to, lse, tlse, None, d["dto"],
                    causal=True, out=out)
    full = jvpattn_bwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], o, to, lse, tlse,
                       torch.zeros_like(d["do"]), d["dto"], causal=True)
    torch.cuda.synchronize()
    assert g[3] is None and g[4] is None and g[5] is None
    for a, b in zip(g[:3], full[:3]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("H,Hkv,causal,dtype", [(4, 2, False, "bf16"), (6, 3, True, "f16"), (4, 1, True, "bf16")],
                         ids=["gqa2", "gqa2-causal-f16", "mqa-causal"])
def test_grouped_kv_heads(H, Hkv, causal, dtype):
    w = I.Workload(f"gqa_bwd_{H}_{Hkv}", B=2, H=H, Hkv=Hkv, N=200, d=64, dtype=dtype, causal=causal, std=1.0,
                   seed=21)
    check(w)


def test_grouped_kv_heads_bool_mask_ragged():
    w = I.Workload("gqa_bwd_bool", B=1, H=4, Hkv=2, N=157, d=64, dtype="bf16", mask_kind="bool", mask_heads=4,
                   keep=0.6, std=1.0, seed=22)
    check(w)


@pytest.mark.parametrize("layout,kind", [("pad_right", "bool"), ("window", "additive")])
def test_key_masks(layout, kind):
    w = I.Workload(f"keymask_bwd_{layout}", B=3, H=2, N=180, d=64, dtype="bf16", mask_kind=kind, mask_layout=layout,
                   std=1.0, seed=23)
    check(w)


@pytest.mark.parametrize("causal", [False, True])
def test_bit_packed_masks(causal):
    """The reverse pass with a bit-packed mask: the bool mask's cotangents (the oracle's bar)."""
    from forward_mode_autodiff_amd.jvpattn import pack_mask_bits
    w = I.Workload("bits_bwd", B=2, H=2, N=190, d=64, dtype="bf16", causal=causal, mask_kind="bool", keep=0.7,
                   std=1.0, seed=24)
    x = I.make_inputs(w, cotangents=True)
    xb = dict(x, mask=pack_mask_bits(x["mask"]))
    d = {k: (None if v is None else v.to(DEV)) for k, v in xb.items()}
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=d["mask"], causal=causal)
    g = jvpattn_bwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], o, to, lse, tlse, d["do"], d["dto"],
                    mask=d["mask"], causal=causal)
    torch.cuda.synchronize()
    ref = oracle_bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["tq"]), f64(x["tk"]), f64(x["tv"]),
                     f64(x["do"]), f64(x["dto"]), mask=x["mask"].numpy(), mask_kind="bool", causal=causal)
    M = term_magnitudes(x, w, ("tq", "tk", "tv"), None)
    for n, gg, r in zip(NAMES, g, ref):
        err = float(np.max(np.abs(gg.float().cpu().numpy() - r)))
        assert err <= RHO[w.dtype] * M[n], (n, err, M[n])


@pytest.mark.parametrize("causal,dtype", [(False, "bf16"), (True, "f16")])
def test_mask_tangent(causal, dtype):
    """jvpattn_bwd_tmask: the reverse pass of the forward along (dQ, dK, dV, dM), against the oracle."""
    w = I.Workload("tmask_bwd", B=2, H=2, N=170, d=64, dtype=dtype, causal=causal, mask_kind="additive",
                   std=1.0, seed=25)
    x = I.make_inputs(w, cotangents=True)
    g = torch.Generator().manual_seed(26)
    tm = torch.randn(x["mask"].shape, generator=g).to(x["mask"].dtype)
    d = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=d["mask"], causal=causal,
                                   tmask=tm.to(DEV))
    got = jvpattn_bwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], o, to, lse, tlse, d["do"], d["dto"],
                      mask=d["mask"], causal=causal, tmask=tm.to(DEV))
    torch.cuda.synchronize()
    ref = oracle_bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["tq"]), f64(x["tk"]), f64(x["tv"]),
                     f64(x["do"]), f64(x["dto"]), mask=f64(x["mask"]), mask_kind="additive", causal=causal,
                     tmask=f64(tm))
    M = term_magnitudes(x, w, ("tq", "tk", "tv"), None, tmask=f64(tm))
    for n, gg, r in zip(NAMES, got, ref):
        gg = gg.float().cpu().numpy()
        assert np.all(np.isfinite(gg)), n
        err = float(np.max(np.abs(gg - r)))
        assert err <= RHO[dtype] * M[n], (n, err, M[n])
