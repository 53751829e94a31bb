"""GPU parity of the reverse pass (jvpattn_bwd) against the float64 oracle.

Each case runs the HIP forward, then the HIP reverse pass on its outputs, and
compares the six cotangents with ``oracle_bwd`` on the same (rounded) inputs,
element by element. The bar is per element: |got_ij - ref_ij| <= rho * M_ij,
where M is the element's term magnitude -- the same sums with every factor
replaced by its absolute value (M >= |ref| elementwise; larger where terms
cancel, e.g. the score cotangent P (dP - del), whose two parts come through
different roundings: del from the 16-bit O and dO the forward returned). rho
is the forward's: 2^-6 (bf16), 2^-8 (fp16), covering the rounding of the
recomputed weights, their tangents and the score cotangents to the input type
before the products. Each check also asserts the bar has power: an all-zero
result would fail it. tests/test_oracle_bwd_mutants.py shows on the CPU that
the same bar rejects single-term mistakes planted in the oracle.
"""
import numpy as np
import pytest
import torch

from forward_mode_autodiff_amd import inputs as I
from forward_mode_autodiff_amd.jvpattn import (JvpattnError, jvpattn_bwd, jvpattn_bwd_set_overlap, jvpattn_fwd,
                                              jvpattn_set_workgroups)
from tests.bwd_cases import HVP_HEADS, HVP_UNIT, SMALL, f64, magnitudes, reference, small as W
from tests.parity import BWD_NAMES as NAMES, bwd_errors, bwd_failures

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def gpu_bwd(x, w, tangents=("tq", "tk", "tv"), scale=None, tmask=None, mask_kind=None):
    """HIP forward then reverse pass on the workload's inputs; the six cotangents as float64 numpy."""
    d = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    t = {n: (d[n] if n in tangents else None) for n in ("tq", "tk", "tv")}
    tm = None if tmask is None else tmask.to(DEV)
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], t["tq"], t["tk"], t["tv"], mask=d["mask"],
                                   causal=w.causal, scale=scale, tmask=tm, mask_kind=mask_kind)
    g = jvpattn_bwd(d["q"], d["k"], d["v"], t["tq"], t["tk"], t["tv"], o, to, lse, tlse, d["do"], d["dto"],
                    mask=d["mask"], causal=w.causal, scale=scale, tmask=tm, mask_kind=mask_kind)
    torch.cuda.synchronize()
    return {n: a.double().cpu().numpy() for n, a in zip(NAMES, g)}


def run(w, x=None, tangents=("tq", "tk", "tv"), scale=None, heads=None):
    x = I.make_inputs(w, cotangents=True) if x is None else x
    got = gpu_bwd(x, w, tangents, scale)
    ref = reference(x, w, tangents, scale, heads)
    if heads is not None:
        got = {n: a[:1, heads] for n, a in got.items()}
    return got, ref


def check(w, x=None, tangents=("tq", "tk", "tv"), scale=None, heads=None, tmask=None):
    """Per-element bar on every cotangent, and proof that the bar can see an all-zero result."""
    x = I.make_inputs(w, cotangents=True) if x is None else x
    got = gpu_bwd(x, w, tangents, scale, tmask)
    if heads is not None:
        got = {n: a[:1, heads] for n, a in got.items()}
    tm = None if tmask is None else f64(tmask)
    ref = reference(x, w, tangents, scale, heads, tm)
    M = magnitudes(x, w, tangents, scale, heads, tm)
    for n in NAMES:
        q, i, e, b, power = bwd_errors(got, ref, M, w.dtype)[n]
        top = float(np.max(np.abs(ref[n]))) if ref[n].size else 0.0
        print(f"{w.name} {w.dtype} {n}: worst err/bar {q:.3f} (err {e:.2e}, bar {b:.2e})  max|ref| {top:.2e}")
        assert np.all(M[n] >= np.abs(ref[n]) * (1 - 1e-12)), n
        if np.any(ref[n] != 0):
            assert power, f"{w.name}: the bar of {n} would accept an all-zero result"
    bad = bwd_failures(got, ref, M, w.dtype)
    assert not bad, f"{w.name}: " + "; ".join(bad)
    return got, ref


@pytest.mark.parametrize("w", SMALL, ids=lambda w: f"{w.dtype}-{'causal' if w.causal else 'full'}-std{w.std}")
def test_small(w):
    check(w)


@pytest.fixture
def _walk_cap():
    yield
    jvpattn_set_workgroups()


# The mask-free key side at d = 64 walks several (key block, K/V head) items
# per workgroup: the next item's K, dK, V, dV rows and first query tiles load
# during the current one's epilogue. A small cap forces many rounds on small
# inputs: the same bits as one item per workgroup, and oracle parity.
@pytest.mark.parametrize("cap", [8, 5, 24])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_walking_key_side(dtype, causal, cap, _walk_cap):
    shapes = [dict(B=2, H=4, N=700), dict(B=4, H=8, Hkv=2, N=300), dict(B=1, H=3, N=200, Nk=450),
              dict(B=2, H=2, N=40)]
    for i, s in enumerate(shapes):
        w = I.Workload(f"walkkv_{i}", d=64, dtype=dtype, causal=causal, std=1.0, seed=80 + i, **s)
        x = I.make_inputs(w, cotangents=True)
        jvpattn_set_workgroups(1 << 30)   # one item per workgroup
        one = gpu_bwd(x, w)
        jvpattn_set_workgroups(cap)
        got = gpu_bwd(x, w)
        for n in NAMES:
            assert np.array_equal(one[n], got[n]), (w.name, n)
        ref = reference(x, w)
        bad = bwd_failures(got, ref, magnitudes(x, w), w.dtype)
        assert not bad, f"{w.name}: " + "; ".join(bad)


@pytest.fixture
def _overlap_auto():
    yield
    jvpattn_bwd_set_overlap()


# The query side may run on a second stream beside the key side (the
# default for grouped K/V heads): the same bits as one stream, for every
# kernel family (d = 64 walking and masked, d = 128 in two key-side launches,
# float32), and oracle parity on the two-stream results.
@pytest.mark.parametrize("case", [
    dict(B=2, H=4, N=700, d=64, dtype="bf16", causal=True),
    dict(B=4, H=8, Hkv=2, N=300, d=64, dtype="f16", causal=True),
    dict(B=1, H=4, Hkv=1, N=157, d=64, dtype="bf16", mask_kind="bool", mask_heads=4, keep=0.6),
    dict(B=1, H=4, Hkv=2, N=200, Nk=260, d=128, dtype="bf16", causal=True),
    dict(B=1, H=4, Hkv=2, N=150, d=64, dtype="f32", causal=True),
], ids=["mha-walk", "gqa-walk-f16", "mqa-bool", "gqa-d128", "gqa-f32"])
def test_overlap_modes_agree(case, _overlap_auto):
    w = I.Workload("overlap", std=1.0, seed=90, **case)
    x = I.make_inputs(w, cotangents=True)
    jvpattn_bwd_set_overlap(False)
    one = gpu_bwd(x, w)
    jvpattn_bwd_set_overlap(True)
    two = gpu_bwd(x, w)
    for n in NAMES:
        assert np.array_equal(one[n], two[n]), n
    bad = bwd_failures(two, reference(x, w), magnitudes(x, w), w.dtype)
    assert not bad, "; ".join(bad)


def test_query_side_kernels_agree_at_the_hvp_shape(_overlap_auto):
    """At the HVP shape the query side runs on its two-workgroups-per-CU kernel with one stream and on
    the pipelined kernel beside the key side with two: the same bits (oracle parity of the one-stream
    call is test_hvp_workload_sampled_heads)."""
    x = I.make_inputs(I.HVP, cotangents=True)
    jvpattn_bwd_set_overlap(False)
    one = gpu_bwd(x, I.HVP)
    jvpattn_bwd_set_overlap(True)
    two = gpu_bwd(x, I.HVP)
    for n in NAMES:
        assert np.array_equal(one[n], two[n]), n


def test_overlap_joins_the_callers_stream(_overlap_auto):
    """Work queued on the caller's stream right after a two-stream call sees every gradient:
    copies taken on a non-default stream with no host synchronisation in between, over
    several calls in a row."""
    w = I.Workload("overlap_join", B=4, H=8, Hkv=2, N=700, d=64, dtype="bf16", causal=True, std=1.0, seed=91)
    x = I.make_inputs(w, cotangents=True)
    d = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], causal=True)
    args = (d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], o, to, lse, tlse, d["do"], d["dto"])
    jvpattn_bwd_set_overlap(False)
    ref = [t.clone() for t in jvpattn_bwd(*args, causal=True)]
    torch.cuda.synchronize()
    jvpattn_bwd_set_overlap(True)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        copies = []
        for _ in range(3):
            g = jvpattn_bwd(*args, causal=True)
            copies.append([t.clone() for t in g])
            for t in g:
                t.fill_(float("nan"))   # the next call must overwrite them after this, in stream order
    torch.cuda.synchronize()
    for c in copies:
        for n, a, b in zip(NAMES, ref, c):
            assert torch.equal(a, b), n


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
    check(I.HVP, heads=HVP_HEADS)


def test_hvp_shape_unit_spread_sampled_heads():
    """The HVP shape at unit input spread (score-tangent and tlse terms well above rounding): two heads."""
    check(HVP_UNIT, heads=HVP_HEADS)


def test_deterministic():
    w = W("det", N=300, causal=True, seed=48)
    a, _ = run(w)
    b, _ = run(w)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


# ------------------------------------------------ d = 128
# Its own kernel instances: the query side one block at a time (no overlap of
# two blocks' products), the key side in two launches (dk, dtk, then dv, dtv).

@pytest.mark.parametrize("std", [None, 1.0, 2.0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_d128(dtype, causal, std):
    check(I.Workload("d128", B=1, H=2, N=200, d=128, dtype=dtype, causal=causal, std=std, seed=61))


@pytest.mark.parametrize("mask_kind", ["bool", "additive"])
@pytest.mark.parametrize("causal", [False, True])
def test_d128_masks(mask_kind, causal):
    check(I.Workload("d128_mask", B=2, H=2, N=170, d=128, dtype="bf16", causal=causal, mask_kind=mask_kind,
                     mask_heads=2 if mask_kind == "additive" else 1, keep=0.7, std=1.0, seed=62))


@pytest.mark.parametrize("N", [1, 33, 129, 257])
def test_d128_ragged_and_grouped(N):
    check(I.Workload("d128_gqa", B=1, H=4, Hkv=2, N=N, Nk=N + 40, d=128, dtype="f16", causal=True, std=1.0,
                     seed=63 + N))


def test_d128_missing_tangents_and_mask_tangent():
    w = I.Workload("d128_iso", B=1, H=2, N=150, d=128, dtype="bf16", std=1.0, seed=64)
    check(w, tangents=("tq",))
    check(w, tangents=("tv",))
    wt = I.Workload("d128_tmask", B=1, H=2, N=150, d=128, dtype="f16", causal=True, mask_kind="additive",
                    mask_heads=2, std=1.0, seed=65)
    g = torch.Generator().manual_seed(66)
    x = I.make_inputs(wt, cotangents=True)
    check(wt, x=x, tmask=torch.randn(x["mask"].shape, generator=g).to(x["mask"].dtype))


# ------------------------------------------------ float32 (d = 64)
# Its own kernels: float32 products throughout, no rounding of the weights or
# score cotangents (bar rho = 1e-4 of each element's term magnitude).

@pytest.mark.parametrize("std", [None, 1.0, 2.0])
@pytest.mark.parametrize("causal", [False, True])
def test_f32(causal, std):
    check(I.Workload("f32", B=1, H=2, N=200, d=64, dtype="f32", causal=causal, std=std, seed=71))


@pytest.mark.parametrize("mask_kind,layout", [("bool", None), ("additive", None), ("bool", "pad_right")])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_masks(mask_kind, layout, causal):
    kw = {"mask_layout": layout} if layout else {"keep": 0.7}
    check(I.Workload("f32_mask", B=2, H=2, N=170, d=64, dtype="f32", causal=causal, mask_kind=mask_kind,
                     mask_heads=2 if mask_kind == "additive" else 1, std=1.0, seed=72, **kw))


@pytest.mark.parametrize("causal", [False, True])
def test_f32_bit_packed_mask(causal):
    from forward_mode_autodiff_amd.jvpattn import pack_mask_bits
    w = I.Workload("f32_bits", B=2, H=2, N=150, d=64, dtype="f32", causal=causal, mask_kind="bool", keep=0.7,
                   std=1.0, seed=73)
    x = I.make_inputs(w, cotangents=True)
    got = gpu_bwd(dict(x, mask=pack_mask_bits(x["mask"])), w, mask_kind="bits")
    bad = bwd_failures(got, reference(x, w), magnitudes(x, w), w.dtype)
    assert not bad, "; ".join(bad)


@pytest.mark.parametrize("N", [1, 33, 129, 257])
def test_f32_ragged_rectangular_grouped(N):
    check(I.Workload("f32_gqa", B=1, H=4, Hkv=2, N=N, Nk=N + 40, d=64, dtype="f32", causal=True, std=1.0,
                     seed=74 + N))


def test_f32_missing_tangents_and_mask_tangent():
    w = I.Workload("f32_iso", B=1, H=2, N=150, d=64, dtype="f32", std=1.0, seed=75)
    check(w, tangents=("tk",))
    check(w, tangents=())
    wt = I.Workload("f32_tmask", B=1, H=2, N=150, d=64, dtype="f32", causal=True, mask_kind="additive",
                    mask_heads=2, std=1.0, seed=76)
    g = torch.Generator().manual_seed(77)
    x = I.make_inputs(wt, cotangents=True)
    check(wt, x=x, tmask=torch.randn(x["mask"].shape, generator=g).to(x["mask"].dtype))


def test_errors_raise():
    x = I.make_inputs(W("err", N=64, dtype="bf16", seed=49), cotangents=True)
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
    got = gpu_bwd(xb, w, mask_kind="bits")
    ref = reference(x, w)
    M = magnitudes(x, w)
    bad = bwd_failures(got, ref, M, w.dtype)
    assert not bad, "; ".join(bad)


@pytest.mark.parametrize("causal,dtype", [(False, "bf16"), (True, "f16")])
def test_mask_tangent(causal, dtype):
    """jvpattn_bwd_tmask: the reverse pass of the forward along (dQ, dK, dV, dM), against the oracle."""
    w = I.Workload("tmask_bwd", B=2, H=2, N=170, d=64, dtype=dtype, causal=causal, mask_kind="additive",
                   std=1.0, seed=25)
    x = I.make_inputs(w, cotangents=True)
    g = torch.Generator().manual_seed(26)
    tm = torch.randn(x["mask"].shape, generator=g).to(x["mask"].dtype)
    check(w, x=x, tmask=tm)
