"""The PyTorch entries on the GPU: attention() in reverse and forward mode, fwd_dual under autograd.

Values must equal the direct library calls bit for bit (the entries only
marshal), and match the float64 oracle to the parity bars.
"""
import pytest
import torch
import torch.autograd.forward_ad as fwAD

from forward_mode_autodiff_amd import inputs as I
from forward_mode_autodiff_amd.autograd import attention, fwd_dual
from forward_mode_autodiff_amd.jvpattn import jvpattn_bwd, jvpattn_fwd
from oracle import oracle_fwd
from tests.bwd_cases import magnitudes, reference
from tests.parity import BWD_NAMES as NAMES, assert_parity, bwd_errors

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def setup(causal, mask_kind="none", seed=61):
    w = I.Workload("ag", B=1, H=2, N=160, d=64, dtype="bf16", causal=causal, std=1.0, seed=seed,
                   mask_kind=mask_kind, keep=0.7)
    x = I.make_inputs(w, cotangents=True)
    d = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    if d["mask"] is not None and mask_kind == "bool":
        d["mask"] = d["mask"].bool()
    return w, x, d


def f64(t):
    return None if t is None else t.double().cpu().numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_attention_reverse_mode(causal):
    w, x, d = setup(causal)
    q, k, v = (d[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = attention(q, k, v, is_causal=causal)
    o.backward(d["do"])
    # the same library call made directly
    o2, to2, lse2, tlse2 = jvpattn_fwd(d["q"], d["k"], d["v"], causal=causal)
    g = jvpattn_bwd(d["q"], d["k"], d["v"], None, None, None, o2, to2, lse2, tlse2, d["do"], None, causal=causal)
    assert torch.equal(o.detach(), o2)
    for t, r in zip((q, k, v), g[:3]):
        assert torch.equal(t.grad, r)
    xz = dict(x, dto=torch.zeros_like(x["dto"]))
    ref, M = reference(xz, w, ()), magnitudes(xz, w, ())
    got = dict(ref, dq=f64(q.grad), dk=f64(k.grad), dv=f64(v.grad))
    for n in ("dq", "dk", "dv"):
        ratio = bwd_errors(got, ref, M, "bf16")[n][0]
        assert ratio <= 1.0, (n, ratio)


def test_attention_forward_mode_dual_tensors():
    w, x, d = setup(False, mask_kind="bool")
    with fwAD.dual_level():
        duals = [fwAD.make_dual(d[p], d[t]) for p, t in (("q", "tq"), ("k", "tk"), ("v", "tv"))]
        out = attention(*duals, attn_mask=d["mask"])
        o, to = fwAD.unpack_dual(out)
    o2, to2, _, _ = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=d["mask"])
    assert torch.equal(o, o2) and torch.equal(to, to2)
    ro, rto, _, _ = oracle_fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["tq"]), f64(x["tk"]), f64(x["tv"]),
                               mask=x["mask"].numpy(), mask_kind="bool")
    assert_parity({"o": o.float().cpu(), "to": to.float().cpu()}, {"o": ro, "to": rto}, "bf16", "dual")


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_dual_reverse_mode_is_the_hvp_route(causal):
    w, x, d = setup(causal, seed=62)
    ins = [d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "tq", "tk", "tv")]
    o, to = fwd_dual(*ins, is_causal=causal)
    grads = torch.autograd.grad((o.float() * d["do"].float()).sum() + (to.float() * d["dto"].float()).sum(), ins)
    o2, to2, lse2, tlse2 = jvpattn_fwd(*[d[n] for n in ("q", "k", "v", "tq", "tk", "tv")], causal=causal)
    direct = jvpattn_bwd(*[d[n] for n in ("q", "k", "v", "tq", "tk", "tv")], o2, to2, lse2, tlse2, d["do"],
                         d["dto"], causal=causal)
    for a, b in zip(grads, direct):
        assert torch.equal(a, b)
    ref, M = reference(x, w), magnitudes(x, w)
    errs = bwd_errors({n: f64(a) for n, a in zip(NAMES, grads)}, ref, M, "bf16")
    for n in NAMES:
        assert errs[n][0] <= 1.0, (n, errs[n])


def test_attention_forward_mode_dual_additive_mask():
    """A dual additive mask: the JVP along (tq, tk, tv, dM) equals jvpattn_fwd_tmask bit for bit."""
    w, x, d = setup(True, mask_kind="additive", seed=63)
    g = torch.Generator().manual_seed(64)
    tm = torch.randn(d["mask"].shape, generator=g).to(d["mask"].dtype).to(DEV)
    with fwAD.dual_level():
        duals = [fwAD.make_dual(d[p], d[t]) for p, t in (("q", "tq"), ("k", "tk"), ("v", "tv"))]
        out = attention(*duals, attn_mask=fwAD.make_dual(d["mask"], tm), is_causal=True)
        o, to = fwAD.unpack_dual(out)
    o2, to2, _, _ = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=d["mask"], causal=True,
                                tmask=tm)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(to, to2)


def test_attention_reverse_mode_grouped_kv_heads():
    """k, v with a quarter of q's heads: gradients equal the direct jvpattn_bwd call bit for bit."""
    w = I.Workload("ag_gqa", B=1, H=4, Hkv=1, N=160, d=64, dtype="bf16", causal=True, std=1.0, seed=65)
    x = I.make_inputs(w, cotangents=True)
    d = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    q, k, v = (d[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    attention(q, k, v, is_causal=True).backward(d["do"])
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], causal=True)
    g = jvpattn_bwd(d["q"], d["k"], d["v"], None, None, None, o, to, lse, tlse, d["do"], None, causal=True)
    torch.cuda.synchronize()
    for t, r in zip((q, k, v), g[:3]):
        assert torch.equal(t.grad, r)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_func_jvp_route(causal):
    """torch.func.jvp around attention(): O and dO equal the direct jvpattn_fwd call bit for bit, and a
    loss of both backpropagates to the direct jvpattn_bwd call's gradients (the HVP route)."""
    w, x, d = setup(causal, seed=66)
    q, k, v = (d[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o, to = torch.func.jvp(lambda a, b, c: attention(a, b, c, is_causal=causal), (q, k, v),
                           (d["tq"], d["tk"], d["tv"]))
    o2, to2, lse2, tlse2 = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], causal=causal)
    assert torch.equal(o.detach(), o2) and torch.equal(to.detach(), to2)
    grads = torch.autograd.grad((o.float() * d["do"].float()).sum() + (to.float() * d["dto"].float()).sum(),
                                (q, k, v))
    ref, M = reference(x, w), magnitudes(x, w)
    errs = bwd_errors(dict(ref, dq=f64(grads[0]), dk=f64(grads[1]), dv=f64(grads[2])), ref, M, "bf16")
    for n in ("dq", "dk", "dv"):
        assert errs[n][0] <= 1.0, (n, errs[n])


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "f32")])
def test_attention_reverse_mode_other_dims_and_float32(d, dtype):
    """attention() backward at d = 128 and in float32 equals the direct jvpattn_bwd call."""
    w = I.Workload("ag_dims", B=1, H=2, N=150, d=d, dtype=dtype, causal=True, std=1.0, seed=67)
    x = I.make_inputs(w, cotangents=True)
    dd = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    q, k, v = (dd[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    attention(q, k, v, is_causal=True).backward(dd["do"])
    o, to, lse, tlse = jvpattn_fwd(dd["q"], dd["k"], dd["v"], causal=True)
    g = jvpattn_bwd(dd["q"], dd["k"], dd["v"], None, None, None, o, to, lse, tlse, dd["do"], None, causal=True)
    torch.cuda.synchronize()
    for t, r in zip((q, k, v), g[:3]):
        assert torch.equal(t.grad, r)


@pytest.mark.parametrize("d", [96, 256])
def test_torch_func_jvp_other_dims(d):
    """torch.func.jvp around attention() at d = 96 / 256 equals the direct forward."""
    w = I.Workload("ag_jvp_dims", B=1, H=2, N=150, d=d, dtype="bf16", std=1.0, seed=68)
    x = I.make_inputs(w)
    dd = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    o, to = torch.func.jvp(lambda a, b, c: attention(a, b, c), (dd["q"], dd["k"], dd["v"]),
                           (dd["tq"], dd["tk"], dd["tv"]))
    o2, to2, _, _ = jvpattn_fwd(dd["q"], dd["k"], dd["v"], dd["tq"], dd["tk"], dd["tv"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(to, to2)
