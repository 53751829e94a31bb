"""The PyTorch integration routes every derivative to the right library call (CPU, no GPU).

``forward_mode_autodiff_amd.autograd`` only marshals: these tests swap the two
library entry points for the float64 oracle and check that reverse mode,
forward mode (forward_ad dual tensors, and torch.func.jvp around a function
that calls attention()), reverse mode over the dual pair and reverse mode
through torch.func.jvp return what the oracle says, in the right places.
"""
import numpy as np
import pytest
import torch
import torch.autograd.forward_ad as fwAD

import forward_mode_autodiff_amd.autograd as A
from forward_mode_autodiff_amd import jvpattn as J
from oracle import oracle_bwd, oracle_fwd


def _np(t):
    return None if t is None else t.detach().double().numpy()


def fake_fwd(q, k, v, tq=None, tk=None, tv=None, mask=None, causal=False, scale=None, want_tlse=True, out=None,
             tmask=None):
    kind = "none" if mask is None else ("bool" if mask.dtype == torch.bool else "additive")
    m = None if mask is None else (mask.numpy().astype(np.uint8) if kind == "bool" else _np(mask))
    o, to, lse, tlse = oracle_fwd(_np(q), _np(k), _np(v), _np(tq), _np(tk), _np(tv), mask=m, mask_kind=kind,
                                  causal=causal, scale=scale, tmask=_np(tmask))
    T = lambda a: torch.from_numpy(a).to(q.dtype)
    return T(o), T(to), torch.from_numpy(lse).float(), torch.from_numpy(tlse).float()


def fake_bwd(q, k, v, tq, tk, tv, o, to, lse, tlse, go, gto, mask=None, causal=False, scale=None, out=None,
             workspace=None, tmask=None):
    kind = "none" if mask is None else ("bool" if mask.dtype == torch.bool else "additive")
    m = None if mask is None else (mask.numpy().astype(np.uint8) if kind == "bool" else _np(mask))
    z = lambda t: np.zeros(q.shape) if t is None else _np(t)
    g = oracle_bwd(_np(q), _np(k), _np(v), _np(tq), _np(tk), _np(tv), z(go), z(gto), mask=m, mask_kind=kind,
                   causal=causal, scale=scale, tmask=_np(tmask))
    res = [torch.from_numpy(a).to(q.dtype) for a in g]
    if out is not None:
        res = [None if slot is None else r for r, slot in zip(res, out)]
    return tuple(res)


@pytest.fixture(autouse=True)
def fake_library(monkeypatch):
    monkeypatch.setattr(J, "jvpattn_fwd", fake_fwd)
    monkeypatch.setattr(J, "jvpattn_bwd", fake_bwd)


def inputs(seed=0, B=1, H=2, N=7, d=4):
    g = torch.Generator().manual_seed(seed)
    r = lambda: torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
    return [r() for _ in range(8)]   # q, k, v, tq, tk, tv, go, gto


@pytest.mark.parametrize("causal", [False, True])
def test_reverse_mode_of_attention(causal):
    q, k, v, tq, tk, tv, go, _ = inputs(1)
    q, k, v = (t.requires_grad_(True) for t in (q, k, v))
    o = A.attention(q, k, v, is_causal=causal)
    o.backward(go)
    ref = oracle_bwd(_np(q), _np(k), _np(v), None, None, None, _np(go), np.zeros(q.shape), causal=causal)
    for t, r in zip((q, k, v), ref[:3]):
        np.testing.assert_allclose(t.grad.numpy(), r, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o.detach().numpy(), oracle_fwd(_np(q), _np(k), _np(v), causal=causal)[0], atol=1e-12)


def test_forward_mode_dual_tensors():
    q, k, v, tq, tk, tv, _, _ = inputs(2)
    mask = torch.rand(1, 1, 7, 7, generator=torch.Generator().manual_seed(3)) < 0.7
    mask[..., 0] = True
    ro, rto, _, _ = oracle_fwd(_np(q), _np(k), _np(v), _np(tq), _np(tk), _np(tv), mask=mask.numpy().astype(np.uint8),
                               mask_kind="bool")
    with fwAD.dual_level():
        duals = [fwAD.make_dual(p, t) for p, t in ((q, tq), (k, tk), (v, tv))]
        out = A.attention(*duals, attn_mask=mask)
        p, t = fwAD.unpack_dual(out)
    np.testing.assert_allclose(p.numpy(), ro, atol=1e-12)
    np.testing.assert_allclose(t.numpy(), rto, atol=1e-12)


def test_reverse_mode_over_the_dual_pair():
    q, k, v, tq, tk, tv, go, gto = inputs(4)
    ins = [t.requires_grad_(True) for t in (q, k, v, tq, tk, tv)]
    o, to = A.fwd_dual(*ins, is_causal=True, scale=0.7)
    grads = torch.autograd.grad((o * go).sum() + (to * gto).sum(), ins)
    ref = oracle_bwd(*[_np(t) for t in ins], _np(go), _np(gto), causal=True, scale=0.7)
    for g, r in zip(grads, ref):
        np.testing.assert_allclose(g.numpy(), r, rtol=0, atol=1e-12)


def test_hessian_vector_product_matches_finite_differences():
    """d/de grad_q f(q + e u) for f = <c, attention(q, k, v)> equals reverse mode over fwd_dual along u."""
    q, k, v, u, _, _, c, _ = inputs(5)
    qq = q.clone().requires_grad_(True)
    o, to = A.fwd_dual(qq, k, v, u, None, None)
    # grad_q <c, dO> with dO = J u is the HVP of f along u
    hvp, = torch.autograd.grad((to * c).sum(), [qq])

    def grad_f(x):
        return torch.from_numpy(oracle_bwd(_np(x), _np(k), _np(v), None, None, None, _np(c), np.zeros(x.shape))[0])
    eps = 1e-6
    fd = (grad_f(q + eps * u) - grad_f(q - eps * u)) / (2 * eps)
    np.testing.assert_allclose(hvp.numpy(), fd.numpy(), rtol=0, atol=1e-7)


def test_forward_mode_with_a_dual_additive_mask():
    # the mask's tangent reaches the library call: the JVP along (tq, tk, tv, tm)
    q, k, v, tq, tk, tv, _, _ = inputs(5)
    g = torch.Generator().manual_seed(9)
    m = torch.randn(1, 1, 7, 7, generator=g, dtype=torch.float64)
    tm = torch.randn(1, 1, 7, 7, generator=g, dtype=torch.float64)
    with fwAD.dual_level():
        duals = [fwAD.make_dual(a, t) for a, t in ((q, tq), (k, tk), (v, tv), (m, tm))]
        o, to = fwAD.unpack_dual(A.attention(*duals[:3], attn_mask=duals[3]))
    ro, rto, _, _ = oracle_fwd(_np(q), _np(k), _np(v), _np(tq), _np(tk), _np(tv), mask=_np(m),
                               mask_kind="additive", tmask=_np(tm))
    np.testing.assert_allclose(_np(o), ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(_np(to), rto, rtol=0, atol=1e-12)
    # fwd_dual takes the same tangent directly, and reverse mode through it carries the tangent along
    q.requires_grad_(True)
    tq.requires_grad_(True)
    o2, to2 = A.fwd_dual(q, k, v, tq, tk, tv, attn_mask=m, tmask=tm)
    np.testing.assert_allclose(_np(to2), rto, rtol=0, atol=1e-12)
    gto = torch.ones_like(to2)
    to2.backward(gto)
    ref = oracle_bwd(_np(q), _np(k), _np(v), _np(tq), _np(tk), _np(tv), np.zeros(q.shape), _np(gto), mask=_np(m),
                     mask_kind="additive", tmask=_np(tm))
    np.testing.assert_allclose(_np(q.grad), ref[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(_np(tq.grad), ref[3], rtol=0, atol=1e-12)


def test_grouped_kv_heads_route_through():
    # k, v with fewer heads than q: the library calls receive them as they are
    g = torch.Generator().manual_seed(11)
    r = lambda h: torch.randn(1, h, 6, 4, generator=g, dtype=torch.float64)
    q, k, v, go = r(4), r(2), r(2), r(4)
    q.requires_grad_(True), k.requires_grad_(True), v.requires_grad_(True)
    A.attention(q, k, v).backward(go)
    ref = oracle_bwd(_np(q), _np(k), _np(v), None, None, None, _np(go), np.zeros(q.shape))
    for t, rr in zip((q, k, v), ref[:3]):
        np.testing.assert_allclose(_np(t.grad), rr, rtol=0, atol=1e-12)


# ------------------------------------------------ torch.func.jvp (the README's route)

@pytest.mark.parametrize("causal", [False, True])
def test_torch_func_jvp_gives_the_oracle_jvp(causal):
    q, k, v, tq, tk, tv, _, _ = inputs(11)
    o, to = torch.func.jvp(lambda a, b, c: A.attention(a, b, c, is_causal=causal), (q, k, v), (tq, tk, tv))
    ro, rto, _, _ = oracle_fwd(_np(q), _np(k), _np(v), _np(tq), _np(tk), _np(tv), causal=causal)
    np.testing.assert_allclose(o.numpy(), ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(to.numpy(), rto, rtol=0, atol=1e-12)


def test_torch_func_jvp_with_closed_over_keys_and_an_additive_mask():
    """Tangent along q only (k, v closed over: their tangents are zero); the mask is a constant."""
    q, k, v, tq, _, _, _, _ = inputs(12)
    mask = torch.randn(1, 1, 7, 7, generator=torch.Generator().manual_seed(13), dtype=torch.float64)
    o, to = torch.func.jvp(lambda a: A.attention(a, k, v, attn_mask=mask), (q,), (tq,))
    ro, rto, _, _ = oracle_fwd(_np(q), _np(k), _np(v), _np(tq), None, None, mask=_np(mask), mask_kind="additive")
    np.testing.assert_allclose(o.numpy(), ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(to.numpy(), rto, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_reverse_mode_through_torch_func_jvp(causal):
    """A loss of (O, dO) from torch.func.jvp, backpropagated to q, k, v: the oracle's reverse pass."""
    q, k, v, tq, tk, tv, go, gto = inputs(14)
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    o, to = torch.func.jvp(lambda a, b, c: A.attention(a, b, c, is_causal=causal), (qq, kk, vv), (tq, tk, tv))
    g = torch.autograd.grad((o * go).sum() + (to * gto).sum(), (qq, kk, vv))
    ref = oracle_bwd(_np(q), _np(k), _np(v), _np(tq), _np(tk), _np(tv), _np(go), _np(gto), causal=causal)
    for a, r in zip(g, ref[:3]):
        np.testing.assert_allclose(a.numpy(), r, rtol=0, atol=1e-12)


def test_other_torch_func_transforms_raise():
    q, k, v, *_ = inputs(15)
    with pytest.raises(Exception, match="vmap"):
        torch.func.vmap(lambda a: A.attention(a[None], k, v))(q[0])
