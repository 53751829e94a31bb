"""Pins for the float64 backward oracle (reverse-mode derivative of (O, dO)).

Each checks ``oracle_bwd`` against something other than itself:
* PyTorch autograd taken reverse-over-forward through its own
  scaled_dot_product_attention (MATH backend, CPU, float64): torch.func.jvp
  gives (O, dO), torch.autograd.grad pulls (gO, gdO) back to all six inputs;
* central finite differences of L = <gO, O> + <gdO, dO>, with (O, dO) from the
  pinned forward oracle, along random directions of all six inputs at once;
* closed forms: with dQ = dK = 0 and gdO = 0 the result is the plain
  attention backward; gradients with respect to dV are P^T gdO (linear in
  gdO, independent of the tangents); rows with no visible key contribute
  nothing; the additive-mask row shift leaves every gradient unchanged;
* mutants: plausible mistakes planted in a copy of the oracle fail these pins.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention import SDPBackend, sdpa_kernel

import oracle.attention_bwd as ob
from oracle import oracle_bwd, oracle_fwd


def make(rng, B=2, H=2, Nq=7, Nk=9, d=5, std=1.0, Hkv=None):
    r = lambda *s, sd=1.0: rng.standard_normal(s) * sd
    Hk = H if Hkv is None else Hkv
    return dict(q=r(B, H, Nq, d, sd=std), k=r(B, Hk, Nk, d, sd=std), v=r(B, Hk, Nk, d, sd=std),
                tq=r(B, H, Nq, d), tk=r(B, Hk, Nk, d), tv=r(B, Hk, Nk, d),
                go=r(B, H, Nq, d), gto=r(B, H, Nq, d))


def torch_reverse_over_forward(x, attn_mask=None, is_causal=False, scale=None):
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).requires_grad_(True)
    ins = [T(x[n]) for n in ("q", "k", "v", "tq", "tk", "tv")]
    m = None if attn_mask is None else torch.from_numpy(np.ascontiguousarray(attn_mask))
    gqa = x["k"].shape[1] != x["q"].shape[1]
    with sdpa_kernel(SDPBackend.MATH):
        o, to = torch.func.jvp(
            lambda a, b, c: F.scaled_dot_product_attention(a, b, c, attn_mask=m, is_causal=is_causal, scale=scale,
                                                           enable_gqa=gqa),
            tuple(ins[:3]), tuple(ins[3:]))
        L = (o * torch.from_numpy(x["go"])).sum() + (to * torch.from_numpy(x["gto"])).sum()
        g = torch.autograd.grad(L, ins)
    return [t.numpy() for t in g]


def run_bwd(x, **kw):
    return oracle_bwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], x["go"], x["gto"], **kw)


NAMES = ("gq", "gk", "gv", "gtq", "gtk", "gtv")


def assert_close(got, ref, atol):
    for n, a, b in zip(NAMES, got, ref):
        np.testing.assert_allclose(a, b, rtol=0, atol=atol, err_msg=n)


@pytest.mark.parametrize("Nq,Nk,d", [(7, 9, 5), (1, 1, 3), (16, 16, 8), (5, 33, 4)])
def test_matches_torch_autograd_no_mask(Nq, Nk, d):
    x = make(np.random.default_rng(30 + Nq), Nq=Nq, Nk=Nk, d=d)
    assert_close(run_bwd(x), torch_reverse_over_forward(x), 1e-11)


def test_matches_torch_autograd_bool_mask():
    rng = np.random.default_rng(31)
    x = make(rng, Nq=6, Nk=8, d=4)
    mask = rng.random((2, 1, 6, 8)) < 0.6
    mask[..., 0] = True
    assert_close(run_bwd(x, mask=mask.astype(np.uint8), mask_kind="bool"),
                 torch_reverse_over_forward(x, attn_mask=mask), 1e-11)


def test_matches_torch_autograd_additive_mask_per_head():
    rng = np.random.default_rng(32)
    x = make(rng, Nq=6, Nk=8, d=4)
    add = rng.standard_normal((2, 2, 6, 8))
    assert_close(run_bwd(x, mask=add, mask_kind="additive"), torch_reverse_over_forward(x, attn_mask=add), 1e-11)


def test_matches_torch_autograd_causal_and_scale():
    x = make(np.random.default_rng(33), Nq=9, Nk=9, d=6)
    assert_close(run_bwd(x, causal=True, scale=0.37), torch_reverse_over_forward(x, is_causal=True, scale=0.37),
                 1e-11)


def test_matches_torch_autograd_causal_rectangular():
    # SDPA's is_causal is top-left aligned (tril of ones(Nq, Nk)), like ours
    x = make(np.random.default_rng(34), Nq=5, Nk=11, d=4)
    assert_close(run_bwd(x, causal=True), torch_reverse_over_forward(x, is_causal=True), 1e-11)


@pytest.mark.parametrize("H,Hkv,causal", [(4, 2, False), (6, 2, True), (3, 1, False)],
                         ids=["gqa2", "gqa3-causal", "mqa"])
def test_matches_torch_autograd_grouped_heads(H, Hkv, causal):
    # a key/value head read by several query heads collects all their cotangents
    x = make(np.random.default_rng(37 + H), H=H, Hkv=Hkv, Nq=6, Nk=8, d=4)
    assert_close(run_bwd(x, causal=causal), torch_reverse_over_forward(x, is_causal=causal), 1e-11)


def loss(x, **kw):
    o, to, _, _ = oracle_fwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], **kw)
    return float(np.sum(o * x["go"]) + np.sum(to * x["gto"]))


@pytest.mark.parametrize("kw,hkv", [({}, 2), ({"causal": True}, 2), ({"scale": 1.7}, 2), ({}, 1)],
                         ids=["plain", "causal", "scale", "grouped"])
def test_directional_finite_differences(kw, hkv):
    rng = np.random.default_rng(35)
    x = make(rng, B=1, H=2, Nq=6, Nk=7, d=4, Hkv=hkv)
    g = run_bwd(x, **kw)
    for trial in range(3):
        dirs = {n: rng.standard_normal(x[n].shape) for n in ("q", "k", "v", "tq", "tk", "tv")}
        eps = 1e-5
        xp = dict(x, **{n: x[n] + eps * dirs[n] for n in dirs})
        xm = dict(x, **{n: x[n] - eps * dirs[n] for n in dirs})
        fd = (loss(xp, **kw) - loss(xm, **kw)) / (2 * eps)
        an = sum(float(np.sum(gi * dirs[n])) for gi, n in zip(g, ("q", "k", "v", "tq", "tk", "tv")))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (trial, fd, an)


def test_plain_attention_backward_when_tangents_and_gdo_vanish():
    rng = np.random.default_rng(36)
    x = make(rng, Nq=6, Nk=8, d=4)
    x["tq"][:] = 0
    x["tk"][:] = 0
    x["gto"][:] = 0
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).requires_grad_(True)
    q, k, v = T(x["q"]), T(x["k"]), T(x["v"])
    with sdpa_kernel(SDPBackend.MATH):
        o = F.scaled_dot_product_attention(q, k, v)
    gq, gk, gv = torch.autograd.grad((o * torch.from_numpy(x["go"])).sum(), [q, k, v])
    g = run_bwd(x)
    for a, b in zip(g[:3], (gq, gk, gv)):
        np.testing.assert_allclose(a, b.numpy(), rtol=0, atol=1e-12)
    # no gradient reaches dV without gdO
    np.testing.assert_array_equal(g[5], 0.0)


def test_gradient_of_dv_is_weights_transposed_times_gdo():
    rng = np.random.default_rng(37)
    x = make(rng, B=1, H=1, Nq=5, Nk=6, d=3)
    s = 1 / math.sqrt(3)
    S = s * x["q"][0, 0] @ x["k"][0, 0].T
    P = np.exp(S - S.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    g = run_bwd(x)
    np.testing.assert_allclose(g[5][0, 0], P.T @ x["gto"][0, 0], rtol=0, atol=1e-13)
    # ... and does not depend on the tangents
    y = dict(x, tq=x["tq"] * 3, tk=-x["tk"], tv=x["tv"] + 1)
    np.testing.assert_allclose(run_bwd(y)[5], g[5], rtol=0, atol=1e-13)


def test_rows_without_visible_keys_contribute_nothing():
    rng = np.random.default_rng(38)
    x = make(rng, B=1, H=1, Nq=4, Nk=5, d=3)
    mask = np.ones((1, 1, 4, 5), dtype=np.uint8)
    mask[0, 0, 2, :] = 0
    g = run_bwd(x, mask=mask, mask_kind="bool")
    np.testing.assert_array_equal(g[0][0, 0, 2], 0.0)
    np.testing.assert_array_equal(g[3][0, 0, 2], 0.0)
    # removing that row's cotangents changes nothing
    y = dict(x, go=x["go"].copy(), gto=x["gto"].copy())
    y["go"][0, 0, 2] = 7.0
    y["gto"][0, 0, 2] = -3.0
    for a, b in zip(run_bwd(y, mask=mask, mask_kind="bool"), g):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_additive_row_shift_leaves_gradients_unchanged():
    rng = np.random.default_rng(39)
    x = make(rng, B=1, H=1, Nq=4, Nk=6, d=3)
    add = rng.standard_normal((1, 1, 4, 6))
    shifted = add + rng.standard_normal((1, 1, 4, 1)) * 5
    for a, b in zip(run_bwd(x, mask=add, mask_kind="additive"), run_bwd(x, mask=shifted, mask_kind="additive")):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


# ---------------------------------------------------------------- mutants

def _mutant(src_old, src_new):
    """A copy of oracle_bwd_head with one line changed (the true module is untouched)."""
    import inspect
    src = inspect.getsource(ob.oracle_bwd_head)
    assert src_old in src, src_old
    ns = dict(ob.__dict__)
    exec(compile(src.replace(src_old, src_new), "<mutant>", "exec"), ns)
    return ns["oracle_bwd_head"]


MUTANTS = {
    "drop_t_cotangent": ("g_t = -np.sum(g_dP * P, axis=1, keepdims=True)", "g_t = 0.0 * g_dP[:, :1]"),
    "sign_softmax_rowsum": ("g_P - np.sum(g_P * P, axis=1, keepdims=True)", "g_P + np.sum(g_P * P, axis=1, keepdims=True)"),
    "drop_dP_in_gv": ("g_v = dP.T @ gto", "g_v = 0.0 * (dP.T @ gto)"),
    "swap_tangent_grads": ("g_tq = scale * (g_dS @ k)", "g_tq = scale * (g_dS @ tk)"),
    "unscaled_tangent_path": ("g_tk = scale * (g_dS.T @ q)", "g_tk = g_dS.T @ q"),
    "drop_dS_in_gP": ("g_P = g_P + g_dP * (dS - t)", "g_P = g_P + g_dP * dS"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_fail_the_autograd_pin(name, monkeypatch):
    x = make(np.random.default_rng(40), Nq=6, Nk=7, d=4)
    ref = torch_reverse_over_forward(x, is_causal=True)
    monkeypatch.setattr(ob, "oracle_bwd_head", _mutant(*MUTANTS[name]))
    got = ob.oracle_bwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], x["go"], x["gto"], causal=True)
    worst = max(float(np.max(np.abs(a - b))) for a, b in zip(got, ref))
    assert worst > 1e-3, f"mutant {name} passes the pin (max diff {worst:.2e})"


def test_grouped_head_mutants_fail_the_autograd_pin(monkeypatch):
    # two plausible grouping mistakes: interleaved instead of blocked head
    # sharing, and keeping only the last query head's cotangent
    x = make(np.random.default_rng(41), H=4, Hkv=2, Nq=6, Nk=7, d=4)
    ref = torch_reverse_over_forward(x)
    run = lambda: ob.oracle_bwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], x["go"], x["gto"])
    with monkeypatch.context() as m:
        m.setattr(ob, "kv_head", lambda h, H, Hkv: h % Hkv)
        assert max(float(np.max(np.abs(a - b))) for a, b in zip(run(), ref)) > 1e-3
    import inspect
    src = inspect.getsource(ob.oracle_bwd).replace("gk[b, g] += r[1]", "gk[b, g] = r[1]")
    ns = dict(ob.__dict__)
    exec(compile(src, "<mutant>", "exec"), ns)
    got = ns["oracle_bwd"](x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], x["go"], x["gto"])
    assert float(np.max(np.abs(got[1] - ref[1]))) > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_with_mask_tangent(causal):
    # reverse mode over the forward-mode pass along (dQ, dK, dV, dM): torch.func.jvp through SDPA with the
    # additive mask as a differentiated input, then autograd back to the six tensors
    rng = np.random.default_rng(42)
    x = make(rng, Nq=6, Nk=8, d=4)
    m = rng.standard_normal((2, 1, 6, 8))
    m[1, ..., 5:] = -np.inf
    tm = rng.standard_normal((2, 1, 6, 8))
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).requires_grad_(True)
    ins = [T(x[n]) for n in ("q", "k", "v", "tq", "tk", "tv")]
    # SDPA takes no explicit mask with is_causal: fold the causal cut into its mask (j <= i visible)
    cut = np.where(np.arange(8)[None, :] <= np.arange(6)[:, None], 0.0, -np.inf) if causal else 0.0
    mm, tt = torch.from_numpy(m + cut), torch.from_numpy(tm)
    with sdpa_kernel(SDPBackend.MATH):
        o, to = torch.func.jvp(
            lambda a, b, c, mk: F.scaled_dot_product_attention(a, b, c, attn_mask=mk),
            (ins[0], ins[1], ins[2], mm), (ins[3], ins[4], ins[5], tt))
        L = (o * torch.from_numpy(x["go"])).sum() + (to * torch.from_numpy(x["gto"])).sum()
        ref = [t.numpy() for t in torch.autograd.grad(L, ins)]
    got = run_bwd(x, mask=m, mask_kind="additive", causal=causal, tmask=tm)
    assert_close(got, ref, 1e-11)
