"""Pins for the float64 oracle: each checks it against something other than itself.

* the primal against PyTorch's own scaled_dot_product_attention (MATH backend,
  CPU, float64) -- the call the README's "Usage" section says the method
  replaces;
* the tangent against PyTorch forward-mode AD (torch.func.jvp) through that
  call, against central finite differences, and against a dual-number
  evaluation of the naive per-element definition;
* closed forms: two keys (logistic), one key, zero queries, zero tangents,
  a tangent of V equal to V, tangents that shift every score of a row equally;
* masks by brute force: a boolean mask equals attention over only the kept
  keys; causal equals a lower-triangular boolean mask; an additive {0, -inf}
  mask equals the boolean one; adding c_i to a row of an additive mask shifts
  lse by c_i and leaves O and dO unchanged;
* lse against scipy's logsumexp, tlse against finite differences of lse.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F
from torch.nn.attention import SDPBackend, sdpa_kernel

from oracle import oracle_fwd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def make(rng, B=2, H=3, Nq=7, Nk=9, d=5, std=1.0):
    q = rnd(rng, B, H, Nq, d, std=std)
    k = rnd(rng, B, H, Nk, d, std=std)
    v = rnd(rng, B, H, Nk, d, std=std)
    tq = rnd(rng, B, H, Nq, d)
    tk = rnd(rng, B, H, Nk, d)
    tv = rnd(rng, B, H, Nk, d)
    return q, k, v, tq, tk, tv


def torch_sdpa_jvp(q, k, v, tq, tk, tv, attn_mask=None, is_causal=False, scale=None, enable_gqa=False):
    """PyTorch's SDPA (MATH backend, float64 CPU) and its forward-mode derivative."""
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    m = None if attn_mask is None else T(attn_mask)
    with sdpa_kernel(SDPBackend.MATH):
        o, to = torch.func.jvp(
            lambda a, b, c: F.scaled_dot_product_attention(a, b, c, attn_mask=m, is_causal=is_causal,
                                                           scale=scale, enable_gqa=enable_gqa),
            (T(q), T(k), T(v)), (T(tq), T(tk), T(tv)))
    return o.numpy(), to.numpy()


# ---------------------------------------------------------------- library pins

@pytest.mark.parametrize("Nq,Nk,d", [(7, 9, 5), (1, 1, 3), (16, 16, 8), (5, 33, 4)])
def test_matches_torch_sdpa_no_mask(Nq, Nk, d):
    rng = np.random.default_rng(10 + Nq)
    args = make(rng, Nq=Nq, Nk=Nk, d=d)
    o, to, _, _ = oracle_fwd(*args)
    ro, rto = torch_sdpa_jvp(*args)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(to, rto, rtol=0, atol=1e-11)


def test_matches_torch_sdpa_bool_mask():
    rng = np.random.default_rng(1)
    args = make(rng, Nq=6, Nk=8, d=4)
    mask = rng.random((2, 1, 6, 8)) < 0.6
    mask[..., 0] = True          # torch gives NaN on fully masked rows; keep one key per row
    o, to, _, _ = oracle_fwd(*args, mask=mask.astype(np.uint8), mask_kind="bool")
    ro, rto = torch_sdpa_jvp(*args, attn_mask=mask)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(to, rto, rtol=0, atol=1e-11)


@pytest.mark.parametrize("kind", ["bool", "additive"])
def test_matches_torch_sdpa_key_padding_mask(kind):
    # a [B, 1, 1, Nk] mask broadcasts over heads and query rows (SDPA broadcasting)
    rng = np.random.default_rng(45)
    args = make(rng, Nq=6, Nk=10)
    keep = np.ones((2, 1, 1, 10), dtype=bool)
    keep[0, ..., 7:] = False     # right padding
    keep[1, ..., :3] = False     # left padding
    if kind == "bool":
        m, mk = keep, keep.astype(np.uint8)
    else:
        m = np.where(keep, rng.standard_normal(keep.shape), -np.inf)
        mk = m
    o, to, _, _ = oracle_fwd(*args, mask=mk, mask_kind=kind)
    ro, rto = torch_sdpa_jvp(*args, attn_mask=m)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(to, rto, rtol=0, atol=1e-11)


def torch_sdpa_jvp_with_mask(q, k, v, m, tq, tk, tv, tm, is_causal=False):
    """SDPA (MATH, float64) and its JVP with the additive mask as a differentiated input."""
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    with sdpa_kernel(SDPBackend.MATH):
        o, to = torch.func.jvp(
            lambda a, b, c, mm: F.scaled_dot_product_attention(a, b, c, attn_mask=mm, is_causal=is_causal),
            (T(q), T(k), T(v), T(m)), (T(tq), T(tk), T(tv), T(tm)))
    return o.numpy(), to.numpy()


@pytest.mark.parametrize("layout", ["full", "key_padding"])
def test_additive_mask_tangent_matches_torch_jvp(layout):
    # the additive mask as a fourth differentiated input: dS gains its tangent dM
    rng = np.random.default_rng(46)
    q, k, v, tq, tk, tv = make(rng, Nq=6, Nk=9)
    shape = (2, 3, 6, 9) if layout == "full" else (2, 1, 1, 9)
    m = rnd(rng, *shape)
    if layout == "key_padding":
        m[0, ..., 6:] = -np.inf
    tm = rnd(rng, *shape)
    o, to, _, tlse = oracle_fwd(q, k, v, tq, tk, tv, mask=m, mask_kind="additive", tmask=tm)
    ro, rto = torch_sdpa_jvp_with_mask(q, k, v, m, tq, tk, tv, tm)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(to, rto, rtol=0, atol=1e-11)
    # tlse is still the derivative of lse, now along the mask too (central differences)
    eps = 1e-6
    lp = oracle_fwd(q + eps * tq, k + eps * tk, v, mask=m + eps * tm, mask_kind="additive")[2]
    lm = oracle_fwd(q - eps * tq, k - eps * tk, v, mask=m - eps * tm, mask_kind="additive")[2]
    fin = np.isfinite(lp)
    np.testing.assert_allclose(tlse[fin], ((lp - lm) / (2 * eps))[fin], rtol=0, atol=1e-7)


def test_additive_mask_tangent_row_constant_changes_nothing_but_tlse():
    # a tangent constant along each row shifts dS uniformly: dO unchanged, tlse shifted by it
    rng = np.random.default_rng(47)
    args = make(rng, Nq=5, Nk=7)
    m = rnd(rng, 2, 1, 5, 7)
    c = rnd(rng, 2, 1, 5, 1)
    tm = np.broadcast_to(c, m.shape).copy()
    base = oracle_fwd(*args, mask=m, mask_kind="additive")
    got = oracle_fwd(*args, mask=m, mask_kind="additive", tmask=tm)
    np.testing.assert_allclose(got[1], base[1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[3], base[3] + c[..., 0], rtol=0, atol=1e-12)


def test_additive_mask_tangent_needs_additive_mask():
    rng = np.random.default_rng(48)
    args = make(rng)
    with pytest.raises(ValueError):
        oracle_fwd(*args, tmask=np.zeros((2, 1, 7, 9)))


def test_bit_packed_mask_unpacks_as_numpy_unpackbits():
    # bit j % 32 of 32-bit word j // 32: numpy's little-endian unpackbits of the words' bytes
    rng = np.random.default_rng(49)
    words = rng.integers(0, 2 ** 32, size=(3, 5), dtype=np.uint64).astype(np.uint32)
    from oracle.attention import unpack_mask_bits
    ref = np.unpackbits(words.astype("<u4").view(np.uint8), axis=-1, bitorder="little").astype(bool)
    np.testing.assert_array_equal(unpack_mask_bits(words, 150), ref[:, :150])


def test_bit_packed_mask_equals_bool_mask():
    rng = np.random.default_rng(50)
    args = make(rng, Nq=6, Nk=40)
    keep = rng.random((2, 3, 6, 40)) < 0.6
    keep[..., 0] = True
    padded = np.zeros((2, 3, 6, 64), dtype=bool)
    padded[..., :40] = keep
    words = np.packbits(padded, axis=-1, bitorder="little").view("<u4")
    a = oracle_fwd(*args, mask=keep.astype(np.uint8), mask_kind="bool")
    b = oracle_fwd(*args, mask=words, mask_kind="bits")
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_matches_torch_sdpa_additive_mask_per_head():
    rng = np.random.default_rng(2)
    args = make(rng, Nq=6, Nk=8, d=4)
    mask = rng.standard_normal((2, 3, 6, 8)) * 2.0
    o, to, _, _ = oracle_fwd(*args, mask=mask, mask_kind="additive")
    ro, rto = torch_sdpa_jvp(*args, attn_mask=mask)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(to, rto, rtol=0, atol=1e-11)


@pytest.mark.parametrize("N", [1, 5, 12])
def test_matches_torch_sdpa_causal(N):
    rng = np.random.default_rng(3 + N)
    args = make(rng, Nq=N, Nk=N, d=4)
    o, to, _, _ = oracle_fwd(*args, causal=True)
    ro, rto = torch_sdpa_jvp(*args, is_causal=True)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(to, rto, rtol=0, atol=1e-11)


def test_matches_torch_sdpa_custom_scale():
    rng = np.random.default_rng(4)
    args = make(rng, Nq=5, Nk=6, d=3)
    o, to, _, _ = oracle_fwd(*args, scale=0.37)
    ro, rto = torch_sdpa_jvp(*args, scale=0.37)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(to, rto, rtol=0, atol=1e-11)


@pytest.mark.parametrize("H,Hkv,causal", [(4, 2, False), (6, 3, True), (4, 1, False)],
                         ids=["gqa2", "gqa3-causal", "mqa"])
def test_matches_torch_sdpa_grouped_heads(H, Hkv, causal):
    # grouped-query attention: SDPA's enable_gqa shares key/value head h // (H // Hkv)
    rng = np.random.default_rng(40 + H + Hkv)
    q, _, _, tq, _, _ = make(rng, H=H, Nq=7, Nk=9, d=5)
    k, v, tk, tv = (rnd(rng, 2, Hkv, 9, 5) for _ in range(4))
    o, to, _, _ = oracle_fwd(q, k, v, tq, tk, tv, causal=causal)
    ro, rto = torch_sdpa_jvp(q, k, v, tq, tk, tv, is_causal=causal, enable_gqa=True)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(to, rto, rtol=0, atol=1e-11)


def test_grouped_heads_reject_non_divisor():
    rng = np.random.default_rng(44)
    q, _, _, tq, _, _ = make(rng, H=3)
    k = rnd(rng, 2, 2, 9, 5)
    with pytest.raises(ValueError):
        oracle_fwd(q, k, k, tq, k, k)


def test_lse_matches_scipy_logsumexp():
    rng = np.random.default_rng(5)
    q, k, v, tq, tk, tv = make(rng, Nq=6, Nk=10, d=4, std=2.0)
    mask = rng.standard_normal((2, 1, 6, 10))
    _, _, lse, _ = oracle_fwd(q, k, v, tq, tk, tv, mask=mask, mask_kind="additive", scale=0.5)
    S = 0.5 * np.einsum("bhid,bhjd->bhij", q, k) + mask
    np.testing.assert_allclose(lse, scipy.special.logsumexp(S, axis=-1), rtol=0, atol=1e-12)


# ----------------------------------------------------------- derivative pins

def _perturbed(args, t):
    q, k, v, tq, tk, tv = args
    return q + t * tq, k + t * tk, v + t * tv


@pytest.mark.parametrize("mask_kind,causal", [("none", False), ("none", True), ("bool", False),
                                              ("additive", False)])
def test_tangent_central_differences(mask_kind, causal):
    rng = np.random.default_rng(6)
    args = make(rng, B=1, H=2, Nq=6, Nk=6, d=4)
    mask = None
    if mask_kind == "bool":
        mask = (rng.random((1, 1, 6, 6)) < 0.7).astype(np.uint8)
        mask[..., 2] = 1
    elif mask_kind == "additive":
        mask = rng.standard_normal((1, 2, 6, 6))
    kw = dict(mask=mask, mask_kind=mask_kind, causal=causal)
    _, to, _, tlse = oracle_fwd(*args, **kw)
    h = 1e-5
    op, _, lp, _ = oracle_fwd(*_perturbed(args, h), **kw)
    om, _, lm, _ = oracle_fwd(*_perturbed(args, -h), **kw)
    np.testing.assert_allclose(to, (op - om) / (2 * h), rtol=0, atol=1e-8)
    np.testing.assert_allclose(tlse, (lp - lm) / (2 * h), rtol=0, atol=1e-8)


class Dual:
    """a + b*eps with eps^2 = 0: forward-mode differentiation by construction."""
    __slots__ = ("a", "b")

    def __init__(self, a, b=0.0):
        self.a, self.b = float(a), float(b)

    def __add__(self, o):
        o = o if isinstance(o, Dual) else Dual(o)
        return Dual(self.a + o.a, self.b + o.b)

    __radd__ = __add__

    def __sub__(self, o):
        o = o if isinstance(o, Dual) else Dual(o)
        return Dual(self.a - o.a, self.b - o.b)

    def __mul__(self, o):
        o = o if isinstance(o, Dual) else Dual(o)
        return Dual(self.a * o.a, self.a * o.b + self.b * o.a)

    __rmul__ = __mul__

    def __truediv__(self, o):
        o = o if isinstance(o, Dual) else Dual(o)
        return Dual(self.a / o.a, (self.b * o.a - self.a * o.b) / (o.a * o.a))

    def exp(self):
        e = math.exp(self.a)
        return Dual(e, e * self.b)


def naive_dual_attention(q, k, v, scale, visible):
    """Per-element attention over Dual numbers: for each row, scores, exp, normalise, weight V."""
    out = []
    for i in range(len(q)):
        js = [j for j in range(len(k)) if visible(i, j)]
        s = {j: scale * sum((q[i][c] * k[j][c] for c in range(len(q[i]))), Dual(0.0)) for j in js}
        mx = max(s[j].a for j in js)               # a constant shift; the softmax does not depend on it
        e = {j: (s[j] - mx).exp() for j in js}
        z = sum((e[j] for j in js), Dual(0.0))
        out.append([sum((e[j] * v[j][c] for j in js), Dual(0.0)) / z for c in range(len(v[0]))])
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_tangent_matches_dual_numbers(causal):
    rng = np.random.default_rng(7)
    q, k, v, tq, tk, tv = make(rng, B=1, H=1, Nq=4, Nk=4, d=3)
    scale = 0.8
    D = lambda x, t: [[Dual(x[i, c], t[i, c]) for c in range(x.shape[1])] for i in range(x.shape[0])]
    res = naive_dual_attention(D(q[0, 0], tq[0, 0]), D(k[0, 0], tk[0, 0]), D(v[0, 0], tv[0, 0]), scale,
                               (lambda i, j: j <= i) if causal else (lambda i, j: True))
    o, to, _, _ = oracle_fwd(q, k, v, tq, tk, tv, causal=causal, scale=scale)
    np.testing.assert_allclose(o[0, 0], [[x.a for x in r] for r in res], rtol=0, atol=1e-13)
    np.testing.assert_allclose(to[0, 0], [[x.b for x in r] for r in res], rtol=0, atol=1e-13)


# --------------------------------------------------------------- closed forms

def test_golden_two_key_logistic():
    with open(os.path.join(GOLDEN, "two_key_logistic.json")) as f:
        g = json.load(f)
    x = {n: np.array(a, dtype=np.float64)[None, None] for n, a in g["inputs"].items() if n != "scale"}
    o, to, lse, tlse = oracle_fwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"],
                                  scale=g["inputs"]["scale"])
    e = g["expected"]
    assert o[0, 0, 0, 0] == pytest.approx(e["o"], abs=1e-14)
    assert to[0, 0, 0, 0] == pytest.approx(e["to"], abs=1e-14)
    assert lse[0, 0, 0] == pytest.approx(e["lse"], abs=1e-14)
    assert tlse[0, 0, 0] == pytest.approx(e["tlse"], abs=1e-14)


def test_two_keys_logistic_random():
    """Two keys: P1 = expit(s1 - s2), dP1 = P1 (1 - P1) (ds1 - ds2)."""
    rng = np.random.default_rng(8)
    q, k, v, tq, tk, tv = make(rng, B=1, H=1, Nq=5, Nk=2, d=3)
    sc = 0.6
    o, to, _, _ = oracle_fwd(q, k, v, tq, tk, tv, scale=sc)
    q, k, v, tq, tk, tv = (a[0, 0] for a in (q, k, v, tq, tk, tv))
    s = sc * q @ k.T
    ds = sc * (tq @ k.T + q @ tk.T)
    p1 = scipy.special.expit(s[:, 0] - s[:, 1])[:, None]
    dp1 = p1 * (1 - p1) * (ds[:, [0]] - ds[:, [1]])
    np.testing.assert_allclose(o[0, 0], p1 * v[0] + (1 - p1) * v[1], atol=1e-13)
    np.testing.assert_allclose(to[0, 0], dp1 * (v[0] - v[1]) + p1 * tv[0] + (1 - p1) * tv[1], atol=1e-13)


def test_single_key():
    """One key: P = 1, so O = V and dO = dV for every query; tlse = ds."""
    rng = np.random.default_rng(9)
    q, k, v, tq, tk, tv = make(rng, Nq=5, Nk=1, d=4)
    o, to, lse, tlse = oracle_fwd(q, k, v, tq, tk, tv)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), atol=1e-14)
    np.testing.assert_allclose(to, np.broadcast_to(tv, to.shape), atol=1e-14)
    sc = 1 / math.sqrt(4)
    np.testing.assert_allclose(lse, sc * np.einsum("bhid,bhjd->bhi", q, k), atol=1e-13)
    np.testing.assert_allclose(tlse, sc * np.einsum("bhid,bhjd->bhi", tq, k)
                               + sc * np.einsum("bhid,bhjd->bhi", q, tk), atol=1e-13)


def test_zero_queries_closed_form():
    """Q = 0: uniform weights, O = mean(V); dO_i = (scale/N) dQ_i^T (K^T V - N kbar vbar^T) + mean(dV)."""
    rng = np.random.default_rng(10)
    _, k, v, tq, tk, tv = make(rng, B=1, H=2, Nq=6, Nk=11, d=4)
    q = np.zeros((1, 2, 6, 4))
    sc = 0.9
    o, to, lse, tlse = oracle_fwd(q, k, v, tq, tk, tv, scale=sc)
    N = 11
    for h in range(2):
        K, V, tQ, tV = k[0, h], v[0, h], tq[0, h], tv[0, h]
        np.testing.assert_allclose(o[0, h], np.broadcast_to(V.mean(0), (6, 4)), atol=1e-14)
        C = K.T @ V - N * np.outer(K.mean(0), V.mean(0))
        np.testing.assert_allclose(to[0, h], sc / N * tQ @ C + tV.mean(0), atol=1e-12)
        np.testing.assert_allclose(lse[0, h], math.log(N), atol=1e-14)
        np.testing.assert_allclose(tlse[0, h], sc * tQ @ K.mean(0), atol=1e-12)


def test_zero_tangents_give_zero():
    rng = np.random.default_rng(11)
    q, k, v, *_ = make(rng)
    _, to, _, tlse = oracle_fwd(q, k, v, None, None, None, causal=False)
    assert np.all(to == 0.0) and np.all(tlse == 0.0)


def test_value_tangent_equal_to_values():
    """dQ = dK = 0 and dV = V: O is linear in V, so dO = O."""
    rng = np.random.default_rng(12)
    q, k, v, *_ = make(rng)
    o, to, _, tlse = oracle_fwd(q, k, v, None, None, v)
    np.testing.assert_allclose(to, o, atol=1e-14)
    assert np.all(tlse == 0.0)


def test_row_constant_score_tangent():
    """dQ = 0 and all rows of dK equal: dS_ij = scale q_i.c is constant along j, so dP = 0 and dO = P dV."""
    rng = np.random.default_rng(13)
    q, k, v, _, _, tv = make(rng, Nq=5, Nk=8, d=4)
    tk = np.broadcast_to(rng.standard_normal((2, 3, 1, 4)), k.shape).copy()
    sc = 0.5
    o, to, _, tlse = oracle_fwd(q, k, v, np.zeros_like(q), tk, tv, scale=sc)
    _, to_v, _, _ = oracle_fwd(q, k, v, None, None, tv, scale=sc)
    np.testing.assert_allclose(to, to_v, atol=1e-13)
    np.testing.assert_allclose(tlse, sc * np.einsum("bhid,bhd->bhi", q, tk[:, :, 0]), atol=1e-13)


def test_linear_in_tangents():
    rng = np.random.default_rng(14)
    q, k, v, tq, tk, tv = make(rng)
    _, _, _, tq2, tk2, tv2 = make(rng)
    a, b = 0.7, -1.3
    _, t1, _, l1 = oracle_fwd(q, k, v, tq, tk, tv)
    _, t2, _, l2 = oracle_fwd(q, k, v, tq2, tk2, tv2)
    _, t3, _, l3 = oracle_fwd(q, k, v, a * tq + b * tq2, a * tk + b * tk2, a * tv + b * tv2)
    np.testing.assert_allclose(t3, a * t1 + b * t2, atol=1e-12)
    np.testing.assert_allclose(l3, a * l1 + b * l2, atol=1e-12)


# --------------------------------------------------------------- masks, brute force

def subset_attention(q, k, v, tq, tk, tv, keep, scale):
    """Row by row: attention over only the kept keys, computed on the reduced key set."""
    n = q.shape[0]
    o = np.zeros((n, v.shape[1]))
    to = np.zeros_like(o)
    for i in range(n):
        js = np.nonzero(keep[i])[0]
        if len(js) == 0:
            continue
        oi, ti, _, _ = oracle_fwd(q[None, None, [i]], k[None, None, js], v[None, None, js],
                                  tq[None, None, [i]], tk[None, None, js], tv[None, None, js], scale=scale)
        o[i], to[i] = oi[0, 0, 0], ti[0, 0, 0]
    return o, to


def test_bool_mask_equals_reduced_key_set_all_4x4():
    """Every one of the 2^16 boolean masks of a 4x4 score block (all-False rows included)."""
    rng = np.random.default_rng(15)
    q, k, v, tq, tk, tv = make(rng, B=1, H=1, Nq=4, Nk=4, d=3)
    q, k, v, tq, tk, tv = (a[0, 0] for a in (q, k, v, tq, tk, tv))
    bits = ((np.arange(1 << 16)[:, None] >> np.arange(16)[None, :]) & 1).reshape(-1, 1, 4, 4)
    # one oracle call with the 65536 masks laid out as the batch dimension
    rep = lambda a: np.broadcast_to(a, (bits.shape[0], 1) + a.shape)
    o, to, lse, tlse = oracle_fwd(rep(q), rep(k), rep(v), rep(tq), rep(tk), rep(tv),
                                  mask=bits.astype(np.uint8), mask_kind="bool", scale=0.7)
    # reference for each row pattern: the 16 row masks per query row are enough
    for i in range(4):
        for pat in range(16):
            keep = np.zeros((4, 4), dtype=bool)
            keep[i] = [(pat >> j) & 1 for j in range(4)]
            ro, rto = subset_attention(q, k, v, tq, tk, tv, keep, 0.7)
            sel = np.all(bits[:, 0, i, :] == keep[i].astype(int), axis=1)
            np.testing.assert_allclose(o[sel, 0, i], np.broadcast_to(ro[i], (sel.sum(), 3)), atol=1e-13)
            np.testing.assert_allclose(to[sel, 0, i], np.broadcast_to(rto[i], (sel.sum(), 3)), atol=1e-13)
            if pat == 0:
                assert np.all(np.isneginf(lse[sel, 0, i])) and np.all(tlse[sel, 0, i] == 0)


def test_causal_equals_tril_bool_mask_and_rectangular():
    rng = np.random.default_rng(16)
    for Nq, Nk in [(9, 9), (5, 9), (9, 5)]:
        args = make(rng, Nq=Nq, Nk=Nk, d=4)
        tril = (np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]).astype(np.uint8)[None, None]
        a = oracle_fwd(*args, causal=True)
        b = oracle_fwd(*args, mask=tril, mask_kind="bool")
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


def test_additive_inf_mask_equals_bool():
    rng = np.random.default_rng(17)
    args = make(rng, Nq=6, Nk=7, d=4)
    keep = rng.random((2, 3, 6, 7)) < 0.5
    keep[0, 0, 2] = False                     # one fully masked row
    add = np.where(keep, 0.0, -np.inf)
    a = oracle_fwd(*args, mask=keep.astype(np.uint8), mask_kind="bool")
    b = oracle_fwd(*args, mask=add, mask_kind="additive")
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-13)
    o, to, lse, tlse = a
    assert np.all(o[0, 0, 2] == 0) and np.all(to[0, 0, 2] == 0)
    assert np.isneginf(lse[0, 0, 2]) and tlse[0, 0, 2] == 0


def test_additive_row_shift():
    rng = np.random.default_rng(18)
    args = make(rng, Nq=6, Nk=7, d=4)
    m = rng.standard_normal((2, 1, 6, 7))
    c = rng.standard_normal((2, 1, 6, 1)) * 3
    o1, t1, l1, s1 = oracle_fwd(*args, mask=m, mask_kind="additive")
    o2, t2, l2, s2 = oracle_fwd(*args, mask=m + c, mask_kind="additive")
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(t2, t1, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + c[..., 0], atol=1e-12)
    np.testing.assert_allclose(s2, s1, atol=1e-12)


def test_causal_and_mask_intersect():
    rng = np.random.default_rng(19)
    args = make(rng, Nq=8, Nk=8, d=4)
    keep = (rng.random((2, 1, 8, 8)) < 0.6).astype(np.uint8)
    tril = (np.arange(8)[None, :] <= np.arange(8)[:, None]).astype(np.uint8)
    a = oracle_fwd(*args, mask=keep, mask_kind="bool", causal=True)
    b = oracle_fwd(*args, mask=keep * tril, mask_kind="bool")
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_row_sample_matches_full():
    """q_pos lets a subset of rows be evaluated alone (used for sampled checks at full size)."""
    rng = np.random.default_rng(20)
    q, k, v, tq, tk, tv = make(rng, Nq=12, Nk=12, d=4)
    rows = np.array([0, 5, 11, 3])
    full = oracle_fwd(q, k, v, tq, tk, tv, causal=True)
    part = oracle_fwd(q[:, :, rows], k, v, tq[:, :, rows], k * 0 + tk, tv, causal=True, q_pos=rows)
    for x, y in zip(full, part):
        np.testing.assert_array_equal(x[:, :, rows], y)
