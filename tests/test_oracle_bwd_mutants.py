"""The reverse-pass bar has power: single-term mistakes planted in the oracle fail it (CPU).

Each mutant is ``oracle_bwd_head`` with one term of the chain rule dropped,
its sign flipped, its scale lost or an operand swapped -- mistakes a kernel
could plausibly make. Each is run through the exact bar of the GPU tests
(tests/parity.py ``bwd_failures``, per element |got - ref| <= rho * M_ij) on
the same inputs and cases as tests/test_gpu_bwd.py, and must fail:
  * the full-size HVP workload (B=4, H=16, N=2048, d=64, bf16, causal), two
    query heads of batch 0, at the specified 1/sqrt(d) spread or at unit
    spread (the terms carried by tlse and the score tangent only stand out of
    the bf16 rounding at unit spread); and
  * at least one of the six small configurations of ``test_small``.
Grouped-head mistakes (interleaved instead of blocked head sharing, keeping
one query head's cotangent instead of the sum) must fail the grouped configs.
"""
import inspect

import numpy as np
import pytest

import oracle.attention as oa
import oracle.attention_bwd as ob
from forward_mode_autodiff_amd import inputs as I
from tests.bwd_cases import HVP_HEADS, HVP_UNIT, SMALL, magnitudes, reference
from tests.parity import bwd_failures


def _mutant(src_old, src_new):
    """A copy of oracle_bwd_head with one line changed (the true module is untouched)."""
    src = inspect.getsource(ob.oracle_bwd_head)
    assert src_old in src, src_old
    ns = dict(ob.__dict__)
    exec(compile(src.replace(src_old, src_new), "<mutant>", "exec"), ns)
    return ns["oracle_bwd_head"]


MUTANTS = {
    # reverse of dO = dP V + P dV
    "gdP_wrong_value_operand": ("g_dP = gto @ v.T", "g_dP = gto @ tv.T"),
    "gv_drop_dP_gto": ("g_v = dP.T @ gto", "g_v = 0.0 * (dP.T @ gto)"),
    "gP_drop_gto_tv": ("g_P = gto @ tv.T", "g_P = 0.0 * (gto @ tv.T)"),
    "gtv_wrong_cotangent": ("g_tv = P.T @ gto", "g_tv = P.T @ go"),
    # reverse of O = P V
    "gP_drop_go_v": ("g_P = g_P + go @ v.T", "g_P = g_P"),
    "gv_drop_P_go": ("g_v = g_v + P.T @ go", "g_v = g_v"),
    # reverse of dP = P (dS - t)
    "gP_drop_tlse": ("g_P = g_P + g_dP * (dS - t)", "g_P = g_P + g_dP * dS"),
    "gP_drop_dP_term": ("g_P = g_P + g_dP * (dS - t)", "g_P = g_P"),
    "gdS_drop_direct": ("g_dS = g_dP * P", "g_dS = 0.0 * g_dP * P"),
    "gt_dropped": ("g_t = -np.sum(g_dP * P, axis=1, keepdims=True)", "g_t = 0.0 * g_dP[:, :1]"),
    "gt_sign": ("g_t = -np.sum(g_dP * P, axis=1, keepdims=True)", "g_t = np.sum(g_dP * P, axis=1, keepdims=True)"),
    # reverse of t = rowsum(P dS)
    "gP_drop_gt_dS": ("g_P = g_P + g_t * dS", "g_P = g_P"),
    "gdS_drop_gt_P": ("g_dS = g_dS + g_t * P", "g_dS = g_dS"),
    # reverse of dS = scale (dQ K^T + Q dK^T)
    "gtq_wrong_operand": ("g_tq = scale * (g_dS @ k)", "g_tq = scale * (g_dS @ tk)"),
    "gk_drop_dS_tq": ("g_k = scale * (g_dS.T @ tq)", "g_k = 0.0 * (g_dS.T @ tq)"),
    "gq_drop_dS_tk": ("g_q = scale * (g_dS @ tk)", "g_q = 0.0 * (g_dS @ tk)"),
    "gtk_unscaled": ("g_tk = scale * (g_dS.T @ q)", "g_tk = g_dS.T @ q"),
    # reverse of P = softmax(S) and S = scale Q K^T + M
    "gS_sign_rowsum": ("g_P - np.sum(g_P * P, axis=1, keepdims=True)", "g_P + np.sum(g_P * P, axis=1, keepdims=True)"),
    "gS_drop_rowsum": ("g_S = P * (g_P - np.sum(g_P * P, axis=1, keepdims=True))", "g_S = P * g_P"),
    "gq_drop_S_k": ("g_q = g_q + scale * (g_S @ k)", "g_q = g_q"),
    "gk_drop_S_q": ("g_k = g_k + scale * (g_S.T @ q)", "g_k = g_k"),
    "gk_unscaled_S_q": ("g_k = g_k + scale * (g_S.T @ q)", "g_k = g_k + g_S.T @ q"),
}


@pytest.fixture(scope="module")
def hvp_cases():
    """(name, workload, inputs, reference, magnitudes) of the two HVP-shaped GPU cases, computed once."""
    out = []
    for w in (I.HVP, HVP_UNIT):
        x = I.make_inputs(w, cotangents=True)
        out.append((w.name, w, x, reference(x, w, heads=HVP_HEADS), magnitudes(x, w, heads=HVP_HEADS)))
    return out


@pytest.fixture(scope="module")
def small_cases():
    out = []
    for w in SMALL:
        x = I.make_inputs(w, cotangents=True)
        out.append((f"{w.dtype}-{w.causal}-{w.std}", w, x, reference(x, w), magnitudes(x, w)))
    return out


def test_true_oracle_passes_the_bar(hvp_cases, small_cases):
    for name, w, x, ref, M in hvp_cases + small_cases:
        assert not bwd_failures(ref, ref, M, w.dtype), name


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_the_bars(name, hvp_cases, small_cases, monkeypatch):
    monkeypatch.setattr(ob, "oracle_bwd_head", _mutant(*MUTANTS[name]))
    caught_hvp = [c for c, w, x, ref, M in hvp_cases
                  if bwd_failures(reference(x, w, heads=HVP_HEADS), ref, M, w.dtype)]
    caught_small = [c for c, w, x, ref, M in small_cases if bwd_failures(reference(x, w), ref, M, w.dtype)]
    print(f"{name}: fails HVP cases {caught_hvp}; small cases {caught_small}")
    assert caught_hvp, f"mutant {name} passes both HVP-shaped bars"
    assert caught_small, f"mutant {name} passes every small configuration"


GQA_CASES = [I.Workload("gqa_bwd_4_2", B=2, H=4, Hkv=2, N=200, d=64, dtype="bf16", causal=False, std=1.0, seed=21),
             I.Workload("gqa_bwd_4_1", B=2, H=4, Hkv=1, N=200, d=64, dtype="bf16", causal=True, std=1.0, seed=21)]


@pytest.mark.parametrize("w", GQA_CASES, ids=lambda w: w.name)
def test_grouped_head_mutants_fail_the_bar(w, monkeypatch):
    x = I.make_inputs(w, cotangents=True)
    ref, M = reference(x, w), magnitudes(x, w)
    assert not bwd_failures(ref, ref, M, w.dtype)
    if w.hkv > 1:   # interleaved sharing only differs from blocked sharing with several K/V heads
        with monkeypatch.context() as m:
            m.setattr(ob, "kv_head", lambda h, H, Hkv: h % Hkv)
            assert bwd_failures(reference(x, w), ref, M, w.dtype)
    src = inspect.getsource(ob.oracle_bwd).replace("gk[b, g] += r[1]", "gk[b, g] = r[1]")
    ns = dict(ob.__dict__)
    exec(compile(src, "<mutant>", "exec"), ns)
    with monkeypatch.context() as m:
        m.setattr(ob, "oracle_bwd", ns["oracle_bwd"])
        import tests.bwd_cases as bc
        m.setattr(bc, "oracle_bwd", ns["oracle_bwd"])
        assert bwd_failures(reference(x, w), ref, M, w.dtype)
    assert oa.kv_head(3, 4, 2) == 1   # the true module is untouched
