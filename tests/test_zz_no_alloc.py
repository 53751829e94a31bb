"""jvpattn_bwd_noalloc (the reverse pass on the library's fixed scratch) against jvpattn_bwd.

For callers that cannot allocate. Two calls in a row through the C ABI, the
second on a smaller problem (the scratch keeps the first call's contents), each
equal bit for bit to jvpattn_bwd with a caller workspace on the same inputs --
the same kernels, so the same rounding -- and within the oracle's bar.
"""
import pytest
import torch

from forward_mode_autodiff_amd import inputs as I
from forward_mode_autodiff_amd.jvpattn import JvpattnError, jvpattn_bwd, jvpattn_fwd
from tests.bwd_cases import magnitudes, reference
from tests.parity import BWD_NAMES, bwd_failures

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def both(w):
    x = I.make_inputs(w, cotangents=True)
    d = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=d["mask"],
                                   causal=w.causal)
    args = (d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], o, to, lse, tlse, d["do"], d["dto"])
    a = jvpattn_bwd(*args, mask=d["mask"], causal=w.causal, noalloc=True)
    b = jvpattn_bwd(*args, mask=d["mask"], causal=w.causal)
    torch.cuda.synchronize()
    return x, a, b


def test_noalloc_matches_workspace_call_twice_shrinking():
    big = I.Workload("noalloc_big", B=2, H=4, N=600, d=64, dtype="bf16", causal=True, std=1.0, seed=70)
    small = I.Workload("noalloc_small", B=1, H=2, N=150, d=64, dtype="f16", mask_kind="bool", keep=0.7, std=1.0,
                       seed=71)
    for w in (big, small):
        x, a, b = both(w)
        for n, u, t in zip(BWD_NAMES, a, b):
            assert torch.equal(u, t), (w.name, n)
        got = {n: u.double().cpu().numpy() for n, u in zip(BWD_NAMES, a)}
        bad = bwd_failures(got, reference(x, w), magnitudes(x, w), w.dtype)
        assert not bad, (w.name, bad)


def test_noalloc_other_head_dims_and_float32():
    """The same entry on the d = 128 and float32 kernels (two calls, the second smaller)."""
    for w in (I.Workload("noalloc_d128", B=2, H=2, N=300, d=128, dtype="bf16", causal=True, std=1.0, seed=73),
              I.Workload("noalloc_f32", B=1, H=2, N=130, d=64, dtype="f32", std=1.0, seed=74)):
        x, a, b = both(w)
        for n, u, t in zip(BWD_NAMES, a, b):
            assert torch.equal(u, t), (w.name, n)
        got = {n: u.double().cpu().numpy() for n, u in zip(BWD_NAMES, a)}
        bad = bwd_failures(got, reference(x, w), magnitudes(x, w), w.dtype)
        assert not bad, (w.name, bad)


def test_noalloc_rejects_more_rows_than_its_scratch():
    w = I.Workload("noalloc_huge", B=1, H=1, N=1, d=64, dtype="bf16", seed=72)
    x = I.make_inputs(w, cotangents=True)
    d = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
    q = torch.zeros((1, 16, (1 << 16) + 1, 64), dtype=torch.bfloat16, device=DEV)   # 2^20 + 16 rows
    k = torch.zeros((1, 16, 64, 64), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(q.shape[:3], device=DEV)
    with pytest.raises(JvpattnError, match="SCRATCH"):
        jvpattn_bwd(q, k, k, None, None, None, q, q, lse, lse, q, q, noalloc=True,
                    out=(torch.empty_like(q), torch.empty_like(k), torch.empty_like(k), None, None, None))
    assert d["q"].shape[2] == 1
