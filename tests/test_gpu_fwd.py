"""Parity of the HIP forward (through the C ABI) against the float64 oracle.

Inputs are seeded and synthetic (forward_mode_autodiff_amd.inputs); the
oracle sees exactly the values the GPU sees. Bars: tests/parity.py. The
workloads the method is specified on run in full, checked element by element
where the oracle finishes in seconds and on sampled rows at the largest
sizes; a stress suite (unit and doubled input spread, isolated tangent terms)
gives the comparisons power the 1/sqrt(d) spread lacks.
"""
import numpy as np
import pytest
import torch

from forward_mode_autodiff_amd import inputs as I
from forward_mode_autodiff_amd.jvpattn import jvpattn_fwd, jvpattn_fwd_set_algo, jvpattn_set_workgroups
from oracle import oracle_fwd
from tests.parity import assert_parity, failures

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# The library picks between an 8-wave ping-pong kernel (16-bit, d = 64, large
# grids), a 4-wave kernel, the 4-wave kernel with the key range split between
# two groups of waves (16-bit, d = 64, small grids), and that split on 64-row
# blocks with two waves per group (smallest grids); the override forces one
# so each is checked on every kernel-sensitive case.
KERNELS = ["pp", "wg4", "split", "split64"]


@pytest.fixture(autouse=True)
def _automatic_plan():
    """Every test starts and ends with the library's own launch plan."""
    jvpattn_fwd_set_algo()
    jvpattn_set_workgroups()
    yield
    jvpattn_fwd_set_algo()
    jvpattn_set_workgroups()


@pytest.fixture(params=KERNELS)
def kernel(request, _automatic_plan):
    jvpattn_fwd_set_algo(kernel=request.param)
    return request.param


def to_dev(x):
    return {k: (None if v is None else v.to(DEV)) for k, v in x.items()}


def gpu_run(x, causal, scale=None, tangents=("tq", "tk", "tv")):
    d = to_dev(x)
    t = {n: (d[n] if n in tangents else None) for n in ("tq", "tk", "tv")}
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], t["tq"], t["tk"], t["tv"], mask=d["mask"],
                                   causal=causal, scale=scale)
    torch.cuda.synchronize()
    return {"o": o.float().cpu(), "to": to.float().cpu(), "lse": lse.cpu(), "tlse": tlse.cpu()}


def f64(t):
    return None if t is None else t.double().numpy()


def oracle_run(x, mask_kind, causal, scale=None, tangents=("tq", "tk", "tv"), heads=None, rows=None):
    """Oracle on all heads and rows, or on heads [(b, h), ...] and query rows `rows` only."""
    tq, tk, tv = (f64(x[n]) if n in tangents else None for n in ("tq", "tk", "tv"))
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    mask = None
    if x["mask"] is not None:
        mask = x["mask"].double().numpy() if mask_kind == "additive" else x["mask"].numpy()
    if heads is None:
        o, to, lse, tlse = oracle_fwd(q, k, v, tq, tk, tv, mask=mask, mask_kind=mask_kind, causal=causal,
                                      scale=scale)
        return {"o": o, "to": to, "lse": lse, "tlse": tlse}
    out = {n: [] for n in ("o", "to", "lse", "tlse")}
    grp = q.shape[1] // k.shape[1]
    for b, h in heads:
        sl = lambda a: None if a is None else a[b:b + 1, h:h + 1]
        slk = lambda a: None if a is None else a[b:b + 1, h // grp:h // grp + 1]   # the K/V head h reads
        m = None if mask is None else mask[b:b + 1, (h if mask.shape[1] > 1 else 0):][:, :1]
        r = oracle_fwd(sl(q)[:, :, rows], slk(k), slk(v), None if tq is None else sl(tq)[:, :, rows], slk(tk),
                       slk(tv), mask=m, mask_kind=mask_kind, causal=causal, scale=scale, q_pos=rows)
        for n, a in zip(("o", "to", "lse", "tlse"), r):
            out[n].append(a[0, 0])
    return {n: np.stack(a) for n, a in out.items()}


def pick(got, heads, rows):
    return {n: np.stack([got[n][b, h][rows].numpy() for b, h in heads]) for n in got}


def check(w, x=None, scale=None, tangents=("tq", "tk", "tv")):
    x = I.make_inputs(w) if x is None else x
    got = gpu_run(x, w.causal, scale, tangents)
    ref = oracle_run(x, w.mask_kind, w.causal, scale, tangents)
    assert_parity(got, ref, w.dtype, w.name, spec_spread=w.std is None)
    return got, ref


# ------------------------------------------------ the specified workloads

def test_tiny_f32():
    check(I.TINY)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", I.SEQ_NS)
def test_seq_sweep_f16(N, causal):
    check(I.seq(N, causal))


@pytest.mark.parametrize("N", [512, 2048])
def test_seq_bf16(N):
    check(I.seq(N, False, dtype="bf16"))


@pytest.mark.parametrize("w", [I.MASKED_BOOL, I.MASKED_ADD], ids=lambda w: w.name)
def test_masked(w):
    check(w)


def sampled_rows(N, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=n, replace=False).tolist()) | {0, 1, 31, 32, 127, 128, N - 1}
    return np.array(sorted(r for r in rows if r < N))


def test_hvp_workload_forward_sampled(kernel):
    """B=4, H=16, N=2048, d=64, bf16, causal: every head launched, sampled heads x rows checked."""
    w = I.HVP
    x = I.make_inputs(w)
    got = gpu_run(x, True)
    heads = [(0, 0), (1, 7), (2, 12), (3, 15)]
    rows = sampled_rows(w.N, 48, 1)
    ref = oracle_run(x, "none", True, heads=heads, rows=rows)
    assert_parity(pick(got, heads, rows), ref, w.dtype, w.name, spec_spread=True)
    assert torch.isfinite(got["o"]).all() and torch.isfinite(got["to"]).all()


def test_wide_workload_sampled():
    """B=256, H=8, N=512, d=128, bf16: every head launched, sampled heads x rows checked."""
    w = I.WIDE
    x = I.make_inputs(w)
    got = gpu_run(x, False)
    heads = [(0, 0), (77, 3), (200, 5), (255, 7)]
    rows = sampled_rows(w.N, 40, 2)
    ref = oracle_run(x, "none", False, heads=heads, rows=rows)
    assert_parity(pick(got, heads, rows), ref, w.dtype, w.name, spec_spread=True)
    assert torch.isfinite(got["o"]).all() and torch.isfinite(got["to"]).all()


# ------------------------------------------------ stress suite (power)

STRESS_SHAPES = [(1, 2, 200, 64), (1, 1, 97, 128)]


@pytest.mark.parametrize("std", [1.0, 2.0])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("mask_kind", ["none", "bool", "additive"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", STRESS_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_stress(shape, causal, mask_kind, dtype, std, kernel):
    B, H, N, d = shape
    w = I.Workload("stress", B=B, H=H, N=N, d=d, dtype=dtype, causal=causal, mask_kind=mask_kind, std=std,
                   seed=11, mask_heads=H if mask_kind == "additive" else 1, keep=0.7)
    check(w)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("tangents", [("tv",), ("tq", "tk"), ("tq",), ("tk",), ()],
                         ids=lambda t: "+".join(t) or "none")
def test_term_isolation(dtype, tangents, kernel):
    """Only some tangents given (others NULL): isolates dP V, P dV, the dQ and dK paths; none -> dO = 0."""
    w = I.Workload("iso", B=1, H=2, N=160, d=64, dtype=dtype, std=1.0, seed=12)
    got, _ = check(w, tangents=tangents)
    if not tangents:
        assert torch.all(got["to"] == 0) and torch.all(got["tlse"] == 0)


# ------------------------------------------------ head dimensions 32, 96, 256
# d = 32 and 96 run the d = 64 and d = 128 kernels with the missing head-dim
# columns read as zeros; d = 256 (16-bit types) has a kernel of its own whose
# wave pairs split the head dimension and swap partial scores.

HEAD_DIMS = [32, 96, 256]


def _dtypes(d):
    return ("bf16", "f16") if d == 256 else ("bf16", "f16", "f32")


@pytest.mark.parametrize("std", [1.0, 2.0])
@pytest.mark.parametrize("mask_kind", ["none", "bool", "additive"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", HEAD_DIMS)
def test_head_dim_stress(d, causal, mask_kind, std):
    for dtype in _dtypes(d):
        w = I.Workload(f"d{d}", B=1, H=2, N=200, d=d, dtype=dtype, causal=causal, mask_kind=mask_kind, std=std,
                       seed=100 + d, mask_heads=2 if mask_kind == "additive" else 1, keep=0.7)
        check(w)


@pytest.mark.parametrize("mask_kind", ["none", "bool"])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dim_32_every_kernel(causal, mask_kind, kernel):
    for dtype in ("bf16", "f16"):
        w = I.Workload("d32k", B=1, H=2, N=300, d=32, dtype=dtype, causal=causal, mask_kind=mask_kind, std=1.0,
                       seed=131, keep=0.7)
        check(w)


@pytest.mark.parametrize("N", [1, 31, 33, 63, 64, 65, 127, 129, 255, 257])
@pytest.mark.parametrize("d", HEAD_DIMS)
def test_head_dim_tile_boundaries(d, N):
    for dtype, causal in (("bf16", False), ("f16", True)):
        w = I.Workload(f"d{d}edge{N}", B=1, H=2, N=N, d=d, dtype=dtype, causal=causal, std=1.0, seed=N + d)
        check(w)


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_head_dim_rectangular_grouped(d):
    for Nq, Nk, causal in ((70, 200, False), (200, 70, True), (1, 130, True)):
        w = I.Workload(f"d{d}rect", B=2, H=4, Hkv=2, N=Nq, Nk=Nk, d=d, dtype="bf16", causal=causal, std=1.0,
                       seed=5 + d)
        check(w)


# The mask-free bfloat16 kernel at 128 columns walks several row blocks per workgroup
# (the next block's Q and first tiles load during the current one's epilogue).
# A small cap forces many rounds on small inputs: the walk must give the same
# bits as one block per workgroup, and oracle parity (float16 runs one block per
# workgroup whatever the cap: the same checks hold).
@pytest.mark.parametrize("cap", [8, 5, 24])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (128, "f16"), (96, "bf16")])
def test_walking_row_blocks(d, dtype, causal, cap):
    shapes = [dict(B=2, H=4, N=700), dict(B=4, H=8, Hkv=2, N=300), dict(B=1, H=3, N=200, Nk=450)]
    for i, s in enumerate(shapes):
        w = I.Workload(f"walk{d}_{i}", d=d, dtype=dtype, causal=causal, std=1.0, seed=40 + i, **s)
        x = I.make_inputs(w)
        for order in (None, "head"):
            jvpattn_fwd_set_algo(order=order)
            jvpattn_set_workgroups(1 << 30)   # one block per workgroup
            one = gpu_run(x, causal)
            jvpattn_set_workgroups(cap)
            walk = gpu_run(x, causal)
            for n in one:
                assert torch.equal(one[n], walk[n]), (w.name, order, n)
        assert_parity(walk, oracle_run(x, "none", causal), dtype, w.name, spec_spread=False)


@pytest.mark.parametrize("case", ["ramp", "jump", "late"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [96, 256])
def test_head_dim_running_reference(d, dtype, case):
    """The rebase paths of the d = 128 and d = 256 kernels: rising scores, a jump past the float32
    range, rows whose first visible key comes late (as in the d = 64 tests below)."""
    w = I.Workload(f"d{d}{case}", B=1, H=2, N=512, d=d, dtype=dtype, mask_kind="additive", std=1.0, seed=24 + d)

    def late(m):
        m[0::2, :300] = float("-inf")
        m[0::2, 300:] = 100.0
    fill = {"ramp": lambda m: m.add_(torch.arange(w.N, dtype=torch.float32)[None, :] * 0.6),
            "jump": lambda m: m[:, 300].fill_(200.0), "late": late}[case]
    check(w, _additive_rows(w, fill))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [96, 256])
def test_head_dim_f16_large_score_tangents(d, causal):
    """|dS| ~ 2^13 in float16: weights are lowered (and the accumulators with them) instead of overflowing."""
    w = I.Workload(f"d{d}big_ds", B=1, H=2, N=300, d=d, dtype="f16", causal=causal, std=1.0, seed=40 + d)
    x = I.make_inputs(w)
    for n in ("tq", "tk"):
        x[n] = (x[n].float() * 2.0 ** 12).to(torch.float16)
    got, _ = check(w, x=x)
    assert np.all(np.isfinite(got["to"].numpy()))


@pytest.mark.parametrize("layout,extra,kind,causal", [
    ("sliding", {"window": 70}, "bool", False),
    ("blockdiag", {"block": 96}, "bits", True),
    ("blockdiag", {"block": 128}, "additive", False),
    ("pad_right", None, "bool", True),
    ("window", None, "additive", False),
])
@pytest.mark.parametrize("d", [96, 256])
def test_head_dim_mask_early_outs(d, layout, extra, kind, causal):
    """Per-row (sliding, block-diagonal) and query-shared (key padding, window) masks at d = 96 / 256:
    the early-outs on and off give the same bits, and the oracle's values."""
    from forward_mode_autodiff_amd.jvpattn import pack_mask_bits
    w = I.Workload(f"d{d}_mask_{layout}", B=2, H=2, N=300, d=d, dtype="bf16", causal=causal,
                   mask_kind="bool" if kind == "bits" else kind, mask_layout=layout, std=1.0, seed=37 + d,
                   **({"extra": extra} if extra else {}))
    x = I.make_inputs(w)
    dd = to_dev(x)
    m = pack_mask_bits(dd["mask"]) if kind == "bits" else dd["mask"]
    runs = []
    for skip in (True, False):
        jvpattn_fwd_set_algo(key_range=skip)
        out = jvpattn_fwd(dd["q"], dd["k"], dd["v"], dd["tq"], dd["tk"], dd["tv"], mask=m, causal=causal,
                          mask_kind="bits" if kind == "bits" else None)
        torch.cuda.synchronize()
        runs.append(tuple(t.clone() for t in out))
    for a, b in zip(*runs):
        assert torch.equal(a, b)
    o, to, lse, tlse = runs[0]
    got = {"o": o.float().cpu(), "to": to.float().cpu(), "lse": lse.cpu(), "tlse": tlse.cpu()}
    assert_parity(got, oracle_run(x, "bool" if kind == "bits" else kind, causal), "bf16", w.name,
                  spec_spread=False)


# ------------------------------------------------ edges

@pytest.mark.parametrize("N", [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 130, 255, 256, 257, 511, 513])
def test_tile_boundaries(N, kernel):
    for dtype, causal in (("bf16", False), ("f16", True)):
        w = I.Workload(f"edge{N}", B=1, H=2, N=N, d=64, dtype=dtype, causal=causal, std=1.0, seed=N)
        check(w)


@pytest.mark.parametrize("Nq,Nk", [(64, 200), (200, 64), (1, 300), (130, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_rectangular(Nq, Nk, causal, kernel):
    w = I.Workload("rect", B=1, H=2, N=Nq, Nk=Nk, d=64, dtype="bf16", causal=causal, std=1.0, seed=3)
    check(w)


def test_d128_f16_and_f32_ragged():
    for dtype in ("f16", "f32"):
        check(I.Workload("d128", B=2, H=1, N=150, d=128, dtype=dtype, causal=True, std=1.0, seed=4))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_fully_masked_rows(dtype, kernel):
    w = I.Workload("fm", B=1, H=2, N=70, d=64, dtype=dtype, mask_kind="bool", std=1.0, seed=5, keep=0.5)
    x = I.make_inputs(w)
    x["mask"][0, 0, 3, :] = 0          # one row with no visible key
    x["mask"][0, 0, 66, :] = 0
    got, _ = check(w, x=x)
    for r in (3, 66):
        assert torch.all(got["o"][0, :, r] == 0) and torch.all(got["to"][0, :, r] == 0)
        assert torch.all(torch.isneginf(got["lse"][0, :, r])) and torch.all(got["tlse"][0, :, r] == 0)


def test_additive_minus_inf_rows(kernel):
    w = I.Workload("addinf", B=1, H=1, N=64, d=64, dtype="f16", mask_kind="additive", std=1.0, seed=6)
    x = I.make_inputs(w)
    x["mask"][0, 0, 5, :] = float("-inf")
    x["mask"][0, 0, 9, ::2] = float("-inf")
    check(w, x=x)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N", [32, 64])
def test_additive_small_n_regression(dtype, N, kernel):
    """The prior implementation's benchmark lists its additive-mask runs at N=32 and 64 as failing."""
    check(I.Workload("addsmall", B=2, H=8, N=N, d=64, dtype=dtype, mask_kind="additive", seed=N))
    check(I.Workload("addsmall_s", B=2, H=8, N=N, d=64, dtype=dtype, mask_kind="additive", std=1.0, seed=N))


def test_key_padding_mask_broadcast_rows(kernel):
    """A [B,1,1,Nk] boolean mask: mask_stride_q = 0 broadcasts one key-padding row to every query."""
    w = I.Workload("pad", B=2, H=3, N=96, d=64, dtype="bf16", mask_kind="bool", std=1.0, seed=7)
    x = I.make_inputs(w)
    pad = torch.ones(2, 1, 1, 96, dtype=torch.uint8)
    pad[0, 0, 0, 50:] = 0
    pad[1, 0, 0, :7] = 0
    x["mask"] = pad
    got = gpu_run(x, False)
    ref = oracle_run(dict(x, mask=pad.expand(2, 1, 96, 96).contiguous()), "bool", False)
    assert_parity(got, ref, "bf16", "pad")


def test_custom_scale(kernel):
    w = I.Workload("scale", B=1, H=2, N=100, d=64, dtype="bf16", std=1.0, seed=8)
    check(w, scale=0.3)
    w = I.Workload("scale_add", B=1, H=2, N=100, d=64, dtype="f16", mask_kind="additive", std=1.0, seed=8)
    check(w, scale=0.05)


# ------------------------------------------------ the running reference
# The kernels keep one reference per row (a past maximum) and rebase it only
# when a block's weights against it grow too large. These inputs force that
# path on every block, across a jump that overflows float32 weights, and for
# rows whose first visible key comes late.

def _additive_rows(w, fill):
    x = I.make_inputs(w)
    N = w.N
    m = torch.zeros(N, N, dtype=torch.float32)
    fill(m)
    x["mask"] = m.to(x["q"].dtype)[None, None].contiguous()
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_rising_scores_rebase_every_block(dtype, kernel):
    """An additive ramp of 0.6 per key lifts each 32-key block ~19 above the last."""
    w = I.Workload("ramp", B=1, H=2, N=512, d=64, dtype=dtype, mask_kind="additive", std=1.0, seed=21)
    x = _additive_rows(w, lambda m: m.add_(torch.arange(w.N, dtype=torch.float32)[None, :] * 0.6))
    check(w, x)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_score_jump_past_float32_range(dtype, kernel):
    """+200 on key 300: weights against the old reference overflow to inf."""
    w = I.Workload("jump", B=1, H=2, N=512, d=64, dtype=dtype, mask_kind="additive", std=1.0, seed=22)
    x = _additive_rows(w, lambda m: m[:, 300].fill_(200.0))
    check(w, x)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_late_first_visible_key(dtype, kernel):
    """Even rows see nothing before key 300 and then scores 100 above the rest."""
    w = I.Workload("late", B=1, H=2, N=512, d=64, dtype=dtype, mask_kind="additive", std=1.0, seed=23)

    def fill(m):
        m[0::2, :300] = float("-inf")
        m[0::2, 300:] = 100.0
    x = _additive_rows(w, fill)
    check(w, x)


def test_all_4x4_bool_masks_in_one_launch():
    """All 2^16 boolean masks of a 4x4 score block as the batch axis of one launch, causal off and on."""
    B = 1 << 16
    for dtype in ("f32", "bf16"):
        w = I.Workload("mask4", B=1, H=1, N=4, d=64, dtype=dtype, std=1.0, seed=9)
        x1 = I.make_inputs(w)
        x = {n: x1[n].expand(B, 1, 4, 64).contiguous() for n in ("q", "k", "v", "tq", "tk", "tv")}
        bits = ((torch.arange(B)[:, None] >> torch.arange(16)[None, :]) & 1).to(torch.uint8)
        x["mask"] = bits.reshape(B, 1, 4, 4).contiguous()
        for causal in (False, True):
            got = gpu_run(x, causal)
            # reference: the oracle for each distinct row pattern of a query row (16 x 4), gathered
            ref = {n: np.zeros(got[n].shape) for n in got}
            base = {n: f64(x1[n]) for n in ("q", "k", "v", "tq", "tk", "tv")}
            pats = ((np.arange(16)[:, None] >> np.arange(4)[None, :]) & 1).astype(np.uint8)
            for i in range(4):
                m = np.broadcast_to(pats[:, None, None, :], (16, 1, 4, 4)).copy()
                rep = {n: np.broadcast_to(a, (16, 1) + a.shape[2:]) for n, a in base.items()}
                o, to, lse, tlse = oracle_fwd(rep["q"], rep["k"], rep["v"], rep["tq"], rep["tk"], rep["tv"],
                                              mask=m, mask_kind="bool", causal=causal)
                rowpat = (bits.numpy().reshape(B, 4, 4)[:, i, :] << np.arange(4)).sum(1)
                for n, a in (("o", o), ("to", to), ("lse", lse), ("tlse", tlse)):
                    ref[n][:, 0, i] = a[rowpat, 0, i]
            assert_parity(got, ref, dtype, f"mask4 {dtype} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_large_scores(kernel, causal, dtype):
    """Scores of a few hundred, carried by head-dim entries 24..31 and 56..63 only.

    The matrix cores accumulate a score block over four 16-wide chunks of the
    head dimension; here the first three add nothing, so a row maximum read
    before the last product has landed would be 0 while the true scores reach
    about 200: exponentials against that reference overflow. Key 0 is set to
    -q_0, so query row 0 (which sees only key 0 when causal) has the score
    -|q_0|^2 scale, about -290: a first reference far below 0, which must not
    scale the (still zero) accumulators by exp(+290). Regression test for both.
    """
    w = I.Workload("large_scores", B=1, H=2, N=300, d=64, dtype=dtype, causal=causal, std=1.0, seed=21)
    x = I.make_inputs(w)
    keep = torch.zeros(64)
    keep[24:32] = 1.0
    keep[56:64] = 1.0
    for n in ("q", "k"):
        x[n] = (x[n].float() * 12.0 * keep).to(x[n].dtype)
    x["k"][:, :, 0] = -x["q"][:, :, 0]
    got, ref = check(w, x=x)
    assert np.abs(ref["lse"]).max() > 100.0
    if causal:
        assert ref["lse"][:, :, 0].max() < -100.0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("log2_ds", [11, 13])
def test_f16_large_score_tangents(kernel, causal, log2_ds):
    """float16 score tangents of |dS| ~ 2^11 and 2^13 (dQ and dK scaled up): a weight times its score
    tangent, rounded to float16, would pass 65504 with weights kept up to 2^4 .. 2^6; the kernels
    must lower the weights instead of overflowing, and still match the oracle."""
    w = I.Workload("f16_big_ds", B=1, H=2, N=300, d=64, dtype="f16", causal=causal, std=1.0, seed=22 + log2_ds)
    x = I.make_inputs(w)
    for n in ("tq", "tk"):
        x[n] = (x[n].float() * 2.0 ** (log2_ds - 1)).to(torch.float16)
    got, ref = check(w, x=x)
    ds = 0.125 * (x["tq"].double() @ x["k"].double().transpose(-1, -2) + x["q"].double() @ x["tk"].double().transpose(-1, -2))
    assert ds.abs().max() > 2.0 ** (log2_ds + 1)
    assert np.all(np.isfinite(got["to"].numpy()))


def test_deterministic(kernel):
    w = I.Workload("det", B=2, H=4, N=300, d=64, dtype="bf16", causal=True, std=1.0, seed=10)
    x = I.make_inputs(w)
    a = gpu_run(x, True)
    b = gpu_run(x, True)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_errors_raise_and_write_nothing():
    from forward_mode_autodiff_amd.jvpattn import JvpattnError
    q = torch.randn(1, 1, 8, 48, device=DEV, dtype=torch.bfloat16)   # an unsupported head dimension
    with pytest.raises(JvpattnError) as e:
        jvpattn_fwd(q, q, q)
    assert e.value.code == -4
    q = torch.randn(1, 1, 8, 64, device=DEV, dtype=torch.bfloat16)
    out = (torch.full_like(q, 7.0), torch.full_like(q, 7.0), torch.full((1, 1, 8), 7.0, device=DEV), None)
    with pytest.raises(JvpattnError):
        jvpattn_fwd(q, q, q, scale=-1.0, out=out)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 7.0) and torch.all(out[2] == 7.0)


# ------------------------------------------------ grouped key/value heads

GQA_CASES = [
    # B*H = 32 is a multiple of 8 x 4: the launcher keeps each K/V group on one XCD
    I.Workload("gqa4_bf16_causal", B=4, H=8, Hkv=2, N=300, d=64, dtype="bf16", causal=True, std=1.0, seed=11),
    I.Workload("gqa2_f16", B=1, H=6, Hkv=3, N=200, d=64, dtype="f16", std=1.0, seed=12),
    I.Workload("mqa_bf16_bool", B=2, H=4, Hkv=1, N=160, d=64, dtype="bf16", mask_kind="bool", mask_heads=4,
               keep=0.7, std=1.0, seed=13),
    I.Workload("gqa2_d128_bf16_causal", B=1, H=4, Hkv=2, N=200, d=128, dtype="bf16", causal=True, std=1.0,
               seed=14),
    I.Workload("gqa2_f32", B=1, H=4, Hkv=2, N=100, d=64, dtype="f32", std=1.0, seed=15),
]


@pytest.mark.parametrize("w", GQA_CASES, ids=lambda w: w.name)
def test_grouped_kv_heads(w, kernel):
    check(w)


def test_grouped_kv_heads_hvp_shape_sampled(kernel):
    """B=4, H=16, Hkv=4, N=2048, d=64, bf16, causal: all heads launched, sampled heads x rows checked."""
    w = I.HVP_GQA
    x = I.make_inputs(w)
    got = gpu_run(x, True)
    heads = [(0, 0), (0, 3), (1, 6), (3, 15)]
    rows = sampled_rows(w.N, 40, 7)
    ref = oracle_run(x, "none", True, heads=heads, rows=rows)
    assert_parity(pick(got, heads, rows), ref, w.dtype, w.name, spec_spread=True)


def test_grouped_kv_heads_match_repeated_heads(kernel):
    """Sharing one K/V head gives bit-identical results to passing it once per query head."""
    w = I.Workload("gqa_vs_mha", B=2, H=8, Hkv=2, N=256, d=64, dtype="bf16", causal=True, std=1.0, seed=16)
    x = to_dev(I.make_inputs(w))
    rep = {n: x[n].repeat_interleave(4, dim=1).contiguous() for n in ("k", "v", "tk", "tv")}
    a = jvpattn_fwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], causal=True)
    b = jvpattn_fwd(x["q"], rep["k"], rep["v"], x["tq"], rep["tk"], rep["tv"], causal=True)
    torch.cuda.synchronize()
    for u, t in zip(a, b):
        assert torch.equal(u, t)


# ------------------------------------------------ workgroup order

@pytest.mark.parametrize("order", ["qb", "head"])
@pytest.mark.parametrize("w", [
    I.Workload("order_bf16_causal", B=2, H=8, N=700, d=64, dtype="bf16", causal=True, std=1.0, seed=17),
    I.Workload("order_gqa_f16", B=4, H=8, Hkv=2, N=520, d=64, dtype="f16", std=1.0, seed=18),
    I.Workload("order_d128_bf16", B=1, H=8, N=300, d=128, dtype="bf16", std=1.0, seed=19),
], ids=lambda w: w.name)
def test_block_order(w, order, kernel):
    """Both workgroup orders (heaviest query block first over all heads, or head-major per XCD) give
    the oracle's results on every kernel."""
    jvpattn_fwd_set_algo(kernel=kernel, order=order)
    check(w)


def test_wide_query_block_major_sampled():
    """B=256, H=8, N=512, d=128, bf16 in the order its grid does not take by default: sampled heads."""
    jvpattn_fwd_set_algo(order="qb")
    w = I.WIDE
    x = I.make_inputs(w)
    got = gpu_run(x, False)
    heads = [(0, 0), (17, 3), (128, 7), (255, 5)]
    rows = sampled_rows(w.N, 40, 9)
    ref = oracle_run(x, "none", False, heads=heads, rows=rows)
    assert_parity(pick(got, heads, rows), ref, w.dtype, w.name, spec_spread=True)


# ------------------------------------------------ key masks shared by all query rows

KEY_MASKS = [
    ("pad_right", "bool", False, "bf16"),
    ("pad_left", "bool", True, "f16"),
    ("window", "additive", False, "bf16"),
    ("window", "bool", True, "bf16"),
    ("pad_right", "additive", True, "f16"),
]


@pytest.mark.parametrize("skip", ["1", "0"], ids=["skip", "noskip"])
@pytest.mark.parametrize("layout,kind,causal,dtype", KEY_MASKS, ids=lambda v: str(v))
def test_key_masks(layout, kind, causal, dtype, skip, kernel):
    """[B,1,1,Nk] masks: the kernels skip the key tiles outside the visible range (or, forced, run them
    all); results as the oracle's."""
    jvpattn_fwd_set_algo(kernel=kernel, key_range=skip == "1")
    w = I.Workload(f"keymask_{layout}_{kind}", B=4, H=2, N=300, d=64, dtype=dtype, causal=causal, mask_kind=kind,
                   mask_layout=layout, std=1.0, seed=30)
    check(w)


@pytest.mark.parametrize("w", [
    # one batch hides every key (rows give O = dO = 0, lse = -inf), one keeps 5, one all, one 33
    I.Workload("keypad_lengths_bf16", B=4, H=2, N=300, d=64, dtype="bf16", mask_kind="bool",
               mask_layout="pad_right", std=1.0, seed=31, extra={"lengths": [0, 5, 300, 33]}),
    I.Workload("keymask_per_head_f16", B=2, H=4, N=257, d=64, dtype="f16", mask_kind="additive", mask_heads=4,
               mask_layout="window", std=1.0, seed=32),
    I.Workload("keymask_d128_bf16_causal", B=2, H=2, N=200, d=128, dtype="bf16", causal=True, mask_kind="bool",
               mask_layout="pad_left", std=1.0, seed=33),
    I.Workload("keymask_f32", B=2, H=2, N=150, d=64, dtype="f32", mask_kind="additive", mask_layout="window",
               std=1.0, seed=34),
    I.Workload("keymask_f32_bool_lengths", B=3, H=1, N=100, d=64, dtype="f32", mask_kind="bool",
               mask_layout="pad_left", std=1.0, seed=35, extra={"lengths": [0, 64, 7]}),
], ids=lambda w: w.name)
def test_key_mask_edges(w, kernel):
    check(w)


def test_key_padding_hvp_shape_sampled(kernel):
    """B=4, H=16, N=2048, d=64, bf16, right-padded key mask (2048/1536/1024/512 valid keys): sampled rows."""
    w = I.HVP_PAD
    x = I.make_inputs(w)
    got = gpu_run(x, False)
    heads = [(0, 0), (1, 5), (2, 9), (3, 15)]
    rows = sampled_rows(w.N, 40, 10)
    ref = oracle_run(x, "bool", False, heads=heads, rows=rows)
    assert_parity(pick(got, heads, rows), ref, w.dtype, w.name, spec_spread=True)


# ------------------------------------------------ tangent of an additive mask

def mask_tangent_for(x, seed):
    g = torch.Generator().manual_seed(seed)
    m = x["mask"]
    return torch.randn(m.shape, generator=g, dtype=torch.float32).to(m.dtype)


def check_tmask(w, seed, tangents=("tq", "tk", "tv")):
    x = I.make_inputs(w)
    tm = mask_tangent_for(x, seed)
    d = to_dev(x)
    t = {n: (d[n] if n in tangents else None) for n in ("tq", "tk", "tv")}
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], t["tq"], t["tk"], t["tv"], mask=d["mask"],
                                   causal=w.causal, tmask=tm.to(DEV))
    torch.cuda.synchronize()
    got = {"o": o.float().cpu(), "to": to.float().cpu(), "lse": lse.cpu(), "tlse": tlse.cpu()}
    tq, tk, tv = (f64(x[n]) if n in tangents else None for n in ("tq", "tk", "tv"))
    r = oracle_fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), tq, tk, tv, mask=f64(x["mask"]), mask_kind="additive",
                   causal=w.causal, tmask=f64(tm))
    assert_parity(got, dict(zip(("o", "to", "lse", "tlse"), r)), w.dtype, w.name, spec_spread=w.std is None)


@pytest.mark.parametrize("w", [
    I.Workload("tmask_f16", B=2, H=2, N=200, d=64, dtype="f16", mask_kind="additive", std=1.0, seed=40),
    I.Workload("tmask_bf16_causal_per_head", B=1, H=3, N=177, d=64, dtype="bf16", causal=True,
               mask_kind="additive", mask_heads=3, std=1.0, seed=41),
    I.Workload("tmask_keywindow_bf16", B=4, H=2, N=300, d=64, dtype="bf16", mask_kind="additive",
               mask_layout="window", std=1.0, seed=42),
    I.Workload("tmask_d128_bf16", B=1, H=2, N=160, d=128, dtype="bf16", mask_kind="additive", std=1.0, seed=43),
    I.Workload("tmask_f32", B=1, H=2, N=100, d=64, dtype="f32", mask_kind="additive", std=1.0, seed=44),
    I.Workload("tmask_masked_spec", B=2, H=8, N=1024, d=64, dtype="f16", mask_kind="additive", seed=2),
], ids=lambda w: w.name)
def test_additive_mask_tangent(w, kernel):
    check_tmask(w, seed=w.seed + 100)


def test_additive_mask_tangent_alone(kernel):
    """Only the mask moves: dO = sum_j P (dM - tlse) V."""
    w = I.Workload("tmask_only", B=2, H=2, N=150, d=64, dtype="bf16", mask_kind="additive", std=1.0, seed=45)
    check_tmask(w, seed=145, tangents=())


def test_zero_mask_tangent_is_bit_identical(kernel):
    w = I.Workload("tmask_zero", B=2, H=4, N=260, d=64, dtype="f16", mask_kind="additive", std=1.0, seed=46)
    d = to_dev(I.make_inputs(w))
    a = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=d["mask"])
    b = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=d["mask"],
                    tmask=torch.zeros_like(d["mask"]))
    torch.cuda.synchronize()
    for u, t in zip(a, b):
        assert torch.equal(u, t)


# ------------------------------------------------ bit-packed boolean masks

@pytest.mark.parametrize("w", [
    I.Workload("bits_full_f16", B=2, H=2, N=200, d=64, dtype="f16", mask_kind="bool", keep=0.7, std=1.0, seed=50),
    I.Workload("bits_per_head_bf16_causal", B=1, H=3, N=257, d=64, dtype="bf16", causal=True, mask_kind="bool",
               mask_heads=3, keep=0.6, std=1.0, seed=51),
    I.Workload("bits_keypad_bf16", B=4, H=2, N=300, d=64, dtype="bf16", mask_kind="bool", mask_layout="pad_right",
               std=1.0, seed=52, extra={"lengths": [0, 5, 300, 33]}),
    I.Workload("bits_d128_bf16", B=1, H=2, N=150, d=128, dtype="bf16", mask_kind="bool", keep=0.8, std=1.0,
               seed=53),
    I.Workload("bits_f32_window", B=2, H=2, N=100, d=64, dtype="f32", mask_kind="bool", mask_layout="window",
               std=1.0, seed=54),
    I.Workload("bits_masked_spec", B=2, H=8, N=1024, d=64, dtype="f16", mask_kind="bool", seed=2),
], ids=lambda w: w.name)
def test_bit_packed_masks(w, kernel):
    """A bit-packed mask gives the bool mask's results to within one rounding of each output (the two
    builds are separate code, which the compiler may contract into fused multiply-adds differently),
    and the oracle's."""
    from forward_mode_autodiff_amd.jvpattn import pack_mask_bits
    x = I.make_inputs(w)
    d = to_dev(x)
    bits = pack_mask_bits(d["mask"])
    a = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=d["mask"], causal=w.causal)
    b = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=bits, causal=w.causal,
                    mask_kind="bits")
    torch.cuda.synchronize()
    for u, t in zip(a, b):
        fin = torch.isfinite(u)
        assert torch.equal(fin, torch.isfinite(t)) and torch.equal(u[~fin], t[~fin])
        ulp = torch.finfo(u.dtype).eps * float(u[fin].abs().max()) if fin.any() else 0.0
        diff = (u[fin].float() - t[fin].float()).abs()
        assert (float(diff.max()) if diff.numel() else 0.0) <= 2 * ulp
    got = {"o": b[0].float().cpu(), "to": b[1].float().cpu(), "lse": b[2].cpu(), "tlse": b[3].cpu()}
    r = oracle_fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["tq"]), f64(x["tk"]), f64(x["tv"]),
                   mask=bits.cpu().numpy(), mask_kind="bits", causal=w.causal)
    assert_parity(got, dict(zip(("o", "to", "lse", "tlse"), r)), w.dtype, w.name, spec_spread=w.std is None)


# ------------------------------------------------ features combined

def test_grouped_heads_with_packed_key_padding(kernel):
    """Shared K/V heads, a bit-packed key-padding mask (with an empty batch) and causality at once."""
    from forward_mode_autodiff_amd.jvpattn import pack_mask_bits
    w = I.Workload("combo_gqa_bits", B=4, H=8, Hkv=2, N=260, d=64, dtype="bf16", causal=True, mask_kind="bool",
                   mask_layout="pad_left", std=1.0, seed=60, extra={"lengths": [260, 0, 97, 33]})
    x = I.make_inputs(w)
    d = to_dev(x)
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=pack_mask_bits(d["mask"]),
                                   mask_kind="bits", causal=True)
    torch.cuda.synchronize()
    got = {"o": o.float().cpu(), "to": to.float().cpu(), "lse": lse.cpu(), "tlse": tlse.cpu()}
    ref = oracle_run(x, "bool", True)
    assert_parity(got, ref, w.dtype, w.name, spec_spread=False)


def test_grouped_heads_with_mask_tangent_per_head(kernel):
    """Shared K/V heads with a per-head additive mask and its tangent."""
    w = I.Workload("combo_gqa_tmask", B=2, H=4, Hkv=1, N=190, d=64, dtype="f16", mask_kind="additive", mask_heads=4,
                   std=1.0, seed=61)
    check_tmask(w, seed=161)


# ------------------------------------------------ structured per-row masks (hidden 32 x 32 blocks skipped)

ROW_MASKS = [
    ("sliding", {"window": 70}, "bool", False, "bf16"),
    ("sliding", {"window": 45}, "bits", True, "f16"),
    ("blockdiag", {"block": 96}, "additive", False, "bf16"),
    ("blockdiag", {"block": 128}, "bool", True, "f16"),
    ("sliding", {"window": 100}, "additive", True, "f16"),
]


@pytest.mark.parametrize("layout,extra,kind,causal,dtype", ROW_MASKS, ids=lambda v: str(v))
def test_structured_row_masks_skip_hidden_blocks(layout, extra, kind, causal, dtype, kernel):
    """Sliding-window and block-diagonal masks per query row: workgroups run only the key tiles some
    of their rows see, and waves skip the 32 x 32 blocks the mask hides from all their rows. Results
    match the oracle with the early-outs on and off, and are equal bit for bit (a hidden block adds
    exact zeros) -- except on the split-key kernels, whose split point moves with the tile range."""
    from forward_mode_autodiff_amd.jvpattn import pack_mask_bits
    w = I.Workload(f"rowmask_{layout}_{kind}", B=2, H=2, N=420, d=64, dtype=dtype, causal=causal,
                   mask_kind="bool" if kind == "bits" else kind, mask_layout=layout, std=1.0, seed=36, extra=extra)
    x = I.make_inputs(w)
    d = to_dev(x)
    m = pack_mask_bits(d["mask"]) if kind == "bits" else d["mask"]
    mk = "bits" if kind == "bits" else None
    runs = []
    for skip in (True, False):
        jvpattn_fwd_set_algo(kernel=kernel, key_range=skip)
        o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=m, causal=causal,
                                       mask_kind=mk)
        torch.cuda.synchronize()
        runs.append((o.clone(), to.clone(), lse.clone(), tlse.clone()))
    if kernel in ("pp", "wg4"):
        for a, b in zip(*runs):
            assert torch.equal(a, b)
    ref = oracle_run(x, "bool" if kind == "bits" else kind, causal)
    for o, to, lse, tlse in runs:
        got = {"o": o.float().cpu(), "to": to.float().cpu(), "lse": lse.cpu(), "tlse": tlse.cpu()}
        assert_parity(got, ref, dtype, w.name, spec_spread=False)
