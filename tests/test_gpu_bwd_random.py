"""Reverse pass on seeded random small shapes: both stream modes give the same bits, and oracle parity.

Each case draws batch, heads, grouping, lengths (ragged, Nq != Nk), head dimension, type, causal
limit and mask from a fixed seed, so combinations the hand-written cases miss get run too. The
query side runs beside the key side on a second stream in one call and after it on one stream in the
other; the results must agree bit for bit and stay within the per-element bar (tests/parity.py) of
the float64 oracle.
"""
import numpy as np
import pytest

from forward_mode_autodiff_amd import inputs as I
from forward_mode_autodiff_amd.jvpattn import jvpattn_bwd_set_overlap
from tests.bwd_cases import magnitudes, reference
from tests.parity import BWD_NAMES as NAMES, bwd_failures
from tests.test_gpu_bwd import gpu_bwd

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 64, 128]))
    dtype = str(rng.choice(["bf16", "f16"] + (["f32"] if d == 64 else [])))
    hkv = int(rng.choice([1, 2]))
    h = hkv * int(rng.choice([1, 2, 3]))
    n = int(rng.integers(1, 300))
    nk = n if rng.random() < 0.5 else int(rng.integers(1, 300))
    kind = str(rng.choice(["none", "none", "bool", "additive"]))
    kw = {}
    if kind != "none":
        kw = dict(mask_kind=kind, mask_heads=int(rng.choice([1, h])), keep=float(rng.uniform(0.3, 0.95)))
    return I.Workload(f"rand{seed}", B=int(rng.integers(1, 3)), H=h, Hkv=hkv, N=n, Nk=nk, d=d, dtype=dtype,
                      causal=bool(rng.random() < 0.5), std=1.0, seed=seed, **kw)


@pytest.fixture
def _overlap_auto():
    yield
    jvpattn_bwd_set_overlap()


@pytest.mark.parametrize("seed", range(600, 616))
def test_random_shapes_both_stream_modes(seed, _overlap_auto):
    w = draw(seed)
    x = I.make_inputs(w, cotangents=True)
    jvpattn_bwd_set_overlap(False)
    one = gpu_bwd(x, w)
    jvpattn_bwd_set_overlap(True)
    two = gpu_bwd(x, w)
    for n in NAMES:
        assert np.array_equal(one[n], two[n]), (w, n)
    bad = bwd_failures(two, reference(x, w), magnitudes(x, w), w.dtype)
    assert not bad, f"{w}: " + "; ".join(bad)
