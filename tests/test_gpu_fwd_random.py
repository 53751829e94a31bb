"""Forward on seeded random small shapes, on the library's own plan and on every forced kernel family.

Each case draws batch, heads, grouping, lengths (ragged, Nq != Nk), head dimension (32 ... 256),
type, causal limit, mask kind and layout from a fixed seed; every kernel family that runs the case
must give results within the forward's bar (tests/parity.py) of the float64 oracle.
"""
import numpy as np
import pytest

from forward_mode_autodiff_amd import inputs as I
from forward_mode_autodiff_amd.jvpattn import jvpattn_fwd_set_algo
from tests.parity import assert_parity
from tests.test_gpu_fwd import gpu_run, oracle_run

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([32, 64, 64, 96, 128, 256]))
    types = ["bf16", "f16"] + (["f32"] if d in (64, 128) else [])
    dtype = str(rng.choice(types))
    hkv = int(rng.choice([1, 2]))
    h = hkv * int(rng.choice([1, 2, 4]))
    n = int(rng.integers(1, 400))
    nk = n if rng.random() < 0.5 else int(rng.integers(1, 400))
    kind = str(rng.choice(["none", "none", "bool", "additive"]))
    kw = {}
    if kind != "none":
        kw = dict(mask_kind=kind, mask_heads=int(rng.choice([1, h])), keep=float(rng.uniform(0.2, 0.95)))
    return I.Workload(f"frand{seed}", B=int(rng.integers(1, 3)), H=h, Hkv=hkv, N=n, Nk=nk, d=d, dtype=dtype,
                      causal=bool(rng.random() < 0.5), std=1.0, seed=seed, **kw)


@pytest.fixture(autouse=True)
def _automatic_plan():
    jvpattn_fwd_set_algo()
    yield
    jvpattn_fwd_set_algo()


@pytest.mark.parametrize("seed", range(700, 724))
def test_random_shapes_every_family(seed):
    w = draw(seed)
    x = I.make_inputs(w)
    ref = oracle_run(x, w.mask_kind, w.causal)
    for kernel in (None, "pp", "wg4", "split", "split64"):
        jvpattn_fwd_set_algo(kernel=kernel)
        got = gpu_run(x, w.causal)
        assert_parity(got, ref, w.dtype, f"{w} kernel={kernel}", spec_spread=False)
