"""The library under HIP graph capture: a captured forward + reverse pass replays to the eager bits.

Callers that capture their step into a graph (torch.cuda.graph over the current stream) get the
same kernels on the capturing stream; the reverse pass never takes its second stream there (the
eager run below does, for grouped heads). Each graph is replayed several times, with eager work on
the same buffers and host synchronisations between replays, and every replay is compared with the
eager results bit for bit. Nothing here allocates inside the library.
"""
import pytest
import torch

from forward_mode_autodiff_amd import inputs as I
from forward_mode_autodiff_amd.jvpattn import (jvpattn_bwd, jvpattn_bwd_workspace_bytes, jvpattn_fwd,
                                              make_params)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CASES = {
    "mha-causal-bf16": dict(B=2, H=4, N=520, d=64, dtype="bf16", causal=True),
    "gqa-causal-f16": dict(B=2, H=8, Hkv=2, N=300, d=64, dtype="f16", causal=True),
    "gqa-d128-bf16": dict(B=1, H=4, Hkv=2, N=200, Nk=260, d=128, dtype="bf16"),
    # the HVP shape: ping-pong forward, walking key side, two-per-CU query side
    "hvp-shape": dict(B=4, H=16, N=2048, d=64, dtype="bf16", causal=True),
    # Wide-like d = 128 rows: the walking d = 128 forward
    "d128-walk": dict(B=16, H=8, N=512, d=128, dtype="bf16"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_captured_forward_and_reverse_replay_eager_bits(name):
    w = I.Workload(f"graph_{name}", std=1.0, seed=95, **CASES[name])
    x = {k: (None if v is None else v.to(DEV)) for k, v in I.make_inputs(w, cotangents=True).items()}
    q, k, v, tq, tk, tv = (x[n] for n in ("q", "k", "v", "tq", "tk", "tv"))
    fwd_out = (torch.empty_like(q), torch.empty_like(q), torch.empty(q.shape[:3], device=DEV),
               torch.empty(q.shape[:3], device=DEV))
    bwd_out = tuple(torch.empty_like(t) for t in (q, k, v, q, k, v))
    params, _ = make_params(q, k, None, w.causal)
    ws = torch.empty(max(jvpattn_bwd_workspace_bytes(params), 1), dtype=torch.uint8, device=DEV)

    def step():
        o, to, lse, tlse = jvpattn_fwd(q, k, v, tq, tk, tv, causal=w.causal, out=fwd_out)
        jvpattn_bwd(q, k, v, tq, tk, tv, o, to, lse, tlse, x["do"], x["dto"], causal=w.causal, out=bwd_out,
                    workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in fwd_out + bwd_out]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on a side stream, as torch asks before a capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in fwd_out + bwd_out:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager, fwd_out + bwd_out)):
            assert torch.equal(a, b), (rep, i)
        step()   # eager work on the same buffers between replays
        torch.cuda.synchronize()
