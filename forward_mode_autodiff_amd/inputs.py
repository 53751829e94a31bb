"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

Holds no arithmetic of the attention method: it only draws random tensors.

Distribution: every input tensor is i.i.d. normal times ``std``; the default
``std = 1/sqrt(d)`` follows the data generator in the equinox issue
"Flash Attention" (#732), which draws (batch, heads, seq, dim) normals scaled
by one over the square root of the embedding size. Values are drawn in float32
from a CPU ``torch.Generator`` and then rounded (round-to-nearest-even) to the
working dtype, so the GPU and the oracle see identical values.

Draw order (fixed): q, k, v, tq, tk, tv, then the boolean mask, the additive
mask, then the cotangents do, dto.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """A named attention problem: shapes, dtype, masking and input spread."""
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool = False
    mask_kind: str = "none"        # "none" | "bool" | "additive"
    std: float | None = None       # None -> 1/sqrt(d)
    seed: int = 0
    Nk: int | None = None          # None -> N (self-attention)
    mask_heads: int = 1            # mask head extent (1 = broadcast over heads)
    keep: float = 0.9              # Bernoulli keep rate of the boolean mask
    Hkv: int | None = None         # key/value heads (None -> H; fewer = grouped-query attention)
    # Mask layout: "bernoulli" (independent keep draws per element, diagonal
    # kept); a key mask shared by all query rows ([B, mask_heads, 1, Nk]):
    # "pad_right" (keys below a drawn length visible), "pad_left" (the last
    # drawn-length keys visible), "window" (a drawn contiguous key range); or
    # a structured mask per query row ([B, mask_heads, N, Nk]): "sliding"
    # (key j visible to query i iff |i - j| < extra["window"]) and
    # "blockdiag" (iff i // extra["block"] == j // extra["block"], packed
    # sequences).
    mask_layout: str = "bernoulli"
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def nk(self) -> int:
        return self.N if self.Nk is None else self.Nk

    @property
    def hkv(self) -> int:
        return self.H if self.Hkv is None else self.Hkv

    @property
    def sigma(self) -> float:
        return 1.0 / math.sqrt(self.d) if self.std is None else self.std


# The five workloads the method is measured on, plus the seq-length sweep.
TINY = Workload("tiny", B=1, H=2, N=32, d=64, dtype="f32", seed=0)
SEQ_NS = (32, 64, 128, 256, 512, 1024, 2048)


def seq(N: int, causal: bool, dtype: str = "f16", seed: int = 1) -> Workload:
    return Workload(f"seq_N{N}_{'causal' if causal else 'full'}_{dtype}", B=2, H=8, N=N, d=64,
                    dtype=dtype, causal=causal, seed=seed)


MASKED_BOOL = Workload("masked_bool", B=2, H=8, N=1024, d=64, dtype="f16", mask_kind="bool", seed=2)
MASKED_ADD = Workload("masked_additive", B=2, H=8, N=1024, d=64, dtype="f16", mask_kind="additive",
                      seed=2)
WIDE = Workload("wide", B=256, H=8, N=512, d=128, dtype="bf16", seed=3)
HVP = Workload("hvp", B=4, H=16, N=2048, d=64, dtype="bf16", causal=True, seed=4)
# The HVP shape with grouped key/value heads (4 query heads per K/V head).
HVP_GQA = Workload("hvp_gqa4", B=4, H=16, N=2048, d=64, dtype="bf16", causal=True, seed=6, Hkv=4)
# The HVP shape, non-causal, with a right-padded key mask: 2048, 1536, 1024, 512 valid keys.
HVP_PAD = Workload("hvp_keypad", B=4, H=16, N=2048, d=64, dtype="bf16", seed=7, mask_kind="bool",
                   mask_layout="pad_right", extra={"lengths": [2048, 1536, 1024, 512]})


def key_mask(w: Workload, g: torch.Generator) -> torch.Tensor:
    """Boolean [B, mask_heads, 1, Nk] key mask of layout w.mask_layout (True = visible).

    Lengths and window ends are drawn uniformly; ``w.extra["lengths"]`` (one
    per batch x mask head) fixes the visible lengths instead, 0 hiding every key.
    """
    n = w.B * w.mask_heads
    j = torch.arange(w.nk)
    fixed = w.extra.get("lengths")
    if fixed is not None:
        lens = torch.tensor(fixed, dtype=torch.int64).reshape(n)
    else:
        lens = torch.randint(1, w.nk + 1, (n,), generator=g)
    if w.mask_layout == "pad_right":
        keep = j[None, :] < lens[:, None]
    elif w.mask_layout == "pad_left":
        keep = j[None, :] >= (w.nk - lens)[:, None]
    elif w.mask_layout == "window":
        start = (torch.rand((n,), generator=g) * (w.nk - lens + 1).float()).long()
        keep = (j[None, :] >= start[:, None]) & (j[None, :] < (start + lens)[:, None])
    else:
        raise ValueError(f"unknown mask layout {w.mask_layout!r}")
    return keep.reshape(w.B, w.mask_heads, 1, w.nk)


def make_inputs(w: Workload, cotangents: bool = False) -> dict:
    """Draw the inputs of workload ``w`` on the CPU.

    Returns a dict of CPU tensors: q, k, v, tq, tk, tv in the working dtype
    ([B,H,N,d] / [B,Hkv,Nk,d]); ``mask`` ([B, mask_heads, N, Nk], or
    [B, mask_heads, 1, Nk] for the key-mask layouts; uint8 with 1 = attend for
    "bool", the working dtype for "additive" (-inf hides a key); None for "none");
    and when ``cotangents`` is set, ``do`` and ``dto`` (i.i.d. N(0,1)).
    """
    dt = DTYPES[w.dtype]
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    qshape = (w.B, w.H, w.N, w.d)
    kshape = (w.B, w.hkv, w.nk, w.d)
    out = {}
    for name, shape in (("q", qshape), ("k", kshape), ("v", kshape),
                        ("tq", qshape), ("tk", kshape), ("tv", kshape)):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        x.mul_(w.sigma)
        out[name] = x.to(dt)
    mask = None
    if w.mask_kind not in ("none", "bool", "additive"):
        raise ValueError(f"unknown mask kind {w.mask_kind!r}")
    if w.mask_kind != "none" and w.mask_layout in ("sliding", "blockdiag"):
        i = torch.arange(w.N)[:, None]
        j = torch.arange(w.nk)[None, :]
        if w.mask_layout == "sliding":
            keep = (i - j).abs() < int(w.extra["window"])
        else:
            keep = (i // int(w.extra["block"])) == (j // int(w.extra["block"]))
        keep = keep.expand(w.B, w.mask_heads, w.N, w.nk)
        if w.mask_kind == "bool":
            mask = keep.to(torch.uint8).contiguous()
        else:
            vals = torch.randn(keep.shape, generator=g, dtype=torch.float32)
            mask = torch.where(keep, vals, torch.full_like(vals, -math.inf)).to(dt)
    elif w.mask_kind != "none" and w.mask_layout != "bernoulli":
        keep = key_mask(w, g)
        if w.mask_kind == "bool":
            mask = keep.to(torch.uint8)
        else:
            vals = torch.randn(keep.shape, generator=g, dtype=torch.float32)
            mask = torch.where(keep, vals, torch.full_like(vals, -math.inf)).to(dt)
    elif w.mask_kind == "bool":
        mshape = (w.B, w.mask_heads, w.N, w.nk)
        keep = torch.rand(mshape, generator=g, dtype=torch.float32) < w.keep
        n = min(w.N, w.nk)
        idx = torch.arange(n)
        keep[:, :, idx, idx] = True     # every query keeps at least its own key
        mask = keep.to(torch.uint8)
    elif w.mask_kind == "additive":
        mshape = (w.B, w.mask_heads, w.N, w.nk)
        mask = torch.randn(mshape, generator=g, dtype=torch.float32).to(dt)
    out["mask"] = mask
    if cotangents:
        out["do"] = torch.randn(qshape, generator=g, dtype=torch.float32).to(dt)
        out["dto"] = torch.randn(qshape, generator=g, dtype=torch.float32).to(dt)
    return out
