"""Throughput of the fused attention forward with tangents on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload hvp] [--no-cpu-baseline]

A step is one jvpattn_fwd call (scores, score tangents, online softmax with
tangent, the value products, epilogue, lse/tlse) over one batch of synthetic
inputs already resident in HBM. The default workload is B=4, H=16, N=2048,
d=64, bfloat16, causal. Throughput counts 12*N^2*d flops per head (half when
causal). A workload name with the suffix "_bwd" (e.g. hvp_bwd) times one
jvpattn_bwd call instead (the reverse pass for the same inputs and N(0,1)
cotangents), counting 30*N^2*d flops per head. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}   # MI355X dense matrix peak per dtype
HBM_GBS = 8000.0
METRIC = "JVP-attention fwd TFLOP/s (12·N²·d/head) and % MFMA peak, N=2048 d=64 bf16"
METRIC_BWD = "JVP-attention reverse pass TFLOP/s (30·N²·d/head) and % MFMA peak, N=2048 d=64 bf16"
ROOT = os.path.dirname(os.path.abspath(__file__))


def workloads():
    from forward_mode_autodiff_amd import inputs as I
    return {
        "hvp": I.HVP,
        "hvp_gqa4": I.HVP_GQA,
        "hvp_keypad": I.HVP_PAD,
        "hvp_full": I.Workload("hvp_full", B=4, H=16, N=2048, d=64, dtype="bf16", causal=False, seed=4),
        # the HVP shape under structured per-row masks (per-row [B,1,N,N] bool): a sliding window of
        # 256 keys each side, and 512-key diagonal blocks (packed sequences); non-causal
        "hvp_window": I.Workload("hvp_window", B=4, H=16, N=2048, d=64, dtype="bf16", seed=9, mask_kind="bool",
                                 mask_layout="sliding", extra={"window": 256}),
        "hvp_blockdiag": I.Workload("hvp_blockdiag", B=4, H=16, N=2048, d=64, dtype="bf16", seed=10,
                                    mask_kind="bool", mask_layout="blockdiag", extra={"block": 512}),
        "seq2048": I.seq(2048, False),
        "seq2048_causal": I.seq(2048, True),
        "seq2048_bf16": I.seq(2048, False, dtype="bf16"),
        "masked_bool": I.MASKED_BOOL,
        "masked_additive": I.MASKED_ADD,
        "wide": I.WIDE,
        # the HVP shape at the other head dimensions (d = 32 and 96 run padded d = 64 / 128 kernels)
        "hvp_d32": I.Workload("hvp_d32", B=4, H=16, N=2048, d=32, dtype="bf16", causal=True, seed=11),
        "hvp_d96": I.Workload("hvp_d96", B=4, H=16, N=2048, d=96, dtype="bf16", causal=True, seed=12),
        "hvp_d128": I.Workload("hvp_d128", B=4, H=16, N=2048, d=128, dtype="bf16", causal=True, seed=13),
        "hvp_d256": I.Workload("hvp_d256", B=4, H=16, N=2048, d=256, dtype="bf16", causal=True, seed=14),
        "tiny": I.TINY,
    }


# Work conventions of the throughput figures, per head: the forward's six products of
# Nq x Nk x d multiply-adds (S = Q K^T; the score tangent dQ K^T + Q dK^T; P V; (P dS) V; P dV) are
# 12 Nq Nk d flops; the reverse pass's fifteen are 30 Nq Nk d. Causal work is counted as half.
FWD_PRODUCTS, BWD_PRODUCTS = 6, 15


def fwd_flops(B, H, Nq, Nk, d, causal):
    """Forward work convention: 12 Nq Nk d flops per head, halved when causal."""
    f = 2.0 * FWD_PRODUCTS * Nq * Nk * d * B * H
    return f / 2.0 if causal else f


def bwd_flops(B, H, Nq, Nk, d, causal):
    """Reverse-pass work convention: 30 Nq Nk d flops per head, halved when causal."""
    f = 2.0 * BWD_PRODUCTS * Nq * Nk * d * B * H
    return f / 2.0 if causal else f


def algorithmic_bytes(w):
    """Bytes a launch must move at least: 6 inputs + 2 outputs + lse/tlse, the mask read once per batch."""
    es = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    per_q_head = 4 * w.N * w.d * es + 8 * w.N          # q, tq, o, to, lse, tlse
    per_kv_head = 4 * w.nk * w.d * es                   # k, v, tk, tv (shared by grouped query heads)
    mask = 0
    if w.mask_kind != "none":
        mes = 1 if w.mask_kind == "bool" else es
        # key masks: one row shared by all queries; the others hold one row per query
        rows = 1 if w.mask_layout in ("pad_right", "pad_left", "window") else w.N
        mask = w.B * w.mask_heads * rows * w.nk * mes
    return w.B * w.H * per_q_head + w.B * w.hkv * per_kv_head + mask


# The forward's device sources and build flags: a counter summary taken before any of them changed
# no longer describes the kernel.
KERNEL_SOURCES = [os.path.join(ROOT, "forward_mode_autodiff_amd", f)
                  for f in ("csrc/jvpattn_fwd.hip", "csrc/jvpattn_fwd_inst.hip", "csrc/jvpattn_fwd_kernels.h",
                            "csrc/jvpattn_fwd_launch.h", "csrc/jvpattn_device.h", "build.py")]


def measured_traffic(workload):
    """HBM bytes per launch from the committed counter summary of this workload (profiles/<kernel>__<workload>.txt),
    or None if absent or the kernel changed since (the summary records a hash of the forward's sources)."""
    import glob
    import hashlib
    found = glob.glob(os.path.join(ROOT, "profiles", f"*__{workload}.txt"))
    if len(found) != 1:
        return None
    path = found[0]
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    sha = hashlib.sha256(b"".join(open(f, "rb").read() for f in KERNEL_SOURCES)).hexdigest()[:16]
    if fields.get("kernel_source_sha256_16") != sha or "traffic_bytes_per_launch" not in fields:
        return None
    return int(float(fields["traffic_bytes_per_launch"]))


def cpu_baseline_bwd(w, x, budget_s=12.0):
    """Time the float64 reverse-pass oracle on whole heads of the same workload for ~budget_s."""
    from threadpoolctl import threadpool_info

    from oracle import oracle_bwd
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    grp = w.H // w.hkv
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b, h = heads[done % len(heads)]
        f64 = lambda t: t[b:b + 1, h:h + 1].double().numpy()
        f64k = lambda t: t[b:b + 1, h // grp:h // grp + 1].double().numpy()   # the K/V head h reads
        mask = None
        if x["mask"] is not None:
            mask = x["mask"][b:b + 1, :1].double().numpy() if w.mask_kind == "additive" else \
                x["mask"][b:b + 1, :1].numpy()
        oracle_bwd(f64(x["q"]), f64k(x["k"]), f64k(x["v"]), f64(x["tq"]), f64k(x["tk"]), f64k(x["tv"]),
                   f64(x["do"]), f64(x["dto"]), mask=mask, mask_kind=w.mask_kind, causal=w.causal)
        done += 1
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": bwd_flops(1, done, w.N, w.nk, w.d, w.causal) / dt / 1e12, "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{done} head evaluations (of {len(heads)} heads) of the same workload's reverse pass, "
                      f"float64 numpy, {dt:.1f} s"}


def cpu_baseline(w, x, budget_s=12.0):
    """Time the float64 oracle on whole heads of the same workload (cycling over the heads) for ~budget_s."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import oracle_fwd
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    grp = w.H // w.hkv
    f64 = lambda t: t[b:b + 1, h:h + 1].double().numpy()
    f64k = lambda t: t[b:b + 1, h // grp:h // grp + 1].double().numpy()   # the K/V head h reads
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b, h = heads[done % len(heads)]
        mask = None
        if x["mask"] is not None:
            mask = x["mask"][b:b + 1, :1].double().numpy() if w.mask_kind == "additive" else \
                x["mask"][b:b + 1, :1].numpy()
        oracle_fwd(f64(x["q"]), f64k(x["k"]), f64k(x["v"]), f64(x["tq"]), f64k(x["tk"]), f64k(x["tv"]),
                   mask=mask, mask_kind=w.mask_kind, causal=w.causal)
        done += 1
    dt = time.perf_counter() - t0
    flops = fwd_flops(1, done, w.N, w.nk, w.d, w.causal)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} head evaluations (of {len(heads)} heads) of the same workload, all {w.N} "
                      f"query rows each, float64 numpy, {dt:.1f} s"}


def bwd_step_setup(w, x, dev):
    """Device inputs, forward outputs and output buffers for timing jvpattn_bwd."""
    import torch

    from forward_mode_autodiff_amd.jvpattn import jvpattn_bwd, jvpattn_bwd_workspace_bytes, jvpattn_fwd, make_params
    d = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    o, to, lse, tlse = jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=d["mask"],
                                   causal=w.causal)
    outs = tuple(torch.empty_like(d[n]) for n in ("q", "k", "v", "q", "k", "v"))
    params, _ = make_params(d["q"], d["k"], d["mask"], w.causal)
    ws = torch.empty(max(jvpattn_bwd_workspace_bytes(params), 1), dtype=torch.uint8, device=dev)

    def step():
        jvpattn_bwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], o, to, lse, tlse, d["do"], d["dto"],
                    mask=d["mask"], causal=w.causal, out=outs, workspace=ws)
    return step


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clock settles under sustained matrix-core load only after a few
    # hundred launches (~30 ms); the defaults time the steady state.
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="hvp")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, copy a 256 MiB buffer twice (known bytes, for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the forward shards "
              f"over batch*heads with no exchange, so N GPUs run N independent copies)", file=sys.stderr)
        sys.exit(2)

    import torch

    from forward_mode_autodiff_amd import inputs as I
    from forward_mode_autodiff_amd.jvpattn import jvpattn_fwd, load_library
    load_library()
    reverse = args.workload.endswith("_bwd")
    w = workloads()[args.workload[:-4] if reverse else args.workload]
    x = I.make_inputs(w, cotangents=reverse)
    dev = "cuda:0"
    d = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    o = torch.empty_like(d["q"])
    to = torch.empty_like(d["q"])
    lse = torch.empty(d["q"].shape[:3], device=dev, dtype=torch.float32)
    tlse = torch.empty_like(lse)
    out = (o, to, lse, tlse)

    def step():
        jvpattn_fwd(d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], mask=d["mask"], causal=w.causal,
                    out=out)

    if reverse:
        step = bwd_step_setup(w, x, dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # K back-to-back launches between two events on the launch stream (torch's
    # current stream); nothing is recorded between launches, so the average
    # launch duration is the region's time over K.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    avg_launch_ms = total_ms / args.steps

    flops = (bwd_flops if reverse else fwd_flops)(w.B, w.H, w.N, w.nk, w.d, w.causal)
    ms_per_step = total_ms / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    rec = {
        "metric": METRIC_BWD if reverse else METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name + ("_bwd" if reverse else ""), "B": w.B, "H": w.H, "Hkv": w.hkv,
                   "N": w.N, "d": w.d,
                   "causal": w.causal, "mask": w.mask_kind, "input_std": round(w.sigma, 6)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": None if reverse else measured_traffic(args.workload)},
        "launch_us": round(avg_launch_ms * 1e3, 2),
        "algorithmic_GBps": None if reverse else round(algorithmic_bytes(w) / (avg_launch_ms * 1e-3) / 1e9, 1),
        "wall_s": round(wall, 4),
    }
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = 256 << 20
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_bwd(w, x) if reverse else cpu_baseline(w, x)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
