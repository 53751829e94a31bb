"""Build libjvpattn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m forward_mode_autodiff_amd.build [--verbose]

Objects go to forward_mode_autodiff_amd/_build/, the library to
forward_mode_autodiff_amd/libjvpattn.so. Every call recompiles.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libjvpattn.so")
ARCH = "gfx950"

# (source, object name, extra defines): the forward's kernel instances build
# once per (mask kind, causal) pair so the objects compile in parallel.
MASK_KINDS = {"none": 0, "bool": 1, "add": 2, "bits": 3, "addt": 4}
SOURCES = [("jvpattn_fwd.hip", "jvpattn_fwd", []), ("jvpattn_bwd.hip", "jvpattn_bwd", []),
           ("jvpattn_check.cpp", "jvpattn_check", [])] + [
    ("jvpattn_fwd_inst.hip", f"jvpattn_fwd_{fam}{name}_{'causal' if c else 'full'}",
     [f"-DJVPATTN_INST_MASK={kind}", f"-DJVPATTN_INST_CAUSAL={c}", f"-DJVPATTN_INST_FAMILY={f}"])
    for f, fam in ((0, ""), (1, "s64_"), (2, "pp_"), (3, "w128_"), (4, "w256_")) for name, kind in MASK_KINDS.items()
    for c in (1, 0)] + [
    ("jvpattn_bwd_inst.hip", f"jvpattn_bwd_d{d}_{side}", [f"-DJVPATTN_BWD_D={d}", f"-DJVPATTN_BWD_PART={part}"])
    for d in (64, 128) for part, side in ((0, "dkv"), (1, "dq"))]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Device code: gfx950 only; packed fp32 instructions disabled.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]
# The matrix products take their accumulators in VGPRs where the register
# budget allows (amdgpu-mfma-vgpr-form): loop-carried accumulators then stop
# bouncing between AGPRs and VGPRs, and the forward's d = 128 / 256 kernels
# and the reverse pass's masked ones no longer spill (the d = 64 ping-pong
# kernel's code is unchanged by it). The reverse pass's d = 128 key-side
# object builds without it: the compiler fails on two of its instances.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
VGPR_FORM_OBJECTS = ("jvpattn_fwd", "jvpattn_bwd_d64", "jvpattn_bwd_d128_dq")
# The compiler's iterative ILP scheduling strategy for the reverse pass (every
# object): 2-16% faster per 16-bit call (most with masks), the same bits. It
# makes the masked d = 64 key-side and the float32 instances keep 20-56 bytes
# per lane in scratch (the masked d = 128 key side 276-280 instead of
# 188-304), and the masked ones still measured faster; float32 without a mask
# is ~4% slower. In the forward
# it suits the ping-pong kernel with a bool or additive mask (1-4% faster, no
# scratch) and the 64-row split kernel with one and no causal limit (2-5%),
# each in objects of their own: the 64-row split with a causal limit changed
# nothing or lost 1%, the 128-row split instances with a mask spill 100-270
# bytes under it and run up to 30% slower. The d = 256 kernel gains 3%
# without a mask and 4-10% with one (objects of its own; with a mask tangent
# it would keep 20 bytes per lane in scratch and stays as it is), while the
# mask-free 128-row split instances keep 12-108 bytes per lane in scratch
# and the d = 128 four-wave kernel loses 1.5% without a mask and moves
# within +-2% with one, so those stay at the default schedule; without a
# mask that kernel takes the max-ILP strategy instead (2% faster at
# (4,16,2048,128), 0.3% at (256,8,512,128), the same bits).
ILP_SCHED = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
MAX_ILP_SCHED = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
MAX_ILP_SCHED_OBJECTS = ("jvpattn_fwd_w128_none_",)
ILP_SCHED_OBJECTS = ("jvpattn_bwd_d64", "jvpattn_bwd_d128", "jvpattn_fwd_s64_bool_full", "jvpattn_fwd_s64_add_full",
                     "jvpattn_fwd_pp_bool_", "jvpattn_fwd_pp_add_", "jvpattn_fwd_w256_none_",
                     "jvpattn_fwd_w256_bool_", "jvpattn_fwd_w256_add_", "jvpattn_fwd_w256_bits_")


def _compile(job, verbose: bool) -> str:
    src, name, defines = job
    obj = os.path.join(BUILD, name + ".o")
    cmd = [hipcc(), *COMMON, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = (["-x", "hip"] + DEVICE + (VGPR_FORM if name.startswith(VGPR_FORM_OBJECTS) else [])
                    + (ILP_SCHED if name.startswith(ILP_SCHED_OBJECTS) else [])
                    + (MAX_ILP_SCHED if name.startswith(MAX_ILP_SCHED_OBJECTS) else []))
    else:
        cmd[1:1] = ["-x", "c++"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    workers = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.verbose))


if __name__ == "__main__":
    main()
