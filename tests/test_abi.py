"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, and rejects every invalid call before touching the device."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

from forward_mode_autodiff_amd import jvpattn as J

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jvpattn.h")

needs_lib = pytest.mark.skipif(not os.path.exists(J.LIB_PATH), reason="libjvpattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jvpattn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_entry_points():
    assert declared_functions() == ["jvpattn_bwd", "jvpattn_bwd_noalloc", "jvpattn_bwd_set_overlap",
                                    "jvpattn_bwd_tmask",
                                    "jvpattn_bwd_workspace_bytes", "jvpattn_check_bwd", "jvpattn_check_bwd_tmask",
                                    "jvpattn_check_fwd",
                                    "jvpattn_check_fwd_tmask", "jvpattn_fwd", "jvpattn_fwd_set_algo",
                                    "jvpattn_fwd_tmask", "jvpattn_last_hip_error", "jvpattn_set_workgroups",
                                    "jvpattn_strerror"]


@needs_lib
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", J.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
    lib = J.load_library()
    for name in declared_functions():
        assert getattr(lib, name) is not None


def test_params_struct_layout():
    assert ctypes.sizeof(J.jvpattn_params) == 64
    assert J.jvpattn_params.mask_stride_b.offset == 32
    assert J.jvpattn_params.scale.offset == 56
    assert J.jvpattn_params.Hkv.offset == 60


@needs_lib
def test_strerror_strings():
    for code in J.ERRORS:
        s = J.jvpattn_strerror(code)
        assert s and s != "unknown error code"
    assert J.jvpattn_strerror(12345) == "unknown error code"


def good_params(**kw):
    p = J.jvpattn_params()
    p.B, p.H, p.Nq, p.Nk, p.d = 2, 3, 100, 90, 64
    p.dtype, p.mask_kind, p.causal = J.JVPATTN_BF16, J.JVPATTN_MASK_NONE, 0
    p.mask_stride_b = p.mask_stride_h = p.mask_stride_q = 0
    p.scale = 0.125
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def ptrs(p, es=2):
    """Fake, disjoint, 256-aligned device addresses sized for the params (never dereferenced)."""
    nq = p.B * p.H * p.Nq * p.d * es
    nk = p.B * p.H * p.Nk * p.d * es
    ns = p.B * p.H * p.Nq * 4
    base = 1 << 40
    out = {}
    for name, n in (("q", nq), ("k", nk), ("v", nk), ("tq", nq), ("tk", nk), ("tv", nk), ("o", nq),
                    ("to", nq), ("lse", ns), ("tlse", ns), ("mask", p.B * p.Nq * p.Nk * 2)):
        out[name] = base
        base += (n + 4096) // 256 * 256 + 256
    return out


def call(p, P, **over):
    a = dict(P)
    a.update(over)
    mask = a["mask"] if p.mask_kind != 0 else None
    mask = over.get("mask", mask)
    return J.jvpattn_check_fwd(p, a["q"], a["k"], a["v"], a["tq"], a["tk"], a["tv"], mask, a["o"],
                               a["to"], a["lse"], a["tlse"])


@needs_lib
def test_check_accepts_valid_calls():
    p = good_params()
    assert call(p, ptrs(p)) == 0
    assert call(p, ptrs(p), tq=None, tk=None, tv=None, tlse=None) == 0
    for d in (32, 64, 96, 128, 256):
        for dt, es in ((J.JVPATTN_F32, 4), (J.JVPATTN_F16, 2), (J.JVPATTN_BF16, 2)):
            if d == 256 and dt == J.JVPATTN_F32:
                continue   # rejected: see test_check_rejects
            p = good_params(d=d, dtype=dt)
            assert call(p, ptrs(p, es)) == 0
    p = good_params(mask_kind=J.JVPATTN_MASK_BOOL, mask_stride_b=100 * 90, mask_stride_q=90)
    assert call(p, ptrs(p)) == 0
    p = good_params(mask_kind=J.JVPATTN_MASK_ADDITIVE, mask_stride_b=0, mask_stride_q=0)
    assert call(p, ptrs(p)) == 0
    # empty problems need no pointers at all
    p = good_params(Nq=0)
    assert J.jvpattn_check_fwd(p, *([None] * 11)) == 0
    p = good_params(B=0)
    assert J.jvpattn_check_fwd(p, *([None] * 11)) == 0


@needs_lib
def test_check_bit_packed_mask():
    # rows of ceil(Nk/32) 32-bit words: Nk = 90 -> 3 words
    p = good_params(mask_kind=J.JVPATTN_MASK_BITS, mask_stride_b=100 * 3, mask_stride_q=3)
    P = ptrs(p)
    assert call(p, P) == 0
    assert call(p, P, mask=P["mask"] + 2) == -6                  # words are 4-byte aligned
    nbytes = (2 * 100 * 3) * 4
    assert call(p, P, o=P["mask"] + nbytes) == 0                 # right after the last word: no overlap
    assert call(p, P, lse=P["mask"] + nbytes - 4) == -8          # overlapping the last word
    # the reverse pass takes them too, with the same extent in words
    pb = good_params(mask_kind=J.JVPATTN_MASK_BITS, mask_stride_b=100 * 3, mask_stride_q=3)
    Q = bwd_ptrs(pb)
    assert call_bwd(pb, Q) == 0
    assert call_bwd(pb, Q, dq=Q["mask"] + nbytes - 16) == -8


@needs_lib
def test_check_mask_tangent():
    p = good_params(mask_kind=J.JVPATTN_MASK_ADDITIVE, mask_stride_b=100 * 90, mask_stride_q=90)
    P = ptrs(p)
    t = P["mask"] + (1 << 30)   # a disjoint tangent laid out as the mask
    args = lambda **o: [dict(dict(P, tmask=t), **o)[n] for n in ("q", "k", "v", "tq", "tk", "tv", "mask", "tmask",
                                                                  "o", "to", "lse", "tlse")]
    assert J.jvpattn_check_fwd_tmask(p, *args()) == 0
    assert J.jvpattn_check_fwd_tmask(p, *args(tmask=None)) == 0           # zero tangent
    assert J.jvpattn_check_fwd_tmask(p, *args(tmask=t + 1)) == -6         # misaligned
    assert J.jvpattn_check_fwd_tmask(p, *args(o=t)) == -8                  # overlaps an output
    pb = good_params(mask_kind=J.JVPATTN_MASK_BOOL, mask_stride_b=100 * 90, mask_stride_q=90)
    assert J.jvpattn_check_fwd_tmask(pb, *args()) == -5                    # needs an additive mask
    pn = good_params()
    assert J.jvpattn_check_fwd_tmask(pn, *args(mask=None)) == -5
    # the forward's own checks come first
    assert J.jvpattn_check_fwd_tmask(p, *args(q=None)) == -1


@needs_lib
def test_check_grouped_kv_heads():
    # Hkv = 0 stands for H; a divisor of H shrinks k, v, tk, tv to B*Hkv heads
    for hkv in (0, 1, 2, 3, 6):
        p = good_params(H=6, Hkv=hkv)
        assert call(p, ptrs(p)) == 0
    # the K/V spans are B*Hkv heads: lse may sit right after a shrunk k (no false alias) ...
    p = good_params(H=6, Hkv=2)
    P = ptrs(p)
    nk = p.B * 2 * p.Nk * p.d * 2
    assert call(p, P, lse=P["k"] + nk) == 0
    # ... and an overlap inside the shrunk span is still caught
    assert call(p, P, lse=P["k"] + nk - 256) == -8


@needs_lib
@pytest.mark.parametrize("case,code", [
    ("params_null", -1), ("q_null", -1), ("o_null", -1), ("to_null", -1), ("lse_null", -1), ("k_null", -1),
    ("neg_B", -2), ("neg_Nk", -2), ("d_zero", -2), ("overflow", -2),
    ("dtype", -3), ("d_48", -4), ("d_512", -4), ("d_256_f32", -4),
    ("kind", -5), ("mask_missing", -5), ("mask_extra", -5), ("mask_neg_stride", -5), ("mask_stride_overflow", -5),
    ("q_misaligned", -6), ("tv_misaligned", -6), ("lse_misaligned", -6), ("mask_misaligned", -6),
    ("scale_nan", -7), ("scale_inf", -7), ("scale_zero", -7), ("scale_neg", -7),
    ("o_is_q", -8), ("to_overlaps_v", -8), ("lse_overlaps_tlse", -8), ("o_overlaps_mask", -8),
    ("hkv_not_divisor", -2), ("hkv_above_h", -2), ("hkv_negative", -2),
])
def test_check_rejects(case, code):
    p = good_params()
    P = ptrs(p)
    over = {}
    if case == "params_null":
        assert J.load_library().jvpattn_check_fwd(None, *[P[n] for n in ("q", "k", "v", "tq", "tk", "tv")],
                                                  None, P["o"], P["to"], P["lse"], P["tlse"]) == code
        return
    if case.endswith("_null"):
        over[case[:-5]] = None
    elif case == "neg_B":
        p.B = -1
    elif case == "neg_Nk":
        p.Nk = -5
    elif case == "d_zero":
        p.d = 0
    elif case == "overflow":
        p.B, p.H, p.Nq = 2 ** 31 - 1, 2 ** 31 - 1, 2 ** 31 - 1
    elif case == "dtype":
        p.dtype = 7
    elif case == "d_48":
        p.d = 48
    elif case == "d_512":
        p.d = 512
    elif case == "d_256_f32":
        p.d, p.dtype = 256, J.JVPATTN_F32
    elif case == "kind":
        p.mask_kind = 5
    elif case == "mask_missing":
        p.mask_kind = J.JVPATTN_MASK_BOOL
        over["mask"] = None
    elif case == "mask_extra":
        over["mask"] = P["mask"]
    elif case == "mask_neg_stride":
        p.mask_kind, p.mask_stride_q = J.JVPATTN_MASK_BOOL, -90
    elif case == "mask_stride_overflow":
        p.mask_kind, p.mask_stride_b = J.JVPATTN_MASK_BOOL, 2 ** 63 - 1
    elif case == "q_misaligned":
        over["q"] = P["q"] + 8
    elif case == "tv_misaligned":
        over["tv"] = P["tv"] + 4
    elif case == "lse_misaligned":
        over["lse"] = P["lse"] + 2
    elif case == "mask_misaligned":
        p.mask_kind, p.mask_stride_q = J.JVPATTN_MASK_ADDITIVE, 90
        over["mask"] = P["mask"] + 1
    elif case.startswith("scale_"):
        p.scale = {"nan": float("nan"), "inf": float("inf"), "zero": 0.0, "neg": -0.125}[case[6:]]
    elif case == "o_is_q":
        over["o"] = P["q"]
    elif case == "to_overlaps_v":
        over["to"] = P["v"] + 256
    elif case == "lse_overlaps_tlse":
        over["tlse"] = P["lse"] + 64
    elif case.startswith("hkv_"):
        p.H = 6
        P = ptrs(p)
        p.Hkv = {"not_divisor": 4, "above_h": 12, "negative": -2}[case[4:]]
    elif case == "o_overlaps_mask":
        p.mask_kind, p.mask_stride_q, p.mask_stride_b = J.JVPATTN_MASK_BOOL, 90, 9000
        over["o"] = P["mask"]
    assert call(p, P, **over) == code


BWD_PTRS = ("q", "k", "v", "tq", "tk", "tv", "mask", "o", "to", "lse", "tlse", "go", "gto",
            "dq", "dk", "dv", "dtq", "dtk", "dtv", "ws")


def bwd_ptrs(p, es=2):
    """Forward pointers plus cotangents, outputs and a workspace (fake, disjoint, aligned)."""
    P = ptrs(p, es)
    nq = p.B * p.H * p.Nq * p.d * es
    nk = p.B * p.H * p.Nk * p.d * es
    base = max(P.values()) + (1 << 30)
    for name, n in (("go", nq), ("gto", nq), ("dq", nq), ("dk", nk), ("dv", nk), ("dtq", nq), ("dtk", nk),
                    ("dtv", nk), ("ws", 1 << 20)):
        P[name] = base
        base += (n + 4096) // 256 * 256 + 256
    return P


def call_bwd(p, P, ws_bytes=None, **over):
    a = dict(P)
    a.update(over)
    if p.mask_kind == 0 and "mask" not in over:
        a["mask"] = None
    if ws_bytes is None:
        ws_bytes = max(J.jvpattn_bwd_workspace_bytes(p), 0)
    return J.jvpattn_check_bwd(p, *[a[n] for n in BWD_PTRS], workspace_bytes=ws_bytes)


@needs_lib
def test_bwd_workspace_size():
    p = good_params()
    n = J.jvpattn_bwd_workspace_bytes(p)
    rows = p.B * p.H * p.Nq
    assert n >= 4 * 4 * rows and n % 256 == 0
    assert J.jvpattn_bwd_workspace_bytes(good_params(B=-1)) == -2
    assert J.jvpattn_bwd_workspace_bytes(good_params(Nq=0)) == 0


@needs_lib
def test_check_bwd_accepts_valid_calls():
    p = good_params(dtype=J.JVPATTN_F32)
    assert call_bwd(p, bwd_ptrs(p, 4)) == 0
    for dt in (J.JVPATTN_F16, J.JVPATTN_BF16):
        p = good_params(dtype=dt, d=128)
        assert call_bwd(p, bwd_ptrs(p)) == 0
        p = good_params(dtype=dt)
        assert call_bwd(p, bwd_ptrs(p)) == 0
        assert call_bwd(p, bwd_ptrs(p), tq=None, tk=None, tv=None) == 0
        # zero cotangents and unwanted tangent cotangents may be NULL
        assert call_bwd(p, bwd_ptrs(p), go=None, gto=None, dtq=None, dtk=None, dtv=None) == 0
    p = good_params(mask_kind=J.JVPATTN_MASK_BOOL, mask_stride_b=100 * 90, mask_stride_q=90, causal=1)
    assert call_bwd(p, bwd_ptrs(p)) == 0
    # no query rows: keys still get (zero) gradients; no workspace is needed
    p = good_params(Nq=0)
    P = bwd_ptrs(p)
    assert call_bwd(p, P, q=None, o=None, to=None, lse=None, tlse=None, go=None, gto=None, dq=None, dtq=None,
                    ws=None, ws_bytes=0) == 0


@needs_lib
@pytest.mark.parametrize("case,code", [
    ("dtype", -3), ("f32_d128", -4), ("d96", -4), ("d256", -4), ("dq_null", -1), ("tlse_null", -1), ("dv_null", -1), ("dq_misaligned", -6),
    ("ws_null", -10), ("ws_small", -10), ("ws_misaligned", -10), ("ws_overlaps_go", -10), ("ws_overlaps_dk", -10),
    ("dq_is_q", -8), ("dk_overlaps_dv", -8), ("dtv_overlaps_gto", -8), ("q_null", -1), ("scale_nan", -7),
])
def test_check_bwd_rejects(case, code):
    p = good_params()
    if case == "dtype":
        p.dtype = 7
        assert call_bwd(p, bwd_ptrs(p)) == code
        return
    if case == "f32_d128":
        p.dtype, p.d = J.JVPATTN_F32, 128
        assert call_bwd(p, bwd_ptrs(p, 4)) == code
        return
    if case in ("d96", "d256"):
        p.d = int(case[1:])
        assert call_bwd(p, bwd_ptrs(p)) == code
        return
    P = bwd_ptrs(p)
    over, wsb = {}, None
    if case.endswith("_null"):
        over[case[:-5]] = None
    elif case == "dq_misaligned":
        over["dq"] = P["dq"] + 8
    elif case == "ws_small":
        wsb = J.jvpattn_bwd_workspace_bytes(p) - 4
    elif case == "ws_misaligned":
        over["ws"] = P["ws"] + 128
    elif case == "ws_overlaps_go":
        over["ws"] = P["go"]
    elif case == "ws_overlaps_dk":
        over["ws"] = P["dk"]
    elif case == "dq_is_q":
        over["dq"] = P["q"]
    elif case == "dk_overlaps_dv":
        over["dk"] = P["dv"] + 512
    elif case == "dtv_overlaps_gto":
        over["dtv"] = P["gto"]
    elif case == "scale_nan":
        p.scale = float("nan")
    assert call_bwd(p, P, ws_bytes=wsb, **over) == code


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_validator_under_host_sanitizers(tmp_path):
    """The validator is plain C++: build it with g++ and ASan/UBSan and run a driver over edge cases."""
    drv = tmp_path / "drv.cpp"
    drv.write_text(r'''
#include "jvpattn.h"
#include <cstdio>
#include <cstdint>
#include <cmath>
int main() {
  jvpattn_params p{};
  p.B = 2; p.H = 2; p.Nq = 33; p.Nk = 17; p.d = 64; p.dtype = JVPATTN_F16; p.scale = 0.125f;
  char* base = reinterpret_cast<char*>(uintptr_t(1) << 40);
  auto at = [&](long i) { return base + i * (1L << 24); };
  int bad = 0;
  bad += jvpattn_check_fwd(&p, at(0), at(1), at(2), at(3), at(4), at(5), nullptr, at(6), at(7),
                           (float*)at(8), (float*)at(9)) != JVPATTN_OK;
  p.B = 2147483647; p.H = 2147483647; p.Nq = 2147483647;
  bad += jvpattn_check_fwd(&p, at(0), at(1), at(2), at(3), at(4), at(5), nullptr, at(6), at(7),
                           (float*)at(8), (float*)at(9)) != JVPATTN_ERR_SHAPE;
  p.B = 2; p.H = 2; p.Nq = 33; p.mask_kind = JVPATTN_MASK_BOOL; p.mask_stride_b = INT64_MAX;
  bad += jvpattn_check_fwd(&p, at(0), at(1), at(2), at(3), at(4), at(5), at(10), at(6), at(7),
                           (float*)at(8), (float*)at(9)) != JVPATTN_ERR_MASK;
  {
    jvpattn_params b = p;
    b.mask_kind = JVPATTN_MASK_NONE; b.mask_stride_b = 0;
    const int64_t ws = jvpattn_bwd_workspace_bytes(&b);
    bad += ws <= 0;
    bad += jvpattn_check_bwd(&b, at(0), at(1), at(2), at(3), at(4), at(5), nullptr, at(6), at(7), (float*)at(8),
                             (float*)at(9), at(11), at(12), at(13), at(14), at(15), at(16), at(17), at(18),
                             at(19), size_t(ws)) != JVPATTN_OK;
    bad += jvpattn_check_bwd(&b, at(0), at(1), at(2), at(3), at(4), at(5), nullptr, at(6), at(7), (float*)at(8),
                             (float*)at(9), at(11), at(12), at(13), at(14), at(15), at(16), at(17), at(18),
                             at(19), size_t(ws) - 1) != JVPATTN_ERR_WORKSPACE;
    b.B = 2147483647; b.H = 2147483647; b.Nq = 2147483647;
    bad += jvpattn_bwd_workspace_bytes(&b) != JVPATTN_ERR_SHAPE;
  }
  p.mask_stride_b = 0; p.scale = NAN;
  bad += jvpattn_check_fwd(&p, at(0), at(1), at(2), at(3), at(4), at(5), at(10), at(6), at(7),
                           (float*)at(8), (float*)at(9)) != JVPATTN_ERR_SCALE;
  bad += jvpattn_check_fwd(nullptr, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) != JVPATTN_ERR_NULL;
  for (int c = -10; c <= 1; ++c) bad += jvpattn_strerror(c) == nullptr;
  std::printf("bad=%d\n", bad);
  return bad;
}
''')
    exe = tmp_path / "drv"
    src = os.path.join(ROOT, "forward_mode_autodiff_amd", "csrc", "jvpattn_check.cpp")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{ROOT}/include", f"-I{ROOT}/forward_mode_autodiff_amd/csrc", str(drv), src, "-o", str(exe)]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bad=0" in r.stdout


@needs_lib
def test_check_bwd_mask_tangent():
    p = good_params(mask_kind=J.JVPATTN_MASK_ADDITIVE, mask_stride_b=100 * 90, mask_stride_q=90)
    Q = bwd_ptrs(p)
    t = Q["ws"] + (1 << 30)   # a disjoint tangent laid out as the mask
    lib = J.load_library()

    def chk(**o):
        a = dict(Q, tmask=t)
        a.update(o)
        names = ("q", "k", "v", "tq", "tk", "tv", "mask", "tmask", "o", "to", "lse", "tlse", "go", "gto",
                 "dq", "dk", "dv", "dtq", "dtk", "dtv", "ws")
        return lib.jvpattn_check_bwd_tmask(p, *[a[n] for n in names], max(J.jvpattn_bwd_workspace_bytes(p), 0))
    assert chk() == 0
    assert chk(tmask=None) == 0
    assert chk(tmask=t + 2 + 1) == -6          # misaligned
    assert chk(dk=t) == -8                     # a gradient over it
    assert chk(ws=t) == -10                    # the workspace over it
    assert chk(o=t) == -8                      # a forward output over it


@needs_lib
def test_fwd_set_algo_rejects_out_of_range_values():
    lib = J.load_library()
    for args in [(4, -1, -1), (-2, -1, -1), (-1, 2, -1), (-1, -1, 2), (-1, -3, -1)]:
        assert lib.jvpattn_fwd_set_algo(*args) == -11, args
    for args in [(-1, -1, -1), (0, 0, 0), (3, 1, 1)]:
        assert lib.jvpattn_fwd_set_algo(*args) == 0, args
    assert lib.jvpattn_fwd_set_algo(-1, -1, -1) == 0
    with pytest.raises(KeyError):
        J.jvpattn_fwd_set_algo(kernel="nope")


@needs_lib
def test_bwd_set_overlap_rejects_other_modes():
    lib = J.load_library()
    for m in (-2, 2, 1 << 20):
        assert lib.jvpattn_bwd_set_overlap(m) == -11, m
    for m in (0, 1, -1):
        assert lib.jvpattn_bwd_set_overlap(m) == 0, m
    J.jvpattn_bwd_set_overlap(True)
    J.jvpattn_bwd_set_overlap()


@needs_lib
def test_set_workgroups_rejects_negative_caps():
    lib = J.load_library()
    assert lib.jvpattn_set_workgroups(-1) == -11
    for n in (5, 8, 1 << 30, 0):
        assert lib.jvpattn_set_workgroups(n) == 0, n
    with pytest.raises(J.JvpattnError):
        J.jvpattn_set_workgroups(-3)
    J.jvpattn_set_workgroups()


@needs_lib
def test_bwd_noalloc_rejects_oversized_problems_before_touching_the_gpu():
    """More than 2^20 query rows in all: JVPATTN_ERR_SCRATCH, decided before any runtime call."""
    lib = J.load_library()
    p = good_params(B=1, H=8, Nq=(1 << 17) + 1, Nk=64)
    args = [None] * 19 + [None]
    assert lib.jvpattn_bwd_noalloc(ctypes.byref(p), *args) == -12
    p = good_params(B=-1)
    assert lib.jvpattn_bwd_noalloc(ctypes.byref(p), *args) == -2
    assert lib.jvpattn_bwd_noalloc(None, *args) == -1
    assert "2^20" in J.jvpattn_strerror(-12)
