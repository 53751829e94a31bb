"""The Python binding rejects every tensor the C interface would misread, before anything is queued.

The C functions receive raw pointers and cannot see shapes, dtypes or devices, so the binding checks
them: q, tq [B,H,Nq,d]; k, v, tk, tv [B,Hkv,Nk,d] (Hkv dividing H); o, to like q; lse, tlse float32
[B,H,Nq]; masks, mask tangents, workspaces and output buffers on q's device with the expected shape
and dtype; an int32 mask only as an explicit bit-packed mask. These checks come before the device
check, so CPU tensors exercise them here with no GPU; a CPU q itself is rejected last.
"""
import pytest
import torch

from forward_mode_autodiff_amd import jvpattn as J


def T(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def base(B=2, H=4, Hkv=2, Nq=40, Nk=56, d=64, dtype=torch.bfloat16):
    q = T(B, H, Nq, d, dtype=dtype)
    k = T(B, Hkv, Nk, d, dtype=dtype)
    return dict(q=q, k=k, v=k.clone(), tq=q.clone(), tk=k.clone(), tv=k.clone())


def fwd(**over):
    a = base()
    a.update(over)
    return J.jvpattn_fwd(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("tq"), a.pop("tk"), a.pop("tv"), **a)


@pytest.mark.parametrize("over,exc,msg", [
    (dict(v=T(2, 2, 55, 64)), ValueError, "v has shape"),
    (dict(tk=T(2, 2, 56, 32)), ValueError, "tk has shape"),
    (dict(tq=T(2, 4, 41, 64)), ValueError, "tq has shape"),
    (dict(tv=T(2, 2, 56, 64, dtype=torch.float16)), TypeError, "tv has dtype"),
    (dict(k=T(2, 3, 56, 64), v=T(2, 3, 56, 64), tk=None, tv=None), ValueError, "does not divide"),
    (dict(k=T(1, 2, 56, 64), v=T(1, 2, 56, 64), tk=None, tv=None), ValueError, "batch and head dim"),
    (dict(k=T(2, 2, 56, 32), v=T(2, 2, 56, 32), tk=None, tv=None), ValueError, "batch and head dim"),
    (dict(tq=base()["q"].transpose(2, 3).contiguous().transpose(2, 3)), ValueError, "contiguous"),
    (dict(mask=torch.ones(2, 1, 40, 56, dtype=torch.int32)), TypeError, "mask_kind='bits'"),
    (dict(mask=torch.ones(2, 1, 40, 56, dtype=torch.float32)), TypeError, "mask dtype"),
    (dict(mask=torch.ones(2, 1, 40, 57, dtype=torch.bool)), ValueError, "does not broadcast"),
    (dict(mask=torch.ones(2, 1, 40, 2, dtype=torch.uint8), mask_kind="bits"), TypeError, "bits mask must have"),
    (dict(mask=torch.ones(2, 1, 40, 1, dtype=torch.int32), mask_kind="bits"), ValueError, "does not broadcast"),
    (dict(mask_kind="bool"), ValueError, "without a mask"),
    (dict(mask=torch.ones(2, 1, 40, 56, dtype=torch.bool), mask_kind="nope"), ValueError, "unknown mask_kind"),
    (dict(mask=torch.zeros(2, 1, 40, 56, dtype=torch.bfloat16), tmask=torch.zeros(2, 1, 40, 55,
                                                                                  dtype=torch.bfloat16)),
     ValueError, "tmask shape"),
    (dict(mask=torch.zeros(2, 1, 40, 56, dtype=torch.bfloat16), tmask=torch.zeros(2, 1, 40, 56)), TypeError,
     "tmask has dtype"),
    (dict(mask=torch.ones(2, 1, 40, 56, dtype=torch.bool), tmask=torch.zeros(2, 1, 40, 56)), ValueError,
     "needs an additive mask"),
    (dict(out=(T(2, 4, 40, 64), T(2, 4, 40, 64), torch.zeros(2, 4, 40), torch.zeros(2, 4, 39))), ValueError,
     "tlse has shape"),
    (dict(out=(T(2, 4, 40, 64), T(2, 4, 40, 64), torch.zeros(2, 4, 40, dtype=torch.float64), None)), TypeError,
     "lse has dtype"),
    (dict(out=(T(2, 4, 40, 63), T(2, 4, 40, 64), torch.zeros(2, 4, 40), None)), ValueError, "o has shape"),
    (dict(), ValueError, "must be a GPU tensor"),
])
def test_fwd_rejects(over, exc, msg):
    with pytest.raises(exc, match=msg):
        fwd(**over)


def bwd(**over):
    a = base()
    q = a["q"]
    a.update(o=q.clone(), to=q.clone(), lse=torch.zeros(2, 4, 40), tlse=torch.zeros(2, 4, 40), go=q.clone(),
             gto=q.clone())
    a.update(over)
    return J.jvpattn_bwd(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("tq"), a.pop("tk"), a.pop("tv"), a.pop("o"),
                         a.pop("to"), a.pop("lse"), a.pop("tlse"), a.pop("go"), a.pop("gto"), **a)


@pytest.mark.parametrize("over,exc,msg", [
    (dict(o=T(2, 4, 40, 32)), ValueError, "o has shape"),
    (dict(lse=torch.zeros(2, 4, 41)), ValueError, "lse has shape"),
    (dict(tlse=None), ValueError, "tlse is required"),
    (dict(gto=T(2, 4, 40, 64, dtype=torch.float16)), TypeError, "gto has dtype"),
    (dict(go=T(2, 2, 40, 64)), ValueError, "go has shape"),
    (dict(out=(T(2, 4, 40, 64), T(2, 4, 56, 64), T(2, 2, 56, 64), None, None, None)), ValueError, "dk has shape"),
    (dict(out=(T(2, 4, 40, 64), T(2, 2, 56, 64), T(2, 2, 56, 64), T(2, 4, 40, 64), T(2, 2, 57, 64), None)),
     ValueError, "dtk has shape"),
    (dict(mask=torch.ones(2, 1, 40, 56, dtype=torch.int32)), TypeError, "mask_kind='bits'"),
    (dict(), ValueError, "must be a GPU tensor"),
])
def test_bwd_rejects(over, exc, msg):
    with pytest.raises(exc, match=msg):
        bwd(**over)


def test_make_params_infers_and_checks_kinds():
    a = base()
    p, m = J.make_params(a["q"], a["k"], torch.ones(2, 1, 40, 56, dtype=torch.bool))
    assert p.mask_kind == J.JVPATTN_MASK_BOOL and m.dtype == torch.uint8
    p, m = J.make_params(a["q"], a["k"], torch.zeros(40, 56, dtype=torch.bfloat16))
    assert p.mask_kind == J.JVPATTN_MASK_ADDITIVE and (p.mask_stride_b, p.mask_stride_h, p.mask_stride_q) == (0, 0, 56)
    words = J.pack_mask_bits(torch.ones(2, 1, 1, 56, dtype=torch.bool))
    p, m = J.make_params(a["q"], a["k"], words, mask_kind="bits")
    assert p.mask_kind == J.JVPATTN_MASK_BITS and m.shape[-1] == 2 and p.mask_stride_q == 0
    assert p.Hkv == 2 and p.H == 4
