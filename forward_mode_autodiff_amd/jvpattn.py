"""Thin Python binding of libjvpattn.so (argument marshalling only).

The names follow the C interface in include/jvpattn.h. Every step of the
computation runs in the HIP library; PyTorch only supplies device memory and
the current stream. There is no CPU fallback: if the library is missing the
first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # loaded first so that the HIP runtime torch ships is the one the library binds to

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libjvpattn.so")

JVPATTN_F32, JVPATTN_F16, JVPATTN_BF16 = 0, 1, 2
JVPATTN_MASK_NONE, JVPATTN_MASK_BOOL, JVPATTN_MASK_ADDITIVE, JVPATTN_MASK_BITS = 0, 1, 2, 3
ERRORS = {
    0: "JVPATTN_OK", -1: "JVPATTN_ERR_NULL", -2: "JVPATTN_ERR_SHAPE", -3: "JVPATTN_ERR_DTYPE",
    -4: "JVPATTN_ERR_HEADDIM", -5: "JVPATTN_ERR_MASK", -6: "JVPATTN_ERR_ALIGN", -7: "JVPATTN_ERR_SCALE",
    -8: "JVPATTN_ERR_ALIAS", -9: "JVPATTN_ERR_HIP", -10: "JVPATTN_ERR_WORKSPACE", -11: "JVPATTN_ERR_ARG",
}
JVPATTN_ALGO_AUTO = -1
FWD_KERNELS = {"wg4": 0, "pp": 1, "split": 2, "split64": 3}   # jvpattn_fwd_kernel values
_DTYPE_CODE = {torch.float32: JVPATTN_F32, torch.float16: JVPATTN_F16, torch.bfloat16: JVPATTN_BF16}


class jvpattn_params(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Nq", ctypes.c_int32), ("Nk", ctypes.c_int32),
        ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("mask_kind", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("mask_stride_b", ctypes.c_int64), ("mask_stride_h", ctypes.c_int64),
        ("mask_stride_q", ctypes.c_int64),
        ("scale", ctypes.c_float), ("Hkv", ctypes.c_int32),
    ]


class JvpattnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libjvpattn.so once; raise loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m forward_mode_autodiff_amd.build`")
    lib = ctypes.CDLL(path)
    vp, fp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)
    P = ctypes.POINTER(jvpattn_params)
    lib.jvpattn_check_fwd.argtypes = [P] + [vp] * 9 + [vp, vp]
    lib.jvpattn_check_fwd.restype = ctypes.c_int
    lib.jvpattn_fwd.argtypes = [P] + [vp] * 7 + [vp, vp, vp, vp, vp]
    lib.jvpattn_fwd.restype = ctypes.c_int
    lib.jvpattn_fwd_tmask.argtypes = [P] + [vp] * 8 + [vp, vp, vp, vp, vp]
    lib.jvpattn_fwd_tmask.restype = ctypes.c_int
    lib.jvpattn_check_fwd_tmask.argtypes = [P] + [vp] * 12
    lib.jvpattn_check_fwd_tmask.restype = ctypes.c_int
    lib.jvpattn_strerror.argtypes = [ctypes.c_int]
    lib.jvpattn_strerror.restype = ctypes.c_char_p
    lib.jvpattn_last_hip_error.argtypes = []
    lib.jvpattn_last_hip_error.restype = ctypes.c_int
    lib.jvpattn_bwd_workspace_bytes.argtypes = [P]
    lib.jvpattn_bwd_workspace_bytes.restype = ctypes.c_int64
    lib.jvpattn_check_bwd.argtypes = [P] + [vp] * 20 + [ctypes.c_size_t]
    lib.jvpattn_check_bwd.restype = ctypes.c_int
    lib.jvpattn_bwd.argtypes = [P] + [vp] * 20 + [ctypes.c_size_t, vp]
    lib.jvpattn_bwd.restype = ctypes.c_int
    lib.jvpattn_bwd_tmask.argtypes = [P] + [vp] * 21 + [ctypes.c_size_t, vp]
    lib.jvpattn_bwd_tmask.restype = ctypes.c_int
    lib.jvpattn_check_bwd_tmask.argtypes = [P] + [vp] * 21 + [ctypes.c_size_t]
    lib.jvpattn_check_bwd_tmask.restype = ctypes.c_int
    lib.jvpattn_fwd_set_algo.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.jvpattn_fwd_set_algo.restype = ctypes.c_int
    _lib = lib
    return lib


def jvpattn_fwd_set_algo(kernel=None, order=None, key_range=None) -> None:
    """Force the forward's launch plan process-wide (None = the library's choice).

    kernel: "wg4" | "pp" | "split" | "split64"; order: "qb" (heaviest query blocks first) | "head"
    (head-major per XCD); key_range: False = never skip key tiles outside a shared mask row's range.
    """
    k = JVPATTN_ALGO_AUTO if kernel is None else FWD_KERNELS[kernel]
    o = JVPATTN_ALGO_AUTO if order is None else {"qb": 0, "head": 1}[order]
    r = JVPATTN_ALGO_AUTO if key_range is None else int(bool(key_range))
    rc = load_library().jvpattn_fwd_set_algo(k, o, r)
    if rc != 0:
        raise JvpattnError(rc, jvpattn_strerror(rc))


def jvpattn_strerror(code: int) -> str:
    return load_library().jvpattn_strerror(int(code)).decode()


def jvpattn_check_fwd(params: jvpattn_params, q, k, v, tq, tk, tv, mask, o, to, lse, tlse) -> int:
    """Host-only validation; pointer arguments are integers (addresses) or None."""
    lib = load_library()
    return lib.jvpattn_check_fwd(ctypes.byref(params), q, k, v, tq, tk, tv, mask, o, to, lse, tlse)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _as_4d(mask):
    """A mask as [B, H, Nq, Nk]: a 2-D mask is [Nq, Nk], a 3-D one [B, Nq, Nk]."""
    if mask.dim() == 2:
        return mask[None, None]
    if mask.dim() == 3:
        return mask[:, None]
    return mask


def _layout(mask):
    """Element strides the library uses for a 4-D mask (0 where an axis has extent 1)."""
    return tuple(0 if mask.shape[i] == 1 else mask.stride(i) for i in range(3)) + (mask.stride(3),)


def make_params(q, k, mask=None, causal=False, scale=None) -> tuple:
    """Fill jvpattn_params from tensors. Returns (params, mask tensor as passed to the library)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if q.dtype not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    p = jvpattn_params()
    p.B, p.H, p.Nq, p.Nk, p.d = B, H, Nq, Nk, d
    p.Hkv = k.shape[1]   # key/value heads; fewer than H means grouped-query attention
    p.dtype = _DTYPE_CODE[q.dtype]
    p.causal = 1 if causal else 0
    p.scale = float(1.0 / math.sqrt(d) if scale is None else scale)
    p.mask_kind = JVPATTN_MASK_NONE
    if mask is not None:
        mask = _as_4d(mask)
        if mask.dim() != 4:
            raise ValueError("mask must broadcast to [B, H, Nq, Nk]")
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        if mask.dtype == torch.uint8:
            p.mask_kind = JVPATTN_MASK_BOOL
        elif mask.dtype == torch.int32:
            p.mask_kind = JVPATTN_MASK_BITS   # bit-packed boolean mask (see pack_mask_bits)
        elif mask.dtype == q.dtype:
            p.mask_kind = JVPATTN_MASK_ADDITIVE
        else:
            raise TypeError("an additive mask must have the dtype of q")
        row = (Nk + 31) // 32 if p.mask_kind == JVPATTN_MASK_BITS else Nk
        if mask.shape[3] != row or mask.shape[2] not in (1, Nq) or mask.shape[1] not in (1, H) \
                or mask.shape[0] not in (1, B):
            raise ValueError(f"mask shape {tuple(mask.shape)} does not broadcast to {(B, H, Nq, Nk)}")
        if mask.stride(3) != 1:
            mask = mask.contiguous()
        p.mask_stride_b, p.mask_stride_h, p.mask_stride_q = _layout(mask)[:3]
    return p, mask


def jvpattn_check_fwd_tmask(params: jvpattn_params, q, k, v, tq, tk, tv, mask, tmask, o, to, lse, tlse) -> int:
    """Host-only validation of a jvpattn_fwd_tmask call; pointer arguments are integers or None."""
    return load_library().jvpattn_check_fwd_tmask(ctypes.byref(params), q, k, v, tq, tk, tv, mask, tmask, o, to,
                                                  lse, tlse)


def pack_mask_bits(mask):
    """A boolean mask [..., Nk] as the library's bit-packed layout: int32 words [..., ceil(Nk/32)],
    key j visible iff bit j % 32 of word j // 32 is set (8x fewer mask bytes than uint8)."""
    m = mask.to(torch.bool)
    nk = m.shape[-1]
    nw = (nk + 31) // 32
    pad = torch.zeros(*m.shape[:-1], nw * 32, dtype=torch.int64, device=m.device)
    pad[..., :nk] = m.to(torch.int64)
    bits = pad.reshape(*m.shape[:-1], nw, 32) << torch.arange(32, device=m.device, dtype=torch.int64)
    words = bits.sum(-1)                                     # 0 .. 2^32 - 1
    return torch.where(words >= 2 ** 31, words - 2 ** 32, words).to(torch.int32)


def jvpattn_fwd(q, k, v, tq=None, tk=None, tv=None, mask=None, causal=False, scale=None,
                want_tlse=True, out=None, tmask=None):
    """O, dO, lse, tlse = jvpattn_fwd(q, k, v, tq, tk, tv, mask, causal, scale).

    q, tq: [B,H,Nq,d]; k, v, tk, tv: [B,Hkv,Nk,d] on the GPU, one dtype
    (float32 / float16 / bfloat16), contiguous; Hkv divides H (query head h
    reads key/value head h // (H // Hkv)). Tangents may be None (zero).
    mask: None, a bool/uint8 tensor (True = attend), a bit-packed boolean
    mask (int32 words [.., ceil(Nk/32)], ``pack_mask_bits``) or an additive
    tensor of q's dtype, broadcastable to [B,H,Nq,Nk]. ``tmask``: the tangent of an
    additive mask, shaped like it (jvpattn_fwd_tmask). Work is queued on
    torch's current stream. ``out`` optionally supplies (o, to, lse, tlse) buffers.
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("tq", tq), ("tk", tk), ("tv", tv)):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, q has {q.dtype}")
    p, mask = make_params(q, k, mask, causal, scale)
    if tmask is not None:
        mask, tmask = _tmask_like(tmask, None, p, mask)
    if out is None:
        o = torch.empty_like(q)
        to = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], device=q.device, dtype=torch.float32)
        tlse = torch.empty_like(lse) if want_tlse else None
    else:
        o, to, lse, tlse = out
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if tmask is not None:
        rc = lib.jvpattn_fwd_tmask(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                                   _ptr(mask), _ptr(tmask), _ptr(o), _ptr(to), _ptr(lse), _ptr(tlse), stream)
    else:
        rc = lib.jvpattn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                             _ptr(mask), _ptr(o), _ptr(to), _ptr(lse), _ptr(tlse), stream)
    if rc != 0:
        msg = jvpattn_strerror(rc)
        if rc == -9:
            msg += f" (hipError {lib.jvpattn_last_hip_error()})"
        raise JvpattnError(rc, msg)
    return o, to, lse, tlse


def jvpattn_bwd_workspace_bytes(params: jvpattn_params) -> int:
    return int(load_library().jvpattn_bwd_workspace_bytes(ctypes.byref(params)))


def jvpattn_check_bwd(params: jvpattn_params, *ptrs, workspace_bytes: int = 0) -> int:
    """Host-only validation of a jvpattn_bwd call; ptrs are the 20 pointer arguments (integers or None)."""
    return load_library().jvpattn_check_bwd(ctypes.byref(params), *ptrs, workspace_bytes)


def _tmask_like(tmask, mask_in, p, mask):
    """tmask laid out as the library-side mask (returns (mask, tmask); may make both contiguous)."""
    if p.mask_kind != JVPATTN_MASK_ADDITIVE:
        raise ValueError("tmask needs an additive mask")
    if not tmask.is_cuda or tmask.dtype != mask.dtype:
        raise ValueError("tmask must be a GPU tensor of the mask's dtype")
    tmask = _as_4d(tmask)
    if tuple(tmask.shape) != tuple(mask.shape):
        raise ValueError(f"tmask shape {tuple(tmask.shape)} differs from the mask's {tuple(mask.shape)}")
    if _layout(tmask) != _layout(mask):
        # the library reads both with one set of strides
        mask, tmask = mask.contiguous(), tmask.contiguous()
        p.mask_stride_b, p.mask_stride_h, p.mask_stride_q = _layout(mask)[:3]
    return mask, tmask


def jvpattn_bwd(q, k, v, tq, tk, tv, o, to, lse, tlse, go, gto, mask=None, causal=False, scale=None,
                out=None, workspace=None, tmask=None):
    """dq, dk, dv, dtq, dtk, dtv = jvpattn_bwd(...): cotangents of q, k, v, tq, tk, tv.

    For L = <go, O> + <gto, dO> with (O, dO, lse, tlse) = jvpattn_fwd(q, k, v, tq, tk, tv, mask, causal,
    scale). Shapes and dtypes as for jvpattn_fwd; go, gto like q, either may be None (zero). ``out``
    optionally supplies the six output tensors (dtq, dtk, dtv may be None: not computed); ``tmask``, the
    additive mask's tangent the forward was taken along (jvpattn_bwd_tmask);
    ``workspace`` a uint8 device tensor of at least jvpattn_bwd_workspace_bytes bytes. Work is queued
    on torch's current stream.
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("tq", tq), ("tk", tk), ("tv", tv), ("o", o), ("to", to),
                    ("go", go), ("gto", gto)):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, q has {q.dtype}")
    p, mask = make_params(q, k, mask, causal, scale)
    if tmask is not None:
        mask, tmask = _tmask_like(tmask, None, p, mask)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dtq, dtk, dtv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv, dtq, dtk, dtv = out
    need = lib.jvpattn_bwd_workspace_bytes(ctypes.byref(p))
    if need < 0:
        raise JvpattnError(int(need), jvpattn_strerror(int(need)))
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    ws_bytes = workspace.numel() * workspace.element_size()
    if tmask is not None:
        rc = lib.jvpattn_bwd_tmask(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                                   _ptr(mask), _ptr(tmask), _ptr(o), _ptr(to), _ptr(lse), _ptr(tlse), _ptr(go),
                                   _ptr(gto), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dtq), _ptr(dtk), _ptr(dtv),
                                   _ptr(workspace), ws_bytes, stream)
    else:
        rc = lib.jvpattn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                             _ptr(mask), _ptr(o), _ptr(to), _ptr(lse), _ptr(tlse), _ptr(go), _ptr(gto),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dtq), _ptr(dtk), _ptr(dtv),
                             _ptr(workspace), ws_bytes, stream)
    if rc != 0:
        msg = jvpattn_strerror(rc)
        if rc == -9:
            msg += f" (hipError {lib.jvpattn_last_hip_error()})"
        raise JvpattnError(rc, msg)
    return dq, dk, dv, dtq, dtk, dtv
