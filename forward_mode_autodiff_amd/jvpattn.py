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
    -12: "JVPATTN_ERR_SCRATCH",
}
BWD_NOALLOC_MAX_ROWS = 1 << 20   # JVPATTN_BWD_NOALLOC_MAX_ROWS
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
    lib.jvpattn_bwd_noalloc.argtypes = [P] + [vp] * 19 + [vp]
    lib.jvpattn_bwd_noalloc.restype = ctypes.c_int
    lib.jvpattn_fwd_set_algo.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.jvpattn_fwd_set_algo.restype = ctypes.c_int
    lib.jvpattn_set_workgroups.argtypes = [ctypes.c_int]
    lib.jvpattn_set_workgroups.restype = ctypes.c_int
    lib.jvpattn_bwd_set_overlap.argtypes = [ctypes.c_int]
    lib.jvpattn_bwd_set_overlap.restype = ctypes.c_int
    _lib = lib
    return lib


def jvpattn_fwd_set_algo(kernel=None, order=None, key_range=None) -> None:
    """Force the forward's launch plan process-wide (None = the library's choice).

    kernel: "wg4" | "pp" | "split" | "split64"; order: "qb" (heaviest query blocks first) | "head"
    (head-major per XCD); key_range: False = no mask early-outs (neither the key range of a mask
    shared by all rows nor the blocks a mask hides from a whole wave are skipped).
    """
    k = JVPATTN_ALGO_AUTO if kernel is None else FWD_KERNELS[kernel]
    o = JVPATTN_ALGO_AUTO if order is None else {"qb": 0, "head": 1}[order]
    r = JVPATTN_ALGO_AUTO if key_range is None else int(bool(key_range))
    rc = load_library().jvpattn_fwd_set_algo(k, o, r)
    if rc != 0:
        raise JvpattnError(rc, jvpattn_strerror(rc))


def jvpattn_set_workgroups(max_workgroups: int = 0) -> None:
    """Cap the workgroups of the kernels that walk several blocks per workgroup (the mask-free bfloat16
    d = 96 / 128 forward, the mask-free d = 64 key side of the reverse pass); 0 = the library's choice,
    one workgroup per CU. Results do not depend on it; for tests and tuning."""
    rc = load_library().jvpattn_set_workgroups(int(max_workgroups))
    if rc != 0:
        raise JvpattnError(rc, jvpattn_strerror(rc))


def jvpattn_bwd_set_overlap(overlap=None) -> None:
    """How the reverse pass queues its key and query sides: False = one after the other on the
    caller's stream, True = the query side on a second stream of the library's, beside the key side;
    None = the library's choice (True where the key side alone would leave compute units idle, and for
    d = 128). Results do not depend on it."""
    mode = -1 if overlap is None else int(bool(overlap))
    rc = load_library().jvpattn_bwd_set_overlap(mode)
    if rc != 0:
        raise JvpattnError(rc, jvpattn_strerror(rc))


def _raise_on(rc: int) -> None:
    if rc != 0:
        msg = jvpattn_strerror(rc)
        if rc == -9:
            msg += f" (hipError {load_library().jvpattn_last_hip_error()})"
        raise JvpattnError(rc, msg)


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


def _tensor(name, t, shape, dtype, device, optional=False):
    """Reject a tensor the library would misread: wrong type, shape, dtype, device or layout.

    Raises TypeError (not a tensor, wrong dtype) or ValueError (shape, device, non-contiguous) before
    anything is queued; the C interface only sees raw pointers and cannot check these itself.
    """
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, q is on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


MASK_KINDS = {"bool": JVPATTN_MASK_BOOL, "additive": JVPATTN_MASK_ADDITIVE, "bits": JVPATTN_MASK_BITS}

# Mask-free parameter blocks of the library calls below, by (q shape, k shape, dtype, causal, scale):
# built once by make_params, then only read (the library takes them as const), so repeated calls on
# the same shapes skip rebuilding them. make_params itself always returns a fresh block.
_PARAMS = {}


def _params(q, k, mask, causal, scale, mask_kind):
    if mask is None and mask_kind is None and type(q) is torch.Tensor and type(k) is torch.Tensor:
        key = (q.shape, k.shape, q.dtype, bool(causal), scale)
        p = _PARAMS.get(key)
        if p is None:
            p, _ = make_params(q, k, None, causal, scale, None)
            if len(_PARAMS) >= 256:
                _PARAMS.clear()
            _PARAMS[key] = p
        return p, None
    return make_params(q, k, mask, causal, scale, mask_kind)


def make_params(q, k, mask=None, causal=False, scale=None, mask_kind=None) -> tuple:
    """Fill jvpattn_params from tensors. Returns (params, mask tensor as passed to the library).

    mask_kind: None infers it from the mask's dtype -- bool/uint8 -> "bool", q's dtype -> "additive";
    a bit-packed mask (int32 words, ``pack_mask_bits``) must say ``mask_kind="bits"``, so an int32 0/1
    mask is never silently read as bits.
    """
    if not isinstance(q, torch.Tensor) or not isinstance(k, torch.Tensor):
        raise TypeError("q and k must be tensors")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"k has shape {tuple(k.shape)}; q is {tuple(q.shape)} (batch and head dim must match)")
    Hkv = k.shape[1]
    if (Hkv == 0) != (H == 0) or (Hkv > 0 and H % Hkv != 0):
        raise ValueError(f"k has {Hkv} heads, which does not divide q's {H}")
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
    if mask is None:
        if mask_kind not in (None, "none"):
            raise ValueError(f"mask_kind={mask_kind!r} without a mask")
        return p, None
    if not isinstance(mask, torch.Tensor):
        raise TypeError("mask must be a tensor")
    mask = _as_4d(mask)
    if mask.dim() != 4:
        raise ValueError("mask must broadcast to [B, H, Nq, Nk]")
    if mask.device != q.device:
        raise ValueError(f"mask is on {mask.device}, q is on {q.device}")
    if mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    if mask_kind is None:
        if mask.dtype == torch.uint8:
            mask_kind = "bool"
        elif mask.dtype == q.dtype:
            mask_kind = "additive"
        elif mask.dtype == torch.int32:
            raise TypeError("an int32 mask is read as bit-packed only with mask_kind='bits' (see pack_mask_bits)")
        else:
            raise TypeError(f"mask dtype {mask.dtype}: expected bool/uint8, q's dtype {q.dtype}, or int32 words "
                            f"with mask_kind='bits'")
    if mask_kind not in MASK_KINDS:
        raise ValueError(f"unknown mask_kind {mask_kind!r}")
    want = {"bool": torch.uint8, "additive": q.dtype, "bits": torch.int32}[mask_kind]
    if mask.dtype != want:
        raise TypeError(f"a {mask_kind} mask must have dtype {want}, got {mask.dtype}")
    p.mask_kind = MASK_KINDS[mask_kind]
    row = (Nk + 31) // 32 if p.mask_kind == JVPATTN_MASK_BITS else Nk
    if mask.shape[3] != row or mask.shape[2] not in (1, Nq) or mask.shape[1] not in (1, H) \
            or mask.shape[0] not in (1, B):
        raise ValueError(f"mask shape {tuple(mask.shape)} does not broadcast to {(B, H, Nq, row)}")
    if mask.stride(3) != 1:
        mask = mask.contiguous()
    p.mask_stride_b, p.mask_stride_h, p.mask_stride_q = _layout(mask)[:3]
    return p, mask


def _all_like(ts, shape, dtype, device) -> bool:
    """Quick test that every tensor of ts (None allowed) is a plain tensor of this shape, dtype and
    device, contiguous; False sends the caller to the per-tensor checks, which name the problem."""
    for t in ts:
        if t is None:
            continue
        if type(t) is not torch.Tensor or t.shape != shape or t.dtype != dtype or t.device != device \
                or not t.is_contiguous():
            return False
    return True


def _check_inputs(q, k, v, tq, tk, tv):
    """q, k, v (and the tangents present) consistent with each other, on q's GPU, contiguous."""
    if type(q) is torch.Tensor and type(k) is torch.Tensor and q.dim() == 4 and k.dim() == 4:
        dt, dev = q.dtype, q.device
        if _all_like((q, tq), q.shape, dt, dev) and _all_like((k, v, tk, tv), k.shape, dt, dev):
            return
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a tensor")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    if not isinstance(k, torch.Tensor) or k.dim() != 4:
        raise ValueError("k must be a [B, Hkv, Nk, d] tensor")
    dev = q.device
    _tensor("q", q, q.shape, q.dtype, None)
    _tensor("k", k, k.shape, q.dtype, dev)
    _tensor("v", v, k.shape, q.dtype, dev)
    _tensor("tq", tq, q.shape, q.dtype, dev, optional=True)
    _tensor("tk", tk, k.shape, q.dtype, dev, optional=True)
    _tensor("tv", tv, k.shape, q.dtype, dev, optional=True)


def _require_gpu(q):
    """Last check before a launch: the tensors (all on q's device by now) must live on a GPU."""
    if not q.is_cuda:
        raise ValueError(f"q must be a GPU tensor (it is on {q.device})")


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
                want_tlse=True, out=None, tmask=None, mask_kind=None):
    """O, dO, lse, tlse = jvpattn_fwd(q, k, v, tq, tk, tv, mask, causal, scale).

    q, tq: [B,H,Nq,d]; k, v, tk, tv: [B,Hkv,Nk,d] on the GPU, one dtype
    (float32 / float16 / bfloat16), contiguous; Hkv divides H (query head h
    reads key/value head h // (H // Hkv)). Tangents may be None (zero).
    mask: None, a bool/uint8 tensor (True = attend), an additive tensor of q's
    dtype, or (with ``mask_kind="bits"``) a bit-packed boolean mask of int32
    words [.., ceil(Nk/32)] (``pack_mask_bits``), broadcastable to
    [B,H,Nq,Nk]. ``tmask``: the tangent of an additive mask, shaped like it
    (jvpattn_fwd_tmask). ``out`` optionally supplies (o, to, lse, tlse)
    buffers (tlse may be None). Every tensor is checked (shape, dtype, device,
    layout) before anything is queued; work goes on torch's current stream.
    """
    lib = load_library()
    _check_inputs(q, k, v, tq, tk, tv)
    p, mask = _params(q, k, mask, causal, scale, mask_kind)
    if tmask is not None:
        mask, tmask = _tmask_like(tmask, p, mask)
    stats = tuple(q.shape[:3])
    if out is None:
        o = torch.empty_like(q)
        to = torch.empty_like(q)
        lse = torch.empty(stats, device=q.device, dtype=torch.float32)
        tlse = torch.empty_like(lse) if want_tlse else None
    else:
        o, to, lse, tlse = out
        if not (o is not None and to is not None and lse is not None
                and _all_like((o, to), q.shape, q.dtype, q.device)
                and _all_like((lse, tlse), stats, torch.float32, q.device)):
            _tensor("o", o, q.shape, q.dtype, q.device)
            _tensor("to", to, q.shape, q.dtype, q.device)
            _tensor("lse", lse, stats, torch.float32, q.device)
            _tensor("tlse", tlse, stats, torch.float32, q.device, optional=True)
    _require_gpu(q)
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


def _tmask_like(tmask, p, mask):
    """tmask laid out as the library-side mask (returns (mask, tmask); may make both contiguous)."""
    if p.mask_kind != JVPATTN_MASK_ADDITIVE:
        raise ValueError("tmask needs an additive mask")
    if not isinstance(tmask, torch.Tensor):
        raise TypeError("tmask must be a tensor")
    if tmask.dtype != mask.dtype:
        raise TypeError(f"tmask has dtype {tmask.dtype}, the mask {mask.dtype}")
    if tmask.device != mask.device:
        raise ValueError(f"tmask is on {tmask.device}, the mask on {mask.device}")
    tmask = _as_4d(tmask)
    if tuple(tmask.shape) != tuple(mask.shape):
        raise ValueError(f"tmask shape {tuple(tmask.shape)} differs from the mask's {tuple(mask.shape)}")
    if _layout(tmask) != _layout(mask):
        # the library reads both with one set of strides
        mask, tmask = mask.contiguous(), tmask.contiguous()
        p.mask_stride_b, p.mask_stride_h, p.mask_stride_q = _layout(mask)[:3]
    return mask, tmask


def jvpattn_bwd(q, k, v, tq, tk, tv, o, to, lse, tlse, go, gto, mask=None, causal=False, scale=None,
                out=None, workspace=None, tmask=None, mask_kind=None, noalloc=False):
    """dq, dk, dv, dtq, dtk, dtv = jvpattn_bwd(...): cotangents of q, k, v, tq, tk, tv.

    For L = <go, O> + <gto, dO> with (O, dO, lse, tlse) = jvpattn_fwd(q, k, v, tq, tk, tv, mask, causal,
    scale). Shapes and dtypes as for jvpattn_fwd; go, gto like q, either may be None (zero). ``out``
    optionally supplies the six output tensors (dtq, dtk, dtv may be None: not computed); ``tmask``, the
    additive mask's tangent the forward was taken along (jvpattn_bwd_tmask);
    ``workspace`` a uint8 device tensor of at least jvpattn_bwd_workspace_bytes bytes. ``noalloc=True``
    calls jvpattn_bwd_noalloc instead: the library's own fixed scratch replaces the workspace (no
    device allocation by the library; B*H*Nq <= BWD_NOALLOC_MAX_ROWS; calls on one GPU must not
    overlap; no mask tangent). Every tensor is checked before anything is queued; work goes on torch's
    current stream.
    """
    lib = load_library()
    _check_inputs(q, k, v, tq, tk, tv)
    dev, stats = q.device, tuple(q.shape[:3])
    _tensor("o", o, q.shape, q.dtype, dev)
    _tensor("to", to, q.shape, q.dtype, dev)
    _tensor("lse", lse, stats, torch.float32, dev)
    _tensor("tlse", tlse, stats, torch.float32, dev)
    _tensor("go", go, q.shape, q.dtype, dev, optional=True)
    _tensor("gto", gto, q.shape, q.dtype, dev, optional=True)
    p, mask = _params(q, k, mask, causal, scale, mask_kind)
    if tmask is not None:
        mask, tmask = _tmask_like(tmask, p, mask)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dtq, dtk, dtv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv, dtq, dtk, dtv = out
        for name, t, like, opt in (("dq", dq, q, False), ("dk", dk, k, False), ("dv", dv, k, False),
                                   ("dtq", dtq, q, True), ("dtk", dtk, k, True), ("dtv", dtv, k, True)):
            _tensor(name, t, like.shape, q.dtype, dev, optional=opt)
    if noalloc:
        if tmask is not None or workspace is not None:
            raise ValueError("noalloc takes neither a workspace nor a mask tangent")
        _require_gpu(q)
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.jvpattn_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                                     _ptr(mask), _ptr(o), _ptr(to), _ptr(lse), _ptr(tlse), _ptr(go), _ptr(gto),
                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dtq), _ptr(dtk), _ptr(dtv), stream)
        _raise_on(rc)
        return dq, dk, dv, dtq, dtk, dtv
    need = lib.jvpattn_bwd_workspace_bytes(ctypes.byref(p))
    if need < 0:
        raise JvpattnError(int(need), jvpattn_strerror(int(need)))
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or workspace.device != dev
                                  or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    _require_gpu(q)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
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
