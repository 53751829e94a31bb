"""PyTorch integration: attention whose derivatives, both modes, run in libjvpattn.

The "JVP Flash Attention" README presents the method as a drop-in for
``torch.nn.functional.scaled_dot_product_attention`` (section "Usage": q, k,
v, attn_mask; no dropout) that supports forward-mode derivatives, with a
``fwd_dual`` entry for dual inputs, and Hessian-vector products (section
"Description"). This module gives both entries on top of the C ABI; every
computation is a libjvpattn call (jvpattn_fwd, jvpattn_bwd) and torch only
supplies tensors, the autograd graph and streams.

``attention(q, k, v, attn_mask=None, is_causal=False, scale=None)``
    the output O. Reverse mode (``.backward()``, ``torch.autograd.grad``)
    runs jvpattn_bwd with a zero cotangent for the tangent output; forward
    mode -- ``torch.autograd.forward_ad`` dual tensors, or ``torch.func.jvp``
    around a model that calls it (the README's use of ``JVPAttn.fwd_dual``
    inside ``torch.func.jvp``) -- runs jvpattn_fwd with the tangents; an
    additive ``attn_mask`` may carry a tangent too (jvpattn_fwd_tmask).
    Under ``torch.func.jvp`` the tangent output stays differentiable in
    reverse mode (through jvpattn_bwd), so a loss of (O, dO) can be
    backpropagated: the HVP route. Other ``torch.func`` transforms (vmap,
    nested jvp) are not supported and raise.

``fwd_dual(q, k, v, tq, tk, tv, attn_mask=None, is_causal=False, scale=None, tmask=None)``
    the pair (O, dO) -- the output and its JVP, along the additive mask's
    tangent ``tmask`` as well when given -- differentiable in reverse mode
    with respect to all six inputs (jvpattn_bwd, jvpattn_bwd_tmask). A
    Hessian-vector product of a loss is reverse mode over this pair.

Inputs: q [B, H, N, d], k and v [B, Hkv, N, d] (Hkv dividing H: grouped
key/value heads) CUDA tensors of one dtype. The reverse pass takes float16
/ bfloat16 with d = 64 or 128 and float32 with d = 64; the forward takes all
three types with d = 32, 64, 96, 128, and d = 256 in the 16-bit types. Masks as in ``jvpattn_fwd`` (bool: True = attend; additive: q's
dtype, no reverse-mode gradient).
"""
from __future__ import annotations

import torch

from torch._C import _functorch

from . import jvpattn as J


def _c(t):
    return None if t is None else t.contiguous()


def _jvp_level(*ts):
    """The torch.func.jvp level whose wrapped tensors a jvp rule received, or None (forward_ad duals).

    torch.func.jvp runs a custom rule with its primals and tangents wrapped one level deep; the
    library needs the tensors with storage underneath. Nested or batched transforms are refused.
    """
    levels = {_functorch.maybe_get_level(t) for t in ts
              if isinstance(t, torch.Tensor) and _functorch.is_functorch_wrapped_tensor(t)}
    if not levels:
        return None
    if len(levels) > 1:
        raise NotImplementedError("attention under nested torch.func transforms is not supported")
    level = levels.pop()
    for t in ts:
        if isinstance(t, torch.Tensor) and _functorch.is_functorch_wrapped_tensor(t):
            inner = _functorch._unwrap_for_grad(t, level)
            if _functorch.is_functorch_wrapped_tensor(inner) or inner.data_ptr() == 0 and inner.numel():
                raise NotImplementedError("attention under torch.func transforms other than one jvp "
                                          "(vmap, nested jvp) is not supported")
    return level


def _unwrap(t, level):
    return None if t is None else _functorch._unwrap_for_grad(t, level)


class _Const:
    """Holds the mask outside the autograd/functorch view: it is a constant of the map."""

    def __init__(self, t):
        self.t = t


class _Attention(torch.autograd.Function):
    """O = attention(q, k, v); lse rides along (not differentiable). The mask is an input so
    that forward mode sees its tangent; reverse mode gives it no gradient."""

    @staticmethod
    def forward(q, k, v, mask, causal, scale):
        o, to, lse, tlse = J.jvpattn_fwd(q, k, v, None, None, None, mask=mask, causal=causal, scale=scale)
        return o, lse, to, tlse

    @staticmethod
    def setup_context(ctx, inputs, output):
        q, k, v, mask, causal, scale = inputs
        o, lse, to, tlse = output
        ctx.save_for_backward(q, k, v, o, lse, to, tlse)
        ctx.save_for_forward(q, k, v)
        ctx.mask, ctx.causal, ctx.scale = mask, causal, scale
        ctx.mark_non_differentiable(lse, to, tlse)

    @staticmethod
    def backward(ctx, go, _glse, _gto, _gtlse):
        q, k, v, o, lse, to, tlse = ctx.saved_tensors
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), None, None, None)
        dq, dk, dv, _, _, _ = J.jvpattn_bwd(q, k, v, None, None, None, o, to, lse, tlse, _c(go), None,
                                            mask=ctx.mask, causal=ctx.causal, scale=ctx.scale, out=out)
        return dq, dk, dv, None, None, None

    @staticmethod
    def jvp(ctx, tq, tk, tv, tmask, _tcausal, _tscale):
        q, k, v = ctx.saved_tensors   # in jvp: the tensors given to save_for_forward
        m = ctx.mask
        # an additive mask's tangent enters the score tangent; a boolean mask has none
        if tmask is not None and (m is None or m.dtype == torch.bool):
            tmask = None
        level = _jvp_level(q, k, v, tq, tk, tv, m, tmask)
        if level is None:
            o, to, lse, tlse = J.jvpattn_fwd(q, k, v, _c(tq), _c(tk), _c(tv), mask=m, causal=ctx.causal,
                                             scale=ctx.scale, tmask=_c(tmask))
            return to, None, None, None   # lse and the aux outputs are not differentiable
        # torch.func.jvp: the same call on the tensors under the wrappers, made through the (O, dO)
        # function so that the tangent keeps a reverse-mode graph (jvpattn_bwd) below this level
        u = lambda t: _c(_unwrap(t, level))
        with torch.enable_grad():
            _, to, _, _ = _AttentionDual.apply(u(q), u(k), u(v), u(tq), u(tk), u(tv), _Const(_unwrap(m, level)),
                                               ctx.causal, ctx.scale, _Const(u(tmask)))
        # the call above already ran through this level's interpreter (its output comes back wrapped)
        if not (_functorch.is_functorch_wrapped_tensor(to) and _functorch.maybe_get_level(to) == level):
            to = _functorch._wrap_for_grad(to, level)
        return to, None, None, None


class _AttentionDual(torch.autograd.Function):
    """(O, dO) = fwd_dual(q, k, v, tq, tk, tv); lse and tlse ride along (not differentiable)."""

    @staticmethod
    def forward(q, k, v, tq, tk, tv, mask, causal, scale, tmask):
        return J.jvpattn_fwd(q, k, v, tq, tk, tv, mask=mask.t, causal=causal, scale=scale, tmask=tmask.t)

    @staticmethod
    def setup_context(ctx, inputs, output):
        q, k, v, tq, tk, tv, mask, causal, scale, tmask = inputs
        o, to, lse, tlse = output
        ctx.save_for_backward(q, k, v, tq, tk, tv, o, to, lse, tlse)
        ctx.mask, ctx.causal, ctx.scale, ctx.tmask = mask.t, causal, scale, tmask.t
        ctx.mark_non_differentiable(lse, tlse)

    @staticmethod
    def backward(ctx, go, gto, _glse, _gtlse):
        q, k, v, tq, tk, tv, o, to, lse, tlse = ctx.saved_tensors
        need = ctx.needs_input_grad
        # outputs for the cotangents of tq, tk, tv only where they are wanted (NULL: not computed)
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
               torch.empty_like(q) if need[3] else None, torch.empty_like(k) if need[4] else None,
               torch.empty_like(v) if need[5] else None)
        g = J.jvpattn_bwd(q, k, v, tq, tk, tv, o, to, lse, tlse, _c(go), _c(gto), mask=ctx.mask,
                          causal=ctx.causal, scale=ctx.scale, out=out, tmask=ctx.tmask)
        return tuple(x if need[i] else None for i, x in enumerate(g)) + (None, None, None, None)


def attention(q, k, v, attn_mask=None, is_causal=False, scale=None):
    """Scaled-dot-product attention (no dropout) with both derivative modes in libjvpattn."""
    return _Attention.apply(q, k, v, attn_mask, bool(is_causal), scale)[0]


def fwd_dual(q, k, v, tq, tk, tv, attn_mask=None, is_causal=False, scale=None, tmask=None):
    """(O, dO): attention and its JVP along (tq, tk, tv) and, if given, the additive mask's tangent
    tmask; reverse-differentiable in all six inputs."""
    o, to, _, _ = _AttentionDual.apply(q, k, v, _c(tq), _c(tk), _c(tv), _Const(attn_mask), bool(is_causal),
                                       scale, _Const(_c(tmask)))
    return o, to
