"""torch.autograd wrapper over the C ABI.

    attention(q, k, v, scale=None, is_causal=False, attn_mask=None, sinks=None) -> o

Both directions run in libsdpa_mi355x.so: the forward is sdpa_fwd and the backward is
sdpa_bwd, which takes the forward's logsumexp. Following the pages' call sites (the
MPS SDPA pull request, "Unused second output"; mps-flash-sdpa, "Usage"), the
logsumexp is computed and kept only when an input requires a gradient, and a call is
checked for eligibility before anything runs. Where those pages fall back to the
unfused math path, an ineligible call here raises ValueError instead: every step of
the computation is meant to run in the library's kernels. Masks and sinks, which those
pages hand to the unfused path (mps-flash-sdpa, "When MFA Dispatches vs. Falls Back";
MLX pull request, "Limitations"), run in the library too: a boolean mask keeps the keys
where it is True, a mask of the operand dtype is added to the scaled scores, and the
sinks (float32, one logit per query head) get a gradient; the mask gets none.
"""

from __future__ import annotations

import math

import torch

from . import _lib

_DTYPES = (torch.float32, torch.float16, torch.bfloat16)
_HEAD_DIMS = (32, 64, 96, 128, 256)


def check_eligible(q, k, v, is_causal=False, attn_mask=None, sinks=None):
    """Raise ValueError naming the first reason the library cannot take these tensors."""
    ts = {"q": q, "k": k, "v": v}
    for name, t in ts.items():
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} is not a tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} is on {t.device}; the library runs on the GPU only")
        if t.dtype not in _DTYPES:
            raise ValueError(f"{name} has dtype {t.dtype}; supported: float32, float16, bfloat16")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, L, D], got shape {tuple(t.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError(f"q, k, v dtypes differ: {q.dtype}, {k.dtype}, {v.dtype}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v are on different devices")
    B, Hq, Lq, D = q.shape
    if k.shape != v.shape:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} differ")
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k/v {tuple(k.shape)} do not match q {tuple(q.shape)} in batch or head size")
    Hkv = k.shape[1]
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"query heads {Hq} are not a multiple of key/value heads {Hkv}")
    if D not in _HEAD_DIMS:
        raise ValueError(f"head size {D} is not supported (supported: {_HEAD_DIMS})")
    if is_causal and Lq > k.shape[2]:
        raise ValueError("causal attention needs Lq <= Lkv (sequences aligned at their ends)")
    if attn_mask is not None:
        if is_causal:
            raise ValueError("attn_mask and is_causal are not combined")
        if not isinstance(attn_mask, torch.Tensor) or attn_mask.device != q.device:
            raise ValueError("attn_mask must be a tensor on the device of q")
        if attn_mask.dtype not in (torch.bool, q.dtype):
            raise ValueError(f"attn_mask must be bool or {q.dtype}, got {attn_mask.dtype}")
        if attn_mask.requires_grad:
            raise ValueError("no gradient is formed for attn_mask")
        try:
            torch.broadcast_shapes(tuple(attn_mask.shape), (B, Hq, Lq, k.shape[2]))
        except RuntimeError:
            raise ValueError(f"attn_mask {tuple(attn_mask.shape)} does not broadcast to {(B, Hq, Lq, k.shape[2])}")
    if sinks is not None:
        if not isinstance(sinks, torch.Tensor) or sinks.device != q.device:
            raise ValueError("sinks must be a tensor on the device of q")
        if sinks.dtype != torch.float32 or tuple(sinks.shape) != (Hq,):
            raise ValueError(f"sinks must be float32 of shape ({Hq},)")


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, scale, is_causal, attn_mask, sinks):
        need_grad = any(ctx.needs_input_grad[:3]) or ctx.needs_input_grad[6]
        o, lse = _lib.sdpa_fwd(q, k, v, scale=scale, is_causal=is_causal, need_lse=need_grad, attn_mask=attn_mask,
                               sinks=sinks)
        if need_grad:
            ctx.save_for_backward(q, k, v, o, lse, attn_mask, sinks)
        ctx.scale, ctx.is_causal = scale, is_causal
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, attn_mask, sinks = ctx.saved_tensors
        grads = _lib.sdpa_bwd(q, k, v, o, lse, do.to(q.dtype).contiguous(), scale=ctx.scale, is_causal=ctx.is_causal,
                              attn_mask=attn_mask, sinks=sinks)
        dsinks = grads[3] if sinks is not None else None
        return grads[0], grads[1], grads[2], None, None, None, dsinks


def attention(q, k, v, scale=None, is_causal=False, attn_mask=None, sinks=None):
    """softmax(q k^T * scale [+ causal or attn_mask], with sinks) v for [B, H, L, D] tensors, differentiable.

    ``scale`` defaults to 1/sqrt(D), rounded to float32 as the library receives it.
    K and V may have fewer heads than Q (grouped-query attention). ``attn_mask``
    (bool, or q's dtype) broadcasts to [B, Hq, Lq, Lkv]; ``sinks`` is float32 [Hq]."""
    check_eligible(q, k, v, is_causal, attn_mask, sinks)
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(q.shape[-1]), dtype=torch.float32))
    return _Attention.apply(q.contiguous(), k.contiguous(), v.contiguous(), float(scale), bool(is_causal), attn_mask,
                            None if sinks is None else sinks.contiguous())
