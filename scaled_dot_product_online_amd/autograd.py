"""torch.autograd wrapper over the C ABI.

    attention(q, k, v, scale=None, is_causal=False) -> o

Both directions run in libsdpa_mi355x.so: the forward is sdpa_fwd and the backward is
sdpa_bwd, which takes the forward's logsumexp. Following the pages' call sites (the
MPS SDPA pull request, "Unused second output"; mps-flash-sdpa, "Usage"), the
logsumexp is computed and kept only when an input requires a gradient, and a call is
checked for eligibility before anything runs. Where those pages fall back to the
unfused math path, an ineligible call here raises ValueError instead: every step of
the computation is meant to run in the library's kernels.
"""

from __future__ import annotations

import math

import torch

from . import _lib

_DTYPES = (torch.float32, torch.float16, torch.bfloat16)
_HEAD_DIMS = (32, 64, 96, 128, 256)


def check_eligible(q, k, v, is_causal=False):
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


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, scale, is_causal):
        need_grad = any(ctx.needs_input_grad[:3])
        o, lse = _lib.sdpa_fwd(q, k, v, scale=scale, is_causal=is_causal, need_lse=need_grad)
        if need_grad:
            ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.is_causal = scale, is_causal
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = _lib.sdpa_bwd(q, k, v, o, lse, do.to(q.dtype).contiguous(), scale=ctx.scale,
                                   is_causal=ctx.is_causal)
        return dq, dk, dv, None, None


def attention(q, k, v, scale=None, is_causal=False):
    """softmax(q k^T * scale [+ causal mask]) v for [B, H, L, D] tensors, differentiable.

    ``scale`` defaults to 1/sqrt(D), rounded to float32 as the library receives it.
    K and V may have fewer heads than Q (grouped-query attention)."""
    check_eligible(q, k, v, is_causal)
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(q.shape[-1]), dtype=torch.float32))
    return _Attention.apply(q.contiguous(), k.contiguous(), v.contiguous(), float(scale), bool(is_causal))
