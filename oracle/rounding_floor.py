"""Rounding-point model of a 16-bit matrix-core attention kernel (test infrastructure only).

Why this exists
---------------
The accuracy figures on the pages (mps-flash-sdpa 0.1.0, section "Gradient
Correctness": fp16 ~5e-4 / ~2e-3, bf16 ~1e-3 / ~1e-3 forward / backward max
difference) were measured against PyTorch's math attention *in the same dtype*.
Measured against an fp64 definition, a kernel whose matrix products take 16-bit
operands cannot beat the error that the rounding of those operands and of the
stored outputs alone produces: storing a bf16 output near |x| = 3 already costs
up to 2^-8 * 2 = 7.8e-3. This module computes that floor, F, for the same inputs,
so that a parity test can state its bound as ``max|gpu - exact| <= tol + F`` per
output tensor, and can also check the kernel against the model directly.

What is modelled (the kernel's rounding points, nothing else)
-------------------------------------------------------------
Forward, with the scores kept exact:
* the probabilities that enter the P.V product are rounded to the operand dtype
  *relative to the reference maximum in force when their key block was processed*
  (online softmax; MLX pull request "[Metal] Add Flash Attention VJP for
  training", section "Implementation Notes", log2-domain exponentials). The
  reference restarts at every ``kv_segment`` keys and may move every ``kv_block``
  keys, when the block's maximum exceeds it by more than ``slack``; the
  unrounded exponentials form the denominator;
* the output is rounded to the output dtype.
A mask enters the scores as in the definition; a sink starts every row's reference
maximum (the kernels enter it before the first key block) and joins the denominator.
Backward:
* Delta_i uses the *stored* (rounded) forward output, as the kernel does;
* P (from the exact logsumexp) is rounded before the dV product, dS before the dQ
  and dK products; the results are rounded to the output dtype.
Everything else is exact float64. Accumulation-order effects of fp32 are not
modelled; they are orders of magnitude below the 16-bit terms.

This is not the oracle: ``sdpa_reference`` is the definition, and a parity test
never passes on this model alone (its bound always includes the distance to the
definition). Pins: ``round_to`` against IEEE conversions and exhaustive bf16
spacing checks; with ``op_dtype = out_dtype = "f64"`` the model reproduces the
definition exactly; at 16 bits the backward's error stays within the rigorous
per-element bounds of its two roundings, has the size that rounding-error theory
predicts for them, vanishes when every rounded operand is representable, and responds
to the stored output through Delta as the first-order formula says
(tests/test_oracle_pins.py).
"""

from __future__ import annotations

import numpy as np

_DTYPES = ("f64", "f32", "f16", "bf16")


def round_to(x, dtype):
    """Round float64 values to ``dtype`` (round to nearest, ties to even) and widen back."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        f = x.astype(np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
        return u.astype(np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}; expected one of {_DTYPES}")


def _running_max(s, kv_block, kv_segment, slack=0.0, start=-np.inf):
    """Per score element, the row's reference maximum in force when its key block is processed.

    The reference starts at ``start`` (-inf, or the sink) at every segment start and is
    replaced by a block's maximum when that maximum exceeds it by more than ``slack``
    (natural-log units); with slack 0 this is the ordinary running maximum."""
    n, L = s.shape
    nblk = -(-L // kv_block)
    pad = np.full((n, nblk * kv_block), -np.inf)
    pad[:, :L] = s
    bmax = pad.reshape(n, nblk, kv_block).max(axis=2)
    seg_blocks = nblk if kv_segment is None else kv_segment // kv_block
    if kv_segment is not None and kv_segment % kv_block:
        raise ValueError("kv_segment must be a multiple of kv_block")
    run = np.empty_like(bmax)
    for s0 in range(0, nblk, seg_blocks):
        m = np.full(n, float(start))
        for j in range(s0, min(s0 + seg_blocks, nblk)):
            m = np.where(bmax[:, j] > m + slack, bmax[:, j], m)
            run[:, j] = m
    return np.repeat(run, kv_block, axis=1)[:, :L]


def _bias_of(mask, B, Hq, Lq, Lkv, b, h):
    """[Lq, Lkv] additive bias of (b, h): 0 / -inf for a boolean mask, the values of a float one."""
    if mask is None:
        return None
    m = np.asarray(mask)
    full = np.where(m, 0.0, -np.inf) if m.dtype == np.bool_ else m.astype(np.float64)
    return np.broadcast_to(full, (B, Hq, Lq, Lkv))[b, h]


def emulate_forward_head(qh, kh, vh, scale, is_causal, op_dtype, out_dtype, kv_block, kv_segment=None, rows=None,
                         slack=0.0, bias=None, sink=None):
    """Modelled kernel output O (already rounded to ``out_dtype``) for one head."""
    qh, kh, vh = (np.asarray(a, dtype=np.float64) for a in (qh, kh, vh))
    if rows is None:
        rows = np.arange(qh.shape[0])
    rows = np.asarray(rows)
    s = (qh[rows] @ kh.T) * float(scale)
    if is_causal:
        s = np.where(np.arange(kh.shape[0])[None, :] <= rows[:, None] + (kh.shape[0] - qh.shape[0]), s, -np.inf)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)[rows]
    start = -np.inf if sink is None else float(sink)
    m_final = np.maximum(s.max(axis=1, keepdims=True), start)
    m_final = np.where(np.isfinite(m_final), m_final, 0.0)
    m_run = _running_max(s, kv_block, kv_segment, slack, start)
    with np.errstate(invalid="ignore"):
        p_tilde = np.where(np.isfinite(s), np.exp(s - m_run), 0.0)
        w = np.where(np.isfinite(m_run), np.exp(m_run - m_final), 0.0)
    r = round_to(p_tilde, op_dtype) * w
    denom = np.exp(s - m_final).sum(axis=1, keepdims=True) + np.exp(start - m_final)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(denom > 0, (r @ vh) / denom, 0.0)
    return round_to(out, out_dtype)


def emulate_forward(q, k, v, scale, is_causal, op_dtype, out_dtype, kv_block, kv_segment=None, slack=0.0, mask=None,
                    sinks=None):
    """Modelled kernel output O [B,Hq,Lq,D], rounded to ``out_dtype``."""
    B, Hq, Lq = q.shape[:3]
    Lkv = k.shape[2]
    G = Hq // k.shape[1]
    o = np.empty(q.shape, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            o[b, h] = emulate_forward_head(q[b, h], k[b, h // G], v[b, h // G], scale, is_causal,
                                           op_dtype, out_dtype, kv_block, kv_segment, slack=slack,
                                           bias=_bias_of(mask, B, Hq, Lq, Lkv, b, h),
                                           sink=None if sinks is None else sinks[h])
    return o


# The backward's two operand roundings, named so that a test can check each one's effect
# (tests/test_oracle_pins.py plants a slip in them and sees it caught): the probabilities
# enter the dV product rounded to the operand type; dS enters the dQ and dK products
# rounded to the operand type *before* the scale is applied (the kernels multiply the
# fp32 accumulators by the scale once, at the end).
def round_p(p, op_dtype):
    return round_to(p, op_dtype)


def round_ds(ds, op_dtype, scale):
    return round_to(ds, op_dtype)


def emulate_backward_group(q, k, v, do, o_stored, lse, scale, is_causal, op_dtype, out_dtype, b, hk, mask=None):
    """Modelled dQ [G,Lq,D], dK, dV [Lkv,D] of KV group (b, hk), rounded to ``out_dtype``.

    ``o_stored`` and ``lse`` are the forward's stored output and logsumexp
    ([B,Hq,Lq,D] and [B,Hq,Lq]); a sink acts only through the logsumexp.
    """
    B, Hq, Hkv = q.shape[0], q.shape[1], k.shape[1]
    G = Hq // Hkv
    kh = np.asarray(k[b, hk], dtype=np.float64)
    vh = np.asarray(v[b, hk], dtype=np.float64)
    Lq, Lkv = q.shape[2], kh.shape[0]
    dq = np.empty((G, Lq, kh.shape[1]))
    dk = np.zeros(kh.shape)
    dv = np.zeros(vh.shape)
    for g in range(G):
        h = hk * G + g
        qh = np.asarray(q[b, h], dtype=np.float64)
        doh = np.asarray(do[b, h], dtype=np.float64)
        s = (qh @ kh.T) * float(scale)
        bias = _bias_of(mask, B, Hq, Lq, Lkv, b, h)
        if bias is not None:
            s = s + bias
        lse_h = np.asarray(lse[b, h], dtype=np.float64)[:, None]
        with np.errstate(invalid="ignore"):
            p = np.where(np.isfinite(lse_h), np.exp(s - lse_h), 0.0)
        if is_causal:
            p = np.where(np.arange(Lkv)[None, :] <= np.arange(Lq)[:, None] + (Lkv - Lq), p, 0.0)
        delta = np.sum(doh * np.asarray(o_stored[b, h], dtype=np.float64), axis=1)
        dp = doh @ vh.T
        ds = p * (dp - delta[:, None])
        rp = round_p(p, op_dtype)
        rds = round_ds(ds, op_dtype, scale)
        dv += rp.T @ doh
        dq[g] = float(scale) * (rds @ kh)
        dk += float(scale) * (rds.T @ qh)
    return round_to(dq, out_dtype), round_to(dk, out_dtype), round_to(dv, out_dtype)


def emulate_dq_rows(qh, kh, vh, doh, o_stored, lse, scale, is_causal, op_dtype, rows, bias=None):
    """Modelled dQ (before its final rounding) of query rows ``rows`` of one head.

    ``o_stored`` and ``lse`` are the stored output and logsumexp of those rows. The
    rounding points are those of ``emulate_backward_group``: Delta from the stored
    output, dS rounded to the operand type before the product with K, then the scale."""
    qh, kh, vh, doh = (np.asarray(a, dtype=np.float64) for a in (qh, kh, vh, doh))
    rows = np.asarray(rows)
    Lq, Lkv = qh.shape[0], kh.shape[0]
    s = (qh[rows] @ kh.T) * float(scale)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)[rows]
    lse = np.asarray(lse, dtype=np.float64)[:, None]
    with np.errstate(invalid="ignore"):
        p = np.where(np.isfinite(lse), np.exp(s - lse), 0.0)
    if is_causal:
        p = np.where(np.arange(Lkv)[None, :] <= rows[:, None] + (Lkv - Lq), p, 0.0)
    do = doh[rows]
    delta = np.sum(do * np.asarray(o_stored, dtype=np.float64), axis=1)
    ds = p * (do @ vh.T - delta[:, None])
    return float(scale) * (round_ds(ds, op_dtype, scale) @ kh)


def emulate_backward(q, k, v, do, o_stored, lse, scale, is_causal, op_dtype, out_dtype, mask=None):
    """Modelled dQ, dK, dV for all groups, rounded to ``out_dtype``."""
    B, Hq = q.shape[:2]
    Hkv = k.shape[1]
    G = Hq // Hkv
    dq = np.empty(q.shape)
    dk = np.empty(k.shape)
    dv = np.empty(v.shape)
    for b in range(B):
        for hk in range(Hkv):
            dq[b, hk * G:(hk + 1) * G], dk[b, hk], dv[b, hk] = emulate_backward_group(
                q, k, v, do, o_stored, lse, scale, is_causal, op_dtype, out_dtype, b, hk, mask=mask)
    return dq, dk, dv


def emulate_sink_gradient(do, o_stored, lse, sinks):
    """Modelled dsinks [Hq]: the kernel forms Delta from the *stored* output, then
    -sum_{b,i} exp(sink_h - LSE_i) Delta_i exactly (float64 here); returns
    (dsinks, magnitude) where magnitude[h] = sum_{b,i} |exp(sink_h - LSE_i) Delta_i|,
    the scale of the sum's rounding error."""
    do = np.asarray(do, dtype=np.float64)
    delta = np.sum(do * np.asarray(o_stored, dtype=np.float64), axis=3)
    s = np.asarray(sinks, dtype=np.float64)[None, :, None]
    with np.errstate(invalid="ignore"):
        w = np.where(np.isfinite(s), np.exp(s - np.asarray(lse, dtype=np.float64)), 0.0)
    return -np.sum(w * delta, axis=(0, 2)), np.sum(np.abs(w * delta), axis=(0, 2))
