"""fp64 reference definition of scaled-dot-product attention, forward and backward.

Test infrastructure only (see the package docstring): never imported by the
product library.

Sources (pages, cited by title and section)
-------------------------------------------
* PyTensor issue "PERF: detect scaled-dot-product-attention pattern and lower to
  mx.fast.scaled_dot_product_attention", section "Sketch": the forward is the
  ``perform()`` of the proposed Op — scores are ``(q @ k^T) * scale``, the row
  maximum is subtracted, the exponentials are normalised by their row sum, and the
  result multiplies ``v``. Section "Current implementation" states the same
  expression ``softmax((Q @ K^T) * scale) @ V``.
* mps-flash-sdpa 0.1.0, section "Quick Start": tensors are laid out
  ``[B, H, S, D]`` and ``is_causal`` selects causal masking.
* MLX pull request "[Metal] Add Flash Attention VJP for training", sections
  "Key Features" (GQA and causal support, logsumexp cached by the forward) and the
  author's reply listing what the backward does (recompute the scores, load the
  logsumexp, form P = exp(S - LSE), compute the gradients).
* MPS SDPA issue (stepcodex), section "Problem - Unused second output tensor": the
  forward's second output is what the backward needs.

Readings where the pages are silent
-----------------------------------
* Causal masking keeps key j for query i iff j <= i + (Lkv - Lq): the query and key
  sequences are aligned at their ends (the last query sees every key, as when new
  queries attend to a key/value cache). With Lq == Lkv this is j <= i. The pages name
  unequal query and key lengths only as a test edge case (MLX pull request "[Metal]
  Add Flash Attention VJP for training", "Test Plan"), not the alignment; Lq <= Lkv
  is required so that every query row sees at least one key.
* GQA: query head h reads key/value head h // (Hq // Hkv) (contiguous groups).
* The logsumexp is the natural log of sum_j exp(s_ij) over the *scaled* scores.
* Masks and sinks. The pages name attention masks (float masks, and boolean masks
  with False entries) and attention sinks only as cases where a fused path falls
  back to the unfused one (mps-flash-sdpa 0.1.0, "When MFA Dispatches vs. Falls
  Back"; MLX pull request "[Metal] Add Flash Attention VJP for training",
  "Limitations"). PyTensor's issue places a mask as a term added to the scaled
  scores before the softmax and leaves it to a later extension with optional inputs
  ("Important guards in the matcher"). Read as the drop-in API those pages target
  (PyTorch's scaled_dot_product_attention):
  - a boolean mask keeps key j for query i where it is True; a float mask is added
    to the scaled scores; either broadcasts to [B, Hq, Lq, Lkv]. A float mask holds
    no +inf or NaN; -inf removes a key as False does. The mask is a constant: no
    gradient is formed for it. A mask and the causal flag are not combined.
  - a sink is one logit per query head (in the units of the scaled scores) that
    joins every row's softmax denominator and carries no value:
        LSE_i = log(exp(sink_h) + sum_j exp(s_ij)),  P_ij = exp(s_ij - LSE_i).
    Its gradient for the loss sum(O * dO) is dsink_h = -sum_{b,i} exp(sink_h - LSE_i) Delta_i
    (the sink's own dP is 0, since it has no value row).
  - a row that sees no key and has no sink has O = 0, LSE = -inf and contributes
    no gradient.
* The backward is the gradient of the scalar sum(O * dO) with respect to Q, K and
  V, written out with the softmax Jacobian:
      dV_j  = sum_i P_ij dO_i           (summed over the query heads of the group)
      dP_ij = dO_i . V_j
      Delta_i = sum_d dO_id O_id        (= sum_j P_ij dP_ij)
      dS_ij = P_ij (dP_ij - Delta_i)
      dQ_i  = scale * sum_j dS_ij K_j
      dK_j  = scale * sum_i dS_ij Q_i   (summed over the query heads of the group)

Parity pins (tests/test_oracle_pins.py): torch's CPU math attention and autograd
in float64 (with boolean and float masks as well), scipy's logsumexp, central finite
differences of sum(O * dO) (also for the sink), the closed forms Lkv = 1, equal
scores, causal row 0 and causal Q = 0, causal with Lq < Lkv as the last rows of the
square causal problem and with Lq = 1 as full attention, a key-padding mask as
attention over the kept keys only, a sink as one extra key with a zero value row in
a head dimension widened by one, and the invariants listed there. No function in this module is "parity
unpinned".
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _causal_keep(rows, n_queries, n_keys):
    """Boolean [len(rows), n_keys]: True where key j is visible to query i,
    j <= i + (n_keys - n_queries) (sequences aligned at their ends)."""
    if n_queries > n_keys:
        raise ValueError("causal attention needs Lq <= Lkv")
    rows = np.asarray(rows)
    return np.arange(n_keys)[None, :] <= rows[:, None] + (n_keys - n_queries)


def mask_bias(mask):
    """The additive form of a mask: a boolean mask gives 0 where True and -inf where
    False; a float mask is its own bias."""
    m = np.asarray(mask)
    if m.dtype == np.bool_:
        return np.where(m, 0.0, -np.inf)
    return m.astype(np.float64)


def head_bias(mask, B, Hq, Lq, Lkv, b, h):
    """The [Lq, Lkv] float64 bias of (batch b, query head h), or None without a mask."""
    if mask is None:
        return None
    return np.broadcast_to(mask_bias(mask), (B, Hq, Lq, Lkv))[b, h]


def head_forward(qh, kh, vh, scale, is_causal, rows=None, bias=None, sink=None):
    """Forward for one (batch, query head) pair, optionally on a subset of query rows.

    qh: [Lq, D], kh and vh: [Lkv, D]; rows: query indices (default all); bias: this
    head's additive mask [Lq, Lkv] or None; sink: this head's sink logit or None.
    Returns (O [n, D], LSE [n], P [n, Lkv]) in float64.
    """
    qh, kh, vh = _f64(qh), _f64(kh), _f64(vh)
    if rows is None:
        rows = np.arange(qh.shape[0])
    rows = np.asarray(rows)
    s = (qh[rows] @ kh.T) * float(scale)
    if is_causal:
        s = np.where(_causal_keep(rows, qh.shape[0], kh.shape[0]), s, -np.inf)
    if bias is not None:
        s = s + _f64(bias)[rows]
    m = s.max(axis=1, keepdims=True)
    if sink is not None:
        m = np.maximum(m, float(sink))
    m = np.where(np.isfinite(m), m, 0.0)  # a row with no key and no sink: every term is 0
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    if sink is not None:
        l = l + np.exp(float(sink) - m)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(l > 0, e / l, 0.0)
        lse = np.where(l[:, 0] > 0, m[:, 0] + np.log(l[:, 0]), -np.inf)
    o = p @ vh
    return o, lse, p


def _check_mask(mask, is_causal):
    if mask is not None and is_causal:
        raise ValueError("a mask and the causal flag are not combined")


def attention_forward(q, k, v, scale, is_causal, mask=None, sinks=None):
    """O [B,Hq,Lq,D] and LSE [B,Hq,Lq] (natural log) for BHLD inputs, float64.

    mask: boolean or float, broadcastable to [B, Hq, Lq, Lkv]; sinks: [Hq] or None."""
    _check_mask(mask, is_causal)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Lq, D = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    o = np.empty((B, Hq, Lq, D))
    lse = np.empty((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            o[b, h], lse[b, h], _ = head_forward(q[b, h], k[b, h // G], v[b, h // G], scale, is_causal,
                                                 bias=head_bias(mask, B, Hq, Lq, Lkv, b, h),
                                                 sink=None if sinks is None else sinks[h])
    return o, lse


def head_backward(qh, kh, vh, doh, scale, is_causal, rows=None, bias=None, sink=None):
    """Backward contributions of one (batch, query head) pair.

    Returns (dQ rows [n, D], dK contribution [Lkv, D], dV contribution [Lkv, D],
    Delta [n]). With ``rows`` a subset, dK/dV are the contributions of those rows
    only; dQ and Delta are exact for the rows given. bias and sink as in head_forward.
    """
    qh, kh, vh, doh = _f64(qh), _f64(kh), _f64(vh), _f64(doh)
    if rows is None:
        rows = np.arange(qh.shape[0])
    rows = np.asarray(rows)
    o, _, p = head_forward(qh, kh, vh, scale, is_causal, rows, bias=bias, sink=sink)
    do = doh[rows]
    dv = p.T @ do
    dp = do @ vh.T
    delta = np.sum(do * o, axis=1)
    ds = p * (dp - delta[:, None])
    dq = float(scale) * (ds @ kh)
    dk = float(scale) * (ds.T @ qh[rows])
    return dq, dk, dv, delta


def group_backward(q, k, v, do, scale, is_causal, b, hk, mask=None, sinks=None):
    """dQ for the G query heads of KV group (b, hk), and that group's dK, dV.

    Returns (dq [G, Lq, D], dk [Lkv, D], dv [Lkv, D]).
    """
    _check_mask(mask, is_causal)
    B, Hq, Lq = q.shape[:3]
    Lkv = k.shape[2]
    G = Hq // k.shape[1]
    dq = np.empty((G,) + tuple(q.shape[2:]))
    dk = np.zeros(k.shape[2:])
    dv = np.zeros(v.shape[2:])
    for g in range(G):
        h = hk * G + g
        dq[g], dkc, dvc, _ = head_backward(q[b, h], k[b, hk], v[b, hk], do[b, h], scale, is_causal,
                                           bias=head_bias(mask, B, Hq, Lq, Lkv, b, h),
                                           sink=None if sinks is None else sinks[h])
        dk += dkc
        dv += dvc
    return dq, dk, dv


def attention_backward(q, k, v, do, scale, is_causal, mask=None, sinks=None):
    """dQ [B,Hq,Lq,D], dK and dV [B,Hkv,Lkv,D] for the loss sum(O * dO), float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq = q.shape[:2]
    Hkv = k.shape[1]
    G = Hq // Hkv
    dq = np.empty(q.shape)
    dk = np.empty(k.shape)
    dv = np.empty(v.shape)
    for b in range(B):
        for hk in range(Hkv):
            dq[b, hk * G:(hk + 1) * G], dk[b, hk], dv[b, hk] = group_backward(q, k, v, do, scale, is_causal, b, hk,
                                                                              mask=mask, sinks=sinks)
    return dq, dk, dv


def sink_gradient(q, k, v, do, scale, is_causal, sinks, mask=None):
    """dsinks [Hq] for the loss sum(O * dO): -sum over batch and rows of
    exp(sink_h - LSE_i) * Delta_i, with Delta_i = sum_d dO_id O_id."""
    do = _f64(do)
    o, lse = attention_forward(q, k, v, scale, is_causal, mask=mask, sinks=sinks)
    delta = np.sum(do * o, axis=3)
    s = _f64(sinks)[None, :, None]
    with np.errstate(invalid="ignore"):
        w = np.where(np.isfinite(s), np.exp(s - lse), 0.0)
    return -np.sum(w * delta, axis=(0, 2))
