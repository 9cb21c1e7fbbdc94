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
* The backward is the gradient of the scalar sum(O * dO) with respect to Q, K and
  V, written out with the softmax Jacobian:
      dV_j  = sum_i P_ij dO_i           (summed over the query heads of the group)
      dP_ij = dO_i . V_j
      Delta_i = sum_d dO_id O_id        (= sum_j P_ij dP_ij)
      dS_ij = P_ij (dP_ij - Delta_i)
      dQ_i  = scale * sum_j dS_ij K_j
      dK_j  = scale * sum_i dS_ij Q_i   (summed over the query heads of the group)

Parity pins (tests/test_oracle_pins.py): torch's CPU math attention and autograd
in float64, scipy's logsumexp, central finite differences of sum(O * dO), the
closed forms Lkv = 1, equal scores, causal row 0 and causal Q = 0, causal with
Lq < Lkv as the last rows of the square causal problem and with Lq = 1 as full
attention, and the invariants listed there. No function in this module is "parity
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


def head_forward(qh, kh, vh, scale, is_causal, rows=None):
    """Forward for one (batch, query head) pair, optionally on a subset of query rows.

    qh: [Lq, D], kh and vh: [Lkv, D]; rows: query indices (default all).
    Returns (O [n, D], LSE [n], P [n, Lkv]) in float64.
    """
    qh, kh, vh = _f64(qh), _f64(kh), _f64(vh)
    if rows is None:
        rows = np.arange(qh.shape[0])
    rows = np.asarray(rows)
    s = (qh[rows] @ kh.T) * float(scale)
    if is_causal:
        s = np.where(_causal_keep(rows, qh.shape[0], kh.shape[0]), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = p @ vh
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse, p


def attention_forward(q, k, v, scale, is_causal):
    """O [B,Hq,Lq,D] and LSE [B,Hq,Lq] (natural log) for BHLD inputs, float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Lq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    o = np.empty((B, Hq, Lq, D))
    lse = np.empty((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            o[b, h], lse[b, h], _ = head_forward(q[b, h], k[b, h // G], v[b, h // G], scale, is_causal)
    return o, lse


def head_backward(qh, kh, vh, doh, scale, is_causal, rows=None):
    """Backward contributions of one (batch, query head) pair.

    Returns (dQ rows [n, D], dK contribution [Lkv, D], dV contribution [Lkv, D],
    Delta [n]). With ``rows`` a subset, dK/dV are the contributions of those rows
    only; dQ and Delta are exact for the rows given.
    """
    qh, kh, vh, doh = _f64(qh), _f64(kh), _f64(vh), _f64(doh)
    if rows is None:
        rows = np.arange(qh.shape[0])
    rows = np.asarray(rows)
    o, _, p = head_forward(qh, kh, vh, scale, is_causal, rows)
    do = doh[rows]
    dv = p.T @ do
    dp = do @ vh.T
    delta = np.sum(do * o, axis=1)
    ds = p * (dp - delta[:, None])
    dq = float(scale) * (ds @ kh)
    dk = float(scale) * (ds.T @ qh[rows])
    return dq, dk, dv, delta


def group_backward(q, k, v, do, scale, is_causal, b, hk):
    """dQ for the G query heads of KV group (b, hk), and that group's dK, dV.

    Returns (dq [G, Lq, D], dk [Lkv, D], dv [Lkv, D]).
    """
    G = q.shape[1] // k.shape[1]
    dq = np.empty((G,) + tuple(q.shape[2:]))
    dk = np.zeros(k.shape[2:])
    dv = np.zeros(v.shape[2:])
    for g in range(G):
        h = hk * G + g
        dq[g], dkc, dvc, _ = head_backward(q[b, h], k[b, hk], v[b, hk], do[b, h], scale, is_causal)
        dk += dkc
        dv += dvc
    return dq, dk, dv


def attention_backward(q, k, v, do, scale, is_causal):
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
            dq[b, hk * G:(hk + 1) * G], dk[b, hk], dv[b, hk] = group_backward(q, k, v, do, scale, is_causal, b, hk)
    return dq, dk, dv
