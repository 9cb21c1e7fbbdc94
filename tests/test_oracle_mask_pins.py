"""Pins of the oracle's masks and sinks to things other than itself (CPU only).

Readings (oracle/sdpa_reference.py, "Masks and sinks"): a boolean mask keeps the
keys where it is True, a float mask is added to the scaled scores, both broadcast to
[B, Hq, Lq, Lkv]; a sink is one logit per query head that joins every row's softmax
denominator and carries no value.

Independent references:
* torch's CPU math attention with ``attn_mask`` (boolean and float) and torch
  autograd, in float64: the API whose semantics the reading adopts;
* attention over the kept keys only (a key-padding mask), computed by the oracle
  without a mask on the truncated K and V;
* a sink as one extra key whose value row is zero, in a head dimension widened by one
  (q' = [q, 1], k_sink = [0, sink / scale]), computed by the oracle without a sink;
  the sink's gradient is then that key's last gradient component times 1 / scale;
* central finite differences of sum(O * dO) with respect to the sinks;
* the closed form O_sink = O * exp(LSE - LSE_sink), LSE_sink = logaddexp(LSE, sink);
* invariants: a row-constant bias changes nothing but the LSE, an all-True mask is no
  mask, a causal-pattern boolean mask is the causal flag, a -inf sink is no sink.
"""

import math

import numpy as np
import pytest

from oracle import sdpa_reference as ref
from oracle.rounding_floor import emulate_backward, emulate_forward

RNG = np.random.default_rng(4321)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def torch_masked(q, k, v, do, scale, mask):
    import torch
    import torch.nn.functional as F

    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    tm = torch.tensor(mask) if mask.dtype == np.bool_ else torch.tensor(mask, dtype=torch.float64)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale, enable_gqa=q.shape[1] != k.shape[1])
    (o * torch.tensor(do)).sum().backward()
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def _bool_mask(shape, p_keep=0.6):
    m = RNG.random(shape) < p_keep
    m[..., 0] = True  # every row keeps a key: torch's math path has no convention for empty rows
    return m


MASK_CASES = [
    # B, Hq, Hkv, Lq, Lkv, D, mask shape (broadcast to [B, Hq, Lq, Lkv]), kind
    (2, 4, 2, 5, 9, 8, (2, 4, 5, 9), "bool"),
    (2, 4, 2, 5, 9, 8, (2, 1, 1, 9), "bool"),      # key padding per batch
    (1, 6, 3, 7, 7, 4, (1, 1, 7, 7), "bool"),      # one pattern for every head
    (2, 4, 1, 6, 11, 8, (2, 4, 6, 11), "float"),
    (1, 2, 2, 8, 8, 16, (1, 2, 1, 8), "float"),    # per-head key bias
    (2, 2, 1, 1, 13, 8, (2, 1, 1, 13), "float"),   # one query row
]


@pytest.mark.parametrize("case", MASK_CASES)
def test_masks_match_torch_math_attention_fp64(case):
    B, Hq, Hkv, Lq, Lkv, D, mshape, kind = case
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D), rand(B, Hq, Lq, D)
    mask = _bool_mask(mshape) if kind == "bool" else rand(*mshape, scale=2.0)
    scale = 1.0 / math.sqrt(D)
    o, _ = ref.attention_forward(q, k, v, scale, False, mask=mask)
    dq, dk, dv = ref.attention_backward(q, k, v, do, scale, False, mask=mask)
    to, tdq, tdk, tdv = torch_masked(q, k, v, do, scale, mask)
    for got, want in ((o, to), (dq, tdq), (dk, tdk), (dv, tdv)):
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_key_padding_mask_is_attention_over_the_kept_keys():
    B, Hq, Hkv, Lq, Lkv, D = 2, 4, 2, 6, 10, 8
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D), rand(B, Hq, Lq, D)
    keep = np.array([7, 10])  # batch 0 keeps its first 7 keys, batch 1 all of them
    mask = np.arange(Lkv)[None, None, None, :] < keep[:, None, None, None]
    scale = 0.4
    o, lse = ref.attention_forward(q, k, v, scale, False, mask=mask)
    dq, dk, dv = ref.attention_backward(q, k, v, do, scale, False, mask=mask)
    for b in range(B):
        n = keep[b]
        ob, lseb = ref.attention_forward(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], scale, False)
        dqb, dkb, dvb = ref.attention_backward(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], do[b:b + 1], scale,
                                               False)
        np.testing.assert_allclose(o[b:b + 1], ob, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b:b + 1], lseb, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dq[b:b + 1], dqb, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dk[b:b + 1, :, :n], dkb, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dv[b:b + 1, :, :n], dvb, rtol=1e-11, atol=1e-12)
        assert np.all(dk[b, :, n:] == 0) and np.all(dv[b, :, n:] == 0)


def test_row_constant_bias_and_trivial_masks():
    B, Hq, Hkv, Lq, Lkv, D = 1, 4, 2, 7, 7, 8
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D), rand(B, Hq, Lq, D)
    scale = 0.3
    o0, lse0 = ref.attention_forward(q, k, v, scale, False)
    g0 = ref.attention_backward(q, k, v, do, scale, False)
    # A bias that is constant along each row shifts the scores of the row: O, dQ, dK, dV
    # are unchanged and the LSE moves by the constant.
    c = rand(B, Hq, Lq, 1, scale=3.0)
    o1, lse1 = ref.attention_forward(q, k, v, scale, False, mask=np.broadcast_to(c, (B, Hq, Lq, Lkv)))
    g1 = ref.attention_backward(q, k, v, do, scale, False, mask=np.broadcast_to(c, (B, Hq, Lq, Lkv)))
    np.testing.assert_allclose(o1, o0, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse1, lse0 + c[..., 0], rtol=1e-12, atol=1e-12)
    for a, b in zip(g1, g0):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)
    # An all-True boolean mask is no mask; the causal pattern as a boolean mask is the flag.
    o2, _ = ref.attention_forward(q, k, v, scale, False, mask=np.ones((1, 1, Lq, Lkv), bool))
    np.testing.assert_array_equal(o2, o0)
    tri = np.tril(np.ones((Lq, Lkv), bool))[None, None]
    oc, lsec = ref.attention_forward(q, k, v, scale, True)
    om, lsem = ref.attention_forward(q, k, v, scale, False, mask=tri)
    np.testing.assert_allclose(om, oc, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lsem, lsec, rtol=1e-13, atol=1e-14)
    for a, b in zip(ref.attention_backward(q, k, v, do, scale, False, mask=tri),
                    ref.attention_backward(q, k, v, do, scale, True)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    with pytest.raises(ValueError):
        ref.attention_forward(q, k, v, scale, True, mask=tri)


def test_fully_masked_rows_are_zero():
    B, Hq, Hkv, Lq, Lkv, D = 1, 2, 1, 4, 5, 8
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D), rand(B, Hq, Lq, D)
    mask = np.ones((1, 1, Lq, Lkv), bool)
    mask[0, 0, 2, :] = False  # query 2 sees nothing
    o, lse = ref.attention_forward(q, k, v, 0.5, False, mask=mask)
    dq, dk, dv = ref.attention_backward(q, k, v, do, 0.5, False, mask=mask)
    assert np.all(o[:, :, 2] == 0) and np.all(np.isneginf(lse[:, :, 2]))
    assert np.all(dq[:, :, 2] == 0)
    # The other rows are the unmasked problem; the empty row contributes nothing to dK/dV.
    rows = [0, 1, 3]
    o_r, lse_r = ref.attention_forward(q[:, :, rows], k, v, 0.5, False)
    dq_r, dk_r, dv_r = ref.attention_backward(q[:, :, rows], k, v, do[:, :, rows], 0.5, False)
    np.testing.assert_allclose(o[:, :, rows], o_r, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dq[:, :, rows], dq_r, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, dk_r, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, dv_r, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_sink_is_an_extra_key_with_a_zero_value_row(causal):
    B, H, Lq, Lkv, D = 2, 3, 6, 6, 8  # one KV head per query head: one extra key per head
    q, k, v, do = rand(B, H, Lq, D), rand(B, H, Lkv, D), rand(B, H, Lkv, D), rand(B, H, Lq, D)
    sinks = np.array([0.7, -1.5, 2.5])
    scale = 0.35
    o, lse = ref.attention_forward(q, k, v, scale, causal, sinks=sinks)
    dq, dk, dv = ref.attention_backward(q, k, v, do, scale, causal, sinks=sinks)
    ds = ref.sink_gradient(q, k, v, do, scale, causal, sinks)
    # Widen D by one: q' = [q, 1]; keys [k, 0] plus the sink key [0, sink/scale] placed
    # first, with a zero value row (values widened by a zero column). Causal: the sink key is visible to every query, which
    # end-aligned causal masking over Lkv + 1 keys gives when it is key 0.
    qa = np.concatenate([q, np.ones((B, H, Lq, 1))], axis=3)
    ks = np.zeros((B, H, 1, D + 1))
    ks[..., D] = (sinks / scale)[None, :, None]
    ka = np.concatenate([ks, np.concatenate([k, np.zeros((B, H, Lkv, 1))], axis=3)], axis=2)
    va = np.concatenate([np.zeros((B, H, 1, D + 1)), np.concatenate([v, np.zeros((B, H, Lkv, 1))], axis=3)], axis=2)
    doa = np.concatenate([do, np.zeros((B, H, Lq, 1))], axis=3)  # the same loss: O' has a zero last column
    if causal:  # keep key 0 for every query: the end-aligned causal rule over Lkv + 1 keys does
        mask = np.concatenate([np.ones((Lq, 1), bool), np.tril(np.ones((Lq, Lkv), bool))], axis=1)[None, None]
        oa, lsea = ref.attention_forward(qa, ka, va, scale, False, mask=mask)
        dqa, dka, dva = ref.attention_backward(qa, ka, va, doa, scale, False, mask=mask)
    else:
        oa, lsea = ref.attention_forward(qa, ka, va, scale, False)
        dqa, dka, dva = ref.attention_backward(qa, ka, va, doa, scale, False)
    np.testing.assert_allclose(o, oa[..., :D], rtol=1e-12, atol=1e-13)
    assert np.all(oa[..., D] == 0)
    np.testing.assert_allclose(lse, lsea, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq, dqa[..., :D], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, dka[:, :, 1:, :D], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, dva[:, :, 1:, :D], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ds, dka[:, :, 0, D].sum(axis=0) / scale, rtol=1e-10, atol=1e-12)


def test_sink_gradient_matches_finite_differences_and_closed_form():
    B, Hq, Hkv, Lq, Lkv, D = 2, 4, 2, 5, 7, 8
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D), rand(B, Hq, Lq, D)
    sinks = np.array([0.3, -0.8, 1.9, -np.inf])  # the last head has no sink
    mask = _bool_mask((B, 1, Lq, Lkv))
    scale = 0.4
    ds = ref.sink_gradient(q, k, v, do, scale, False, sinks, mask=mask)
    eps = 1e-5
    for h in range(3):
        fd = []
        for sgn in (1, -1):
            sp = sinks.copy()
            sp[h] += sgn * eps
            fd.append(np.sum(ref.attention_forward(q, k, v, scale, False, mask=mask, sinks=sp)[0] * do))
        assert abs((fd[0] - fd[1]) / (2 * eps) - ds[h]) < 1e-7 * max(1.0, abs(ds[h]))
    assert ds[3] == 0.0
    # Closed form against the no-sink problem.
    o0, lse0 = ref.attention_forward(q, k, v, scale, False, mask=mask)
    o1, lse1 = ref.attention_forward(q, k, v, scale, False, mask=mask, sinks=sinks)
    lse_want = np.logaddexp(lse0, sinks[None, :, None])
    np.testing.assert_allclose(lse1, lse_want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o1, o0 * np.exp(lse0 - lse_want)[..., None], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(o1[:, 3], o0[:, 3])


def test_sink_keeps_a_fully_masked_row_defined():
    B, Hq, Hkv, Lq, Lkv, D = 1, 1, 1, 2, 3, 4
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D), rand(B, Hq, Lq, D)
    mask = np.array([[[[True, True, False], [False, False, False]]]])
    o, lse = ref.attention_forward(q, k, v, 1.0, False, mask=mask, sinks=np.array([0.25]))
    assert np.all(o[0, 0, 1] == 0) and lse[0, 0, 1] == 0.25  # only the sink: P_sink = 1
    ds = ref.sink_gradient(q, k, v, do, 1.0, False, np.array([0.25]), mask=mask)
    assert np.isfinite(ds).all()


@pytest.mark.parametrize("kind", ["bool", "float"])
def test_rounding_model_with_mask_and_sink_reduces_to_definition(kind):
    B, Hq, Hkv, Lq, Lkv, D = 1, 4, 2, 9, 40, 8
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D), rand(B, Hq, Lq, D)
    mask = _bool_mask((B, Hq, Lq, Lkv)) if kind == "bool" else rand(1, 1, Lq, Lkv)
    sinks = np.array([0.5, -0.2, 3.0, -np.inf])
    o, lse = ref.attention_forward(q, k, v, 0.3, False, mask=mask, sinks=sinks)
    om = emulate_forward(q, k, v, 0.3, False, "f64", "f64", kv_block=16, slack=2.0, mask=mask, sinks=sinks)
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-13)
    want = ref.attention_backward(q, k, v, do, 0.3, False, mask=mask, sinks=sinks)
    got = emulate_backward(q, k, v, do, o, lse, 0.3, False, "f64", "f64", mask=mask)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
