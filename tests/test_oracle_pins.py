"""Pins of the fp64 oracle to things other than itself (CPU only).

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, the wrong GQA head map, the mask off
by one, a missing scale) fails at least one of them; ``test_pins_catch_planted_mistakes``
plants such slips in copies of the oracle's outputs and checks that they are caught.

Independent references used:
* torch's CPU math attention (``scaled_dot_product_attention`` with
  ``enable_gqa``) and torch autograd, both in float64;
* ``scipy.special.logsumexp``;
* central finite differences of the scalar sum(O * dO);
* closed forms: Lkv = 1, equal scores, causal row 0, causal Q = 0, two keys;
* invariants: key shift, joint key/value permutation, convex hull, zero-sum dK,
  dV column sums, GQA == MHA on repeated K/V.
"""

import math

import numpy as np
import pytest
import scipy.special

from oracle import sdpa_reference as ref
from oracle.rounding_floor import emulate_backward, emulate_forward, round_to

RNG = np.random.default_rng(1234)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def torch_reference(q, k, v, do, scale, causal):
    import torch
    import torch.nn.functional as F

    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, scale=scale, is_causal=causal,
                                       enable_gqa=q.shape[1] != k.shape[1])
    (o * torch.tensor(do)).sum().backward()
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


SHAPES = [
    # B, Hq, Hkv, Lq, Lkv, D, causal
    (1, 2, 1, 3, 5, 4, False),
    (2, 4, 2, 7, 7, 8, True),
    (1, 8, 2, 16, 33, 16, False),
    (1, 3, 3, 20, 20, 32, True),
    (2, 4, 1, 1, 9, 8, False),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_matches_torch_math_attention_fp64(shape):
    B, Hq, Hkv, Lq, Lkv, D, causal = shape
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D), rand(B, Hq, Lq, D)
    scale = 1.0 / math.sqrt(D)
    o, lse = ref.attention_forward(q, k, v, scale, causal)
    dq, dk, dv = ref.attention_backward(q, k, v, do, scale, causal)
    to, tdq, tdk, tdv = torch_reference(q, k, v, do, scale, causal)
    np.testing.assert_allclose(o, to, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, tdq, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tdk, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tdv, rtol=0, atol=1e-11)


@pytest.mark.parametrize("shape", SHAPES)
def test_lse_matches_scipy_logsumexp(shape):
    B, Hq, Hkv, Lq, Lkv, D, causal = shape
    q, k, v = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D)
    scale = 0.37
    _, lse = ref.attention_forward(q, k, v, scale, causal)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            s = scale * q[b, h] @ k[b, h // G].T
            for i in range(Lq):
                row = s[i, : i + 1] if causal else s[i]
                assert abs(lse[b, h, i] - scipy.special.logsumexp(row)) < 1e-12


def _fd_check(q, k, v, do, scale, causal, backward_fn, forward_fn, h=1e-6):
    """Max relative error between the explicit gradients and central differences."""
    grads = backward_fn(q, k, v, do, scale, causal)
    worst = 0.0
    for arr, g in zip((q, k, v), grads):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = arr[idx]
            arr[idx] = old + h
            fp = np.sum(forward_fn(q, k, v, scale, causal)[0] * do)
            arr[idx] = old - h
            fm = np.sum(forward_fn(q, k, v, scale, causal)[0] * do)
            arr[idx] = old
            fd = (fp - fm) / (2 * h)
            worst = max(worst, abs(fd - g[idx]) / max(1.0, abs(fd)))
    return worst


@pytest.mark.parametrize("case", [((1, 2, 1, 3, 5, 4), False), ((1, 2, 1, 4, 4, 4), True), ((1, 4, 2, 3, 3, 2), True)])
def test_gradients_match_finite_differences(case):
    (B, Hq, Hkv, Lq, Lkv, D), causal = case
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D), rand(B, Hq, Lq, D)
    err = _fd_check(q, k, v, do, 0.7, causal, ref.attention_backward, ref.attention_forward)
    assert err < 1e-7, err


def test_single_key_returns_v():
    B, Hq, Hkv, Lq, D = 2, 4, 2, 5, 8
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, 1, D), rand(B, Hkv, 1, D), rand(B, Hq, Lq, D)
    scale = 0.25
    o, lse = ref.attention_forward(q, k, v, scale, False)
    dq, dk, dv = ref.attention_backward(q, k, v, do, scale, False)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_array_equal(o[b, h], np.broadcast_to(v[b, h // G, 0], (Lq, D)))
            np.testing.assert_allclose(lse[b, h], scale * q[b, h] @ k[b, h // G, 0], atol=1e-12)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    for b in range(B):
        for hk in range(Hkv):
            np.testing.assert_allclose(dv[b, hk, 0], do[b, hk * G:(hk + 1) * G].sum(axis=(0, 1)), atol=1e-12)


def test_equal_scores_return_mean_v():
    B, H, Lq, Lkv, D = 1, 2, 6, 11, 8
    q = np.zeros((B, H, Lq, D))
    k, v = rand(B, H, Lkv, D), rand(B, H, Lkv, D)
    o, lse = ref.attention_forward(q, k, v, 0.5, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(Lkv), atol=1e-14)
    # all key rows equal, Q random: also uniform weights
    k2 = np.broadcast_to(rand(B, H, 1, D), (B, H, Lkv, D)).copy()
    o2, lse2 = ref.attention_forward(rand(B, H, Lq, D), k2, v, 0.5, False)
    np.testing.assert_allclose(o2, np.broadcast_to(v.mean(axis=2, keepdims=True), o2.shape), atol=1e-13)


def test_causal_row0_and_causal_zero_q():
    B, H, L, D = 1, 3, 9, 4
    q, k, v, do = rand(B, H, L, D), rand(B, H, L, D), rand(B, H, L, D), rand(B, H, L, D)
    o, lse = ref.attention_forward(q, k, v, 0.9, True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.9 * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), atol=1e-14)
    qz = np.zeros_like(q)
    o, lse = ref.attention_forward(qz, k, v, 0.9, True)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, L + 1)[None, None, :, None]
    np.testing.assert_allclose(o, prefix_mean, atol=1e-14)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, L + 1)), lse.shape), atol=1e-14)
    _, dk, _ = ref.attention_backward(qz, k, v, do, 0.9, True)
    assert np.abs(dk).max() < 1e-14


def test_causal_unequal_lengths_are_the_tail_of_the_square_problem():
    # Causal with Lq < Lkv (sequences aligned at their ends) equals the last Lq rows of
    # the square causal problem whose queries end with the same Lq rows; the square
    # case is pinned to torch above. Gradients: the prefix rows carry dO = 0.
    B, Hq, Hkv, Lq, Lkv, D = 1, 4, 2, 5, 13, 8
    qt, k, v, dot = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D), rand(B, Hq, Lq, D)
    qfull = np.concatenate([rand(B, Hq, Lkv - Lq, D), qt], axis=2)
    dofull = np.concatenate([np.zeros((B, Hq, Lkv - Lq, D)), dot], axis=2)
    o, lse = ref.attention_forward(qt, k, v, 0.6, True)
    of, lsef = ref.attention_forward(qfull, k, v, 0.6, True)
    np.testing.assert_allclose(o, of[:, :, Lkv - Lq:], atol=1e-14)
    np.testing.assert_allclose(lse, lsef[:, :, Lkv - Lq:], atol=1e-14)
    dq, dk, dv = ref.attention_backward(qt, k, v, dot, 0.6, True)
    dqf, dkf, dvf = ref.attention_backward(qfull, k, v, dofull, 0.6, True)
    np.testing.assert_allclose(dq, dqf[:, :, Lkv - Lq:], atol=1e-13)
    np.testing.assert_allclose(dk, dkf, atol=1e-13)
    np.testing.assert_allclose(dv, dvf, atol=1e-13)
    # One query row sees every key: causal equals full attention.
    q1 = qt[:, :, -1:]
    for a, b_ in zip(ref.attention_forward(q1, k, v, 0.6, True), ref.attention_forward(q1, k, v, 0.6, False)):
        np.testing.assert_array_equal(a, b_)
    with pytest.raises(ValueError):
        ref.attention_forward(qfull, k[:, :, :Lq], v[:, :, :Lq], 0.6, True)


def test_two_keys_logistic():
    q = np.array([[[[1.0, 2.0]]]])
    k = np.array([[[[0.5, -1.0], [2.0, 1.0]]]])
    v = np.array([[[[3.0, -1.0], [-2.0, 5.0]]]])
    scale = 0.8
    a, b = scale * (0.5 - 2.0), scale * (2.0 + 2.0)
    p0 = 1.0 / (1.0 + math.exp(b - a))
    o, lse = ref.attention_forward(q, k, v, scale, False)
    np.testing.assert_allclose(o[0, 0, 0], p0 * v[0, 0, 0] + (1 - p0) * v[0, 0, 1], atol=1e-15)
    assert abs(lse[0, 0, 0] - (b + math.log1p(math.exp(a - b)))) < 1e-15


def test_invariants():
    B, Hq, Hkv, Lq, Lkv, D = 2, 4, 2, 7, 13, 8
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D), rand(B, Hq, Lq, D)
    scale = 0.3
    o, lse = ref.attention_forward(q, k, v, scale, False)
    # probabilities sum to one and P recomputed from LSE matches
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            _, l2, p = ref.head_forward(q[b, h], k[b, h // G], v[b, h // G], scale, False)
            np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
            p_from_lse = np.exp(scale * q[b, h] @ k[b, h // G].T - l2[:, None])
            np.testing.assert_allclose(p_from_lse, p, atol=1e-12)
    # key shift: O unchanged, LSE shifted by scale * q.c
    c = rand(D)
    o2, lse2 = ref.attention_forward(q, k + c, v, scale, False)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + scale * np.einsum("bhld,d->bhl", q, c), atol=1e-12)
    # joint permutation of key/value rows
    perm = RNG.permutation(Lkv)
    o3, lse3 = ref.attention_forward(q, k[:, :, perm], v[:, :, perm], scale, False)
    np.testing.assert_allclose(o3, o, atol=1e-12)
    np.testing.assert_allclose(lse3, lse, atol=1e-12)
    # convex hull
    for b in range(B):
        for h in range(Hq):
            vv = v[b, h // G]
            assert np.all(o[b, h] <= vv.max(axis=0) + 1e-12) and np.all(o[b, h] >= vv.min(axis=0) - 1e-12)
    # gradient sums: sum_j dK_j = 0, sum_j dV_j = sum over group and rows of dO
    dq, dk, dv = ref.attention_backward(q, k, v, do, scale, False)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    for hk in range(Hkv):
        np.testing.assert_allclose(dv[:, hk].sum(axis=1), do[:, hk * G:(hk + 1) * G].sum(axis=(1, 2)), atol=1e-12)
    # GQA equals MHA on repeat-interleaved K/V, with dK/dV summed over the group
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    om, lm = ref.attention_forward(q, kr, vr, scale, False)
    np.testing.assert_allclose(om, o, atol=1e-14)
    dqm, dkm, dvm = ref.attention_backward(q, kr, vr, do, scale, False)
    np.testing.assert_allclose(dqm, dq, atol=1e-12)
    np.testing.assert_allclose(dkm.reshape(B, Hkv, G, Lkv, D).sum(axis=2), dk, atol=1e-12)
    np.testing.assert_allclose(dvm.reshape(B, Hkv, G, Lkv, D).sum(axis=2), dv, atol=1e-12)


def test_pins_catch_planted_mistakes():
    """Slips planted in copies of the oracle's outputs are caught by the pins above."""
    B, Hq, Hkv, Lq, Lkv, D = 1, 4, 2, 6, 6, 8
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, Lkv, D), rand(B, Hkv, Lkv, D), rand(B, Hq, Lq, D)
    scale = 0.35
    to, tdq, tdk, tdv = torch_reference(q, k, v, do, scale, True)
    o, _ = ref.attention_forward(q, k, v, scale, True)
    dq, dk, dv = ref.attention_backward(q, k, v, do, scale, True)
    assert np.abs(o - to).max() < 1e-12

    def caught(o_, dq_, dk_, dv_):
        return max(np.abs(o_ - to).max(), np.abs(dq_ - tdq).max(), np.abs(dk_ - tdk).max(),
                   np.abs(dv_ - tdv).max()) > 1e-6

    G = Hq // Hkv
    # wrong GQA head map: head h reading KV head h % Hkv instead of h // G
    o_bad, _ = ref.attention_forward(q, np.tile(k, (1, G, 1, 1)), np.tile(v, (1, G, 1, 1)), scale, True)
    assert caught(o_bad, dq, dk, dv)
    # mask dropped, and mask off by one (key i hidden from query i)
    o_nc, _ = ref.attention_forward(q, k, v, scale, False)
    assert caught(o_nc, dq, dk, dv)
    o_off = np.empty_like(o)
    for h in range(Hq):
        s = scale * q[0, h] @ k[0, h // G].T
        s = np.where(np.arange(Lkv)[None, :] < np.arange(Lq)[:, None], s, -np.inf)
        s[0, 0] = 0.0  # row 0 would otherwise see no key
        e = np.exp(s - s.max(axis=1, keepdims=True))
        o_off[0, h] = (e / e.sum(axis=1, keepdims=True)) @ v[0, h // G]
    assert caught(o_off, dq, dk, dv)
    # missing scale in dQ, sign flip in dK, transposed role of dO in dV
    assert caught(o, dq / scale, dk, dv)
    assert caught(o, dq, -dk, dv)
    assert caught(o, dq, dk, dv[:, :, ::-1])
    # Delta dropped: dS = P * dP instead of P * (dP - Delta)
    dq_nodelta = np.empty_like(dq)
    for h in range(Hq):
        _, _, p = ref.head_forward(q[0, h], k[0, h // G], v[0, h // G], scale, True)
        dq_nodelta[0, h] = scale * (p * (do[0, h] @ v[0, h // G].T)) @ k[0, h // G]
    assert caught(o, dq_nodelta, dk, dv)


def test_round_to_matches_ieee_conversions():
    import torch

    x = np.concatenate([RNG.standard_normal(100000) * 10.0 ** RNG.integers(-6, 6, 100000),
                        [0.0, 1.0, -1.0, 65504.0, 1e-8]])
    tb = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_to(x.astype(np.float32).astype(np.float64), "bf16"), tb)
    x32 = x[np.abs(x) < 6.0e4].astype(np.float32).astype(np.float64)  # within fp16 range
    th = torch.tensor(x32, dtype=torch.float32).to(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_to(x32, "f16"), th)
    # ties to even on bf16: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert round_to(np.array([1.0 + 2.0 ** -8]), "bf16")[0] == 1.0
    assert round_to(np.array([1.0 + 3 * 2.0 ** -8]), "bf16")[0] == 1.0 + 2.0 ** -6


@pytest.mark.parametrize("causal,Lq", [(False, 37), (True, 37), (True, 20)])
def test_rounding_model_reduces_to_definition_in_fp64(causal, Lq):
    B, Hq, Hkv, L, D = 1, 4, 2, 37, 16
    q, k, v, do = rand(B, Hq, Lq, D), rand(B, Hkv, L, D), rand(B, Hkv, L, D), rand(B, Hq, Lq, D)
    o, lse = ref.attention_forward(q, k, v, 0.25, causal)
    oe = emulate_forward(q, k, v, 0.25, causal, "f64", "f64", kv_block=8)
    np.testing.assert_allclose(oe, o, atol=1e-13)
    oe2 = emulate_forward(q, k, v, 0.25, causal, "f64", "f64", kv_block=4, kv_segment=12)
    np.testing.assert_allclose(oe2, o, atol=1e-13)
    oe3 = emulate_forward(q, k, v, 0.25, causal, "f64", "f64", kv_block=8, slack=5.5)
    np.testing.assert_allclose(oe3, o, atol=1e-13)
    dq, dk, dv = ref.attention_backward(q, k, v, do, 0.25, causal)
    edq, edk, edv = emulate_backward(q, k, v, do, o, lse, 0.25, causal, "f64", "f64")
    for a, b_ in ((edq, dq), (edk, dk), (edv, dv)):
        np.testing.assert_allclose(a, b_, atol=1e-12)


def test_reference_max_slack_rule():
    from oracle.rounding_floor import _running_max

    s = np.array([[0.0, 1.0, 5.0, 2.0, 9.0, 20.0, -np.inf, 30.0]])
    # blocks of 2: maxima 1, 5, 20, 30; slack 3: 1 -> 5 (moves, 5 > 1+3) -> 20 -> 30
    np.testing.assert_array_equal(_running_max(s, 2, None, 3.0)[0], [1, 1, 5, 5, 20, 20, 30, 30])
    # slack 10: 1, then 5 (not > 11) stays 1, 20 > 11 moves, 30 not > 30 stays 20
    np.testing.assert_array_equal(_running_max(s, 2, None, 10.0)[0], [1, 1, 1, 1, 20, 20, 20, 20])
    # slack 0 is the running max; segments restart it
    np.testing.assert_array_equal(_running_max(s, 2, 4, 0.0)[0], [1, 1, 5, 5, 20, 20, 30, 30])


def test_rounding_model_floor_scales_with_precision():
    B, Hq, Hkv, L, D = 1, 2, 1, 64, 16
    q, k, v = rand(B, Hq, L, D), rand(B, Hkv, L, D), rand(B, Hkv, L, D)
    o, _ = ref.attention_forward(q, k, v, 0.25, True)
    errs = {dt: np.abs(emulate_forward(q, k, v, 0.25, True, dt, "f32", kv_block=16) - o).max()
            for dt in ("f32", "f16", "bf16")}
    assert errs["f32"] < 1e-6 < errs["f16"] < errs["bf16"] < 3e-2
    # bf16 unit roundoff is 2^-8; the P rounding error is bounded by it times max|V|
    assert errs["bf16"] <= 2.0 ** -8 * np.abs(v).max() + 1e-6
