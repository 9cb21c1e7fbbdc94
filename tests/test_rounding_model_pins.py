"""Pins of the 16-bit backward rounding model (oracle/rounding_floor.py) (CPU only).

The model's backward sets the floor F that the dQ, dK and dV parity bounds allow, so it
is pinned to things other than itself:
* rigorous per-element bounds: rounding to nearest changes x by at most u|x| (u the unit
  roundoff of the operand type, plus half the subnormal spacing near zero), so the
  model can differ from the fp64 definition by no more than
      |dV_j - dV_j*| <= sum_i u|P_ij| |dO_i|,
      |dQ_i - dQ_i*| <= |scale| sum_j (u|dS_ij| + (1 + u)|P_ij||dDelta_i|) |K_j|,
      |dK_j - dK_j*| <= |scale| sum_i (u|dS_ij| + (1 + u)|P_ij||dDelta_i|) |Q_i|,
  where dDelta_i is the change of Delta_i that the stored output's rounding causes;
* the size of the error: with independent rounding errors spread evenly over half an
  ulp (the standard probabilistic model of rounding error, as in Higham and Mary, "A
  New Approach to Probabilistic Rounding Error Analysis", SIAM J. Sci. Comput. 2019),
  the mean square error of dV is sum_i (ulp(P_ij)^2 / 12) dO_i^2, and likewise for dQ
  and dK with dS; the model's mean square error must come out at that size;
* exactness: when P and dS are exactly representable in the operand type (uniform
  weights over 4 keys, small integer operands), every rounding is a no-op and the model
  equals the definition to fp64 rounding, whatever the scale;
* Delta from the stored output: with the rounding switched off, changing the stored O
  by E changes dQ and dK by exactly the first-order formula
      -scale sum_j P_ij (dO_i . E_i) K_j   and   -scale sum_i P_ij (dO_i . E_i) Q_i,
  and leaves dV alone.
Planted slips in the model (P not rounded, dS rounded after the scale, the wrong operand
type, Delta from the exact output) each fail one of these.
"""

import numpy as np
import pytest

from oracle import rounding_floor as rf
from oracle import sdpa_reference as ref

U = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
HALF_SUB = {"bf16": 2.0 ** -134, "f16": 2.0 ** -25}  # half the subnormal spacing
MANT = {"bf16": 7, "f16": 10}
EMIN = {"bf16": -126, "f16": -14}


def _inputs(seed, B=1, Hq=4, Hkv=2, Lq=96, Lkv=128, D=32):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal(s) for s in ((B, Hq, Lq, D), (B, Hkv, Lkv, D), (B, Hkv, Lkv, D),
                                                        (B, Hq, Lq, D)))
    return q, k, v, do


def _exact_parts(q, k, v, do, scale, causal, o_stored):
    """Per head: P, dS (from the exact LSE, Delta from o_stored) and the Delta change."""
    B, Hq = q.shape[:2]
    G = Hq // k.shape[1]
    o, lse = ref.attention_forward(q, k, v, scale, causal)
    parts = {}
    for b in range(B):
        for h in range(Hq):
            _, _, p = ref.head_forward(q[b, h], k[b, h // G], v[b, h // G], scale, causal)
            dp = do[b, h] @ v[b, h // G].T
            delta = np.sum(do[b, h] * o[b, h], axis=1)
            ddelta = np.sum(do[b, h] * (o_stored[b, h] - o[b, h]), axis=1)
            parts[(b, h)] = (p, p * (dp - delta[:, None]), ddelta)
    return o, lse, parts


@pytest.mark.parametrize("op", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("stored", ["exact", "rounded"])
def test_backward_model_within_rigorous_bounds(op, causal, stored):
    q, k, v, do = _inputs(11)
    scale = 0.17677669529663687
    o, lse = ref.attention_forward(q, k, v, scale, causal)
    o_st = o if stored == "exact" else rf.round_to(o, op)
    dq, dk, dv = ref.attention_backward(q, k, v, do, scale, causal)
    mdq, mdk, mdv = rf.emulate_backward(q, k, v, do, o_st, lse, scale, causal, op, "f64")
    _, _, parts = _exact_parts(q, k, v, do, scale, causal, o_st)
    u, eta = U[op], HALF_SUB[op]
    G = q.shape[1] // k.shape[1]
    bdv, bdk = np.zeros(k.shape), np.zeros(k.shape)
    for (b, h), (p, ds, dd) in parts.items():
        hk = h // G
        w = u * np.abs(ds) + eta + (1 + u) * np.abs(p) * np.abs(dd)[:, None]
        bdq = abs(scale) * (w @ np.abs(k[b, hk]))
        assert np.all(np.abs(mdq[b, h] - dq[b, h]) <= bdq * (1 + 1e-9) + 1e-13)
        bdk[b, hk] += abs(scale) * (w.T @ np.abs(q[b, h]))
        bdv[b, hk] += (u * np.abs(p) + eta).T @ np.abs(do[b, h])
    assert np.all(np.abs(mdk - dk) <= bdk * (1 + 1e-9) + 1e-13)
    assert np.all(np.abs(mdv - dv) <= bdv * (1 + 1e-9) + 1e-13)
    # ... and the bounds are not vacuous: the model does move away from the definition.
    assert np.abs(mdv - dv).max() > 0.05 * bdv.max()


def _ulp(x, op):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** EMIN[op])))
    return 2.0 ** (e - MANT[op])


def _predicted_ms(parts, q, k, do, scale, op, G):
    """Mean square error of dV, dQ, dK under independent uniform rounding errors."""
    var = lambda x: np.where(rf.round_to(x, op) != x, _ulp(x, op) ** 2 / 12.0, 0.0)  # noqa: E731
    vdv, vdk, vdq = np.zeros(k.shape), np.zeros(k.shape), []
    for (b, h), (p, ds, _) in parts.items():
        hk = h // G
        vp, vds = var(p), var(ds)
        vdv[b, hk] += vp.T @ do[b, h] ** 2
        vdk[b, hk] += scale ** 2 * (vds.T @ q[b, h] ** 2)
        vdq.append(scale ** 2 * (vds @ k[b, hk] ** 2))
    return {"dv": vdv.mean(), "dk": vdk.mean(), "dq": np.mean(vdq)}


def _model_ms(q, k, v, do, scale, causal, op, o, lse):
    dq, dk, dv = ref.attention_backward(q, k, v, do, scale, causal)
    mdq, mdk, mdv = rf.emulate_backward(q, k, v, do, o, lse, scale, causal, op, "f64")
    return {"dv": np.mean((mdv - dv) ** 2), "dk": np.mean((mdk - dk) ** 2), "dq": np.mean((mdq - dq) ** 2)}


def _size_ratios(op, causal=False, seed=21):
    q, k, v, do = _inputs(seed, Lq=128, Lkv=128)
    scale = 0.125
    o, lse = ref.attention_forward(q, k, v, scale, causal)
    _, _, parts = _exact_parts(q, k, v, do, scale, causal, o)
    pred = _predicted_ms(parts, q, k, do, scale, op, q.shape[1] // k.shape[1])
    got = _model_ms(q, k, v, do, scale, causal, op, o, lse)
    return {n: got[n] / pred[n] for n in pred}


@pytest.mark.parametrize("op", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_model_error_has_the_predicted_size(op, causal):
    for name, ratio in _size_ratios(op, causal).items():
        assert 0.6 < ratio < 1.6, (name, ratio)


def _uniform_case(scale):
    """Q and K with every key row equal (so P = 1/4 over the 4 keys), small integer V, dO."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, L, D = 1, 2, 1, 6, 2
    q = rng.integers(-3, 4, (B, Hq, L, D)).astype(np.float64)
    k = np.broadcast_to(np.array([1.0, -2.0]), (B, Hkv, 4, D)).copy()
    v = rng.integers(-1, 2, (B, Hkv, 4, D)).astype(np.float64)
    do = rng.integers(-1, 2, (B, Hq, L, D)).astype(np.float64)
    return q, k, v, do


@pytest.mark.parametrize("op", ["bf16", "f16"])
@pytest.mark.parametrize("scale", [0.3, -1.7, 0.125])
def test_backward_model_is_exact_on_representable_operands(op, scale):
    q, k, v, do = _uniform_case(scale)
    o, lse = ref.attention_forward(q, k, v, scale, False)
    dq, dk, dv = ref.attention_backward(q, k, v, do, scale, False)
    mdq, mdk, mdv = rf.emulate_backward(q, k, v, do, o, lse, scale, False, op, "f64")
    for a, b_ in ((mdq, dq), (mdk, dk), (mdv, dv)):
        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-13)
    assert np.abs(dk).max() > 0.1  # a case with real gradients


def test_backward_model_delta_follows_the_stored_output():
    q, k, v, do = _inputs(31, Lq=40, Lkv=50, D=16)
    scale = 0.25
    o, lse = ref.attention_forward(q, k, v, scale, True)
    e = 0.05 * np.random.default_rng(3).standard_normal(o.shape)
    a = rf.emulate_backward(q, k, v, do, o, lse, scale, True, "f64", "f64")
    b_ = rf.emulate_backward(q, k, v, do, o + e, lse, scale, True, "f64", "f64")
    G = q.shape[1] // k.shape[1]
    want_dq = np.empty(q.shape)
    want_dk = np.zeros(k.shape)
    for h in range(q.shape[1]):
        _, _, p = ref.head_forward(q[0, h], k[0, h // G], v[0, h // G], scale, True)
        dd = np.sum(do[0, h] * e[0, h], axis=1)
        want_dq[0, h] = -scale * ((p * dd[:, None]) @ k[0, h // G])
        want_dk[0, h // G] += -scale * ((p * dd[:, None]).T @ q[0, h])
    np.testing.assert_allclose(b_[0] - a[0], want_dq, atol=1e-12)
    np.testing.assert_allclose(b_[1] - a[1], want_dk, atol=1e-12)
    np.testing.assert_array_equal(b_[2], a[2])


def test_planted_slips_in_the_backward_model_are_caught(monkeypatch):
    # 1. P not rounded before the dV product: the dV error vanishes, far below its size.
    with monkeypatch.context() as m:
        m.setattr(rf, "round_p", lambda p, op: p)
        assert _size_ratios("bf16")["dv"] < 0.01
    # 2. dS rounded after the scale: the exactness case breaks (scale 0.3 is not a power of 2).
    with monkeypatch.context() as m:
        m.setattr(rf, "round_ds", lambda ds, op, scale: rf.round_to(ds * scale, op) / scale)
        q, k, v, do = _uniform_case(0.3)
        o, lse = ref.attention_forward(q, k, v, 0.3, False)
        dq, dk, dv = ref.attention_backward(q, k, v, do, 0.3, False)
        mdq, mdk, _ = rf.emulate_backward(q, k, v, do, o, lse, 0.3, False, "bf16", "f64")
        assert max(np.abs(mdq - dq).max(), np.abs(mdk - dk).max()) > 1e-6
    # 3. dS rounded to fp16 where the operands are bf16: 8x less error than predicted.
    with monkeypatch.context() as m:
        m.setattr(rf, "round_ds", lambda ds, op, scale: rf.round_to(ds, "f16"))
        r = _size_ratios("bf16")
        assert r["dq"] < 0.1 and r["dk"] < 0.1
    # 4. Delta from the exact output instead of the stored one: the stored output no longer
    #    moves dQ (checked through the first-order formula's test on a planted model).
    with monkeypatch.context() as m:
        orig = rf.emulate_backward_group

        def exact_delta(q, k, v, do, o_stored, lse, *args, **kw):
            o_exact, _ = ref.attention_forward(q, k, v, args[0], args[1])
            return orig(q, k, v, do, o_exact, lse, *args, **kw)

        m.setattr(rf, "emulate_backward_group", exact_delta)
        with pytest.raises(AssertionError):
            test_backward_model_delta_follows_the_stored_output()
