"""Parity machinery shared by the GPU tests and ``smoke()``.

The GPU result is compared element by element with the fp64 oracle on the same
seeded inputs. Bound per element x of output tensor X (tests/golden/tolerances.json):

    |x_gpu - x_oracle| <= tol_X + F_X + ulp_out(x) / 2,
    F_X = max|X_model_pre - X_oracle|

where tol_X is the stated tolerance for the operand dtype and direction, X_model_pre
is the rounding-point model of the 16-bit kernels (oracle.rounding_floor, with the
kernels' key-block size) before its final rounding to the output dtype, and
ulp_out(x) / 2 is that final rounding at the element (the larger magnitude of the two
values decides the binade). The pages' tolerances were measured against attention in
the same dtype (mps-flash-sdpa 0.1.0, "Gradient Correctness"), whose outputs carry that
rounding too.

The backward is checked on decoupled inputs: it receives the oracle's O rounded to the
output dtype and the oracle's LSE rounded to fp32 (not the GPU forward's), and the model
is driven by exactly those, so the bound needs no allowance for which neighbour the
forward's stored output took. One end-to-end check (the backward fed by the GPU
forward) keeps that allowance, R_X: the largest difference between the backward model
driven by the model's stored O and by the exact O rounded to the output dtype (two
roundings of the same O, which Delta_i = sum_d dO_id O_id sees). For fp32 operands F
and R are ~1e-7, so the fp32 bound is about the literal 1e-5.
"""

from __future__ import annotations

import json
import os

import numpy as np

from oracle import sdpa_reference as ref
from oracle import rounding_floor as rf
from scaled_dot_product_online_amd import inputs as inp

_HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(_HERE, "golden", "tolerances.json")) as _f:
    TOL = json.load(_f)

# Key-block sizes of the kernels' online softmax (the reference max may move per block),
# and the slack (natural-log units) a block max must exceed it by to move it.
KV_BLOCK = {"tiled": 64, "vector": 32, "fp32": 32}
SLACK = {"tiled": 8.0 * np.log(2.0), "vector": 0.0, "fp32": 0.0}


def path_name(case):
    if case.dtype == "f32":
        return "fp32"
    G = case.Hq // case.Hkv
    return "vector" if (case.Lq <= 8 and G * case.Lq <= 32) else "tiled"


def _torch_mask(case, mask, device):
    import torch

    if mask is None:
        return None
    kind, arr = mask
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device) if kind == "bool" else inp.to_torch(arr, case.dtype,
                                                                                                      device)


def oracle_mask(case, mask):
    """The mask as the oracle takes it: a bool array, or the additive values widened to float64."""
    if mask is None:
        return None
    kind, arr = mask
    return np.asarray(arr, dtype=bool) if kind == "bool" else inp.as_float64(arr, case.dtype)


def fed_tensors(want, case, out_dtype, device):
    """The oracle's O (rounded to out_dtype) and LSE (fp32) as device tensors for sdpa_bwd."""
    import torch

    o = inp.to_torch(inp.from_f32(np.asarray(want["o_fed"], dtype=np.float32), out_dtype), out_dtype, device)
    lse = torch.from_numpy(np.asarray(want["lse_fed"], dtype=np.float32)).to(device)
    return o, lse


def run_gpu(case, out_dtype, device, backward=True, mask=None, sinks=None, fed=None):
    """Run sdpa_fwd (and sdpa_bwd) through the C ABI; returns float64 numpy arrays.

    mask: None or (kind, storage array) from inputs.make_mask; sinks: float32 [Hq] or None.
    fed: None (the backward takes the GPU forward's O and LSE: end to end), or the dict
    that ``reference`` returned, whose ``o_fed`` / ``lse_fed`` the backward then takes."""
    import torch

    import scaled_dot_product_online_amd as sd

    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out_dtype]
    q, k, v = (inp.to_torch(getattr(case, n), case.dtype, device) for n in ("q", "k", "v"))
    tm = _torch_mask(case, mask, device)
    ts = None if sinks is None else torch.from_numpy(np.ascontiguousarray(sinks, dtype=np.float32)).to(device)
    extra = f" mask={mask[0]}{tuple(mask[1].shape)}" if mask is not None else ""
    extra += " sinks" if sinks is not None else ""
    extra += f" scale={case.scale:g}"
    print(f"[gpu] fwd {case.shape_str} out={out_dtype}{extra}", flush=True)
    o, lse = sd.sdpa_fwd(q, k, v, scale=case.scale, is_causal=case.is_causal, out_dtype=tdt, attn_mask=tm, sinks=ts)
    torch.cuda.synchronize()
    res = {"o": inp.from_torch(o, out_dtype), "lse": inp.from_torch(lse, "f32")}
    if backward:
        do = inp.to_torch(case.do, case.dtype, device)
        if fed is not None:
            o, lse = fed_tensors(fed, case, out_dtype, device)
        print(f"[gpu] bwd {case.shape_str} out={out_dtype}{extra} {'decoupled' if fed is not None else 'end-to-end'}",
              flush=True)
        g = sd.sdpa_bwd(q, k, v, o, lse, do, scale=case.scale, is_causal=case.is_causal, out_dtype=tdt, attn_mask=tm,
                        sinks=ts)
        torch.cuda.synchronize()
        res.update(dq=inp.from_torch(g[0], out_dtype), dk=inp.from_torch(g[1], out_dtype),
                   dv=inp.from_torch(g[2], out_dtype))
        if sinks is not None:
            res["dsinks"] = inp.from_torch(g[3], "f32")
    return res


def _op_dtype(case):
    return case.dtype if case.dtype != "f32" else "f32"


def reference(case, out_dtype, backward=True, mask=None, sinks=None, end_to_end=False):
    """Oracle values and the rounding-model values for the whole case.

    The backward model is driven by ``o_fed`` / ``lse_fed`` (the oracle's O rounded to
    out_dtype, its LSE rounded to fp32), which run_gpu(fed=...) hands to the GPU backward.
    With ``end_to_end`` it is driven instead by the model's own stored forward output, as
    the GPU backward is when it takes the GPU forward's, and R (``*_spread``) is added."""
    q, k, v = case.f64("q"), case.f64("k"), case.f64("v")
    m = oracle_mask(case, mask)
    sk = None if sinks is None else np.asarray(sinks, dtype=np.float64)
    o, lse = ref.attention_forward(q, k, v, case.scale, case.is_causal, mask=m, sinks=sk)
    op = _op_dtype(case)
    pn = path_name(case)
    o_pre = rf.emulate_forward(q, k, v, case.scale, case.is_causal, op, "f64", KV_BLOCK[pn], slack=SLACK[pn],
                               mask=m, sinks=sk)
    o_fed, lse_fed = rf.round_to(o, out_dtype), rf.round_to(lse, "f32")
    out = {"o": o, "lse": lse, "o_model": o_pre, "out_dtype": out_dtype, "o_fed": o_fed, "lse_fed": lse_fed}
    if backward:
        do = case.f64("do")
        dq, dk, dv = ref.attention_backward(q, k, v, do, case.scale, case.is_causal, mask=m, sinks=sk)
        out.update(dq=dq, dk=dk, dv=dv)
        if end_to_end:
            # The kernels form Delta from their stored (rounded) output: the model does too.
            o_model = rf.round_to(o_pre, out_dtype)
            mdq, mdk, mdv = rf.emulate_backward(q, k, v, do, o_model, lse, case.scale, case.is_causal, op, "f64",
                                                mask=m)
            alt = rf.emulate_backward(q, k, v, do, o_fed, lse, case.scale, case.is_causal, op, "f64", mask=m)
            out.update({n + "_spread": float(np.abs(a - b).max())
                        for n, a, b in zip(("dq", "dk", "dv"), (mdq, mdk, mdv), alt)})
            o_sink, lse_sink = o_model, lse
        else:
            mdq, mdk, mdv = rf.emulate_backward(q, k, v, do, o_fed, lse_fed, case.scale, case.is_causal, op, "f64",
                                                mask=m)
            o_sink, lse_sink = o_fed, lse_fed
        out.update(dq_model=mdq, dk_model=mdk, dv_model=mdv)
        if sk is not None:
            out["dsinks"] = ref.sink_gradient(q, k, v, do, case.scale, case.is_causal, sk, mask=m)
            out["dsinks_model"], out["dsinks_mag"] = rf.emulate_sink_gradient(do, o_sink, lse_sink, sk)
    return out


def half_ulp(x, dtype):
    """Half the spacing of ``dtype`` at |x| (float64 array; normal range, subnormals floored)."""
    mant, emin = {"f32": (23, -126), "f16": (10, -14), "bf16": (7, -126), "f64": (52, -1022)}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** emin)))
    return 2.0 ** (e - mant - 1)


def compare(case, got, want, backward=True):
    """Per-tensor report {name: (max err/bound, 1, floor)}; raises AssertionError on a violation."""
    tol = TOL["stated"][case.dtype]
    odt = want.get("out_dtype", case.dtype)
    report = {}
    names = ["o"] + (["dq", "dk", "dv"] if backward else [])
    for name in names:
        t = tol["fwd"] if name == "o" else tol["bwd"]
        g, w, m = got[name], want[name], want[name + "_model"]
        assert np.all(np.isfinite(g)), f"{name}: non-finite output"
        floor = float(np.abs(m - w).max()) + want.get(name + "_spread", 0.0)
        bound = t + floor + half_ulp(np.maximum(np.abs(g), np.abs(w)), odt)
        report[name] = (float((np.abs(g - w) / bound).max()), 1.0, floor)
    # Rows that see no key (a mask) have LSE = -inf on both sides; the rest are compared.
    gl, wl = got["lse"], want["lse"]
    assert np.array_equal(np.isneginf(gl), np.isneginf(wl)), "lse: -inf rows differ"
    fin = np.isfinite(wl)
    lse_err = float(np.abs(gl[fin] - wl[fin]).max()) if fin.any() else 0.0
    report["lse"] = (lse_err, TOL["lse"][case.dtype], 0.0)
    if "dsinks" in got:
        # A sum over B*Lq rows: the stated backward tolerance relative to the sum of the
        # terms' magnitudes, plus the modelled floor (Delta from the stored output).
        t = tol["bwd"]
        g, w, m, mag = got["dsinks"], want["dsinks"], want["dsinks_model"], want["dsinks_mag"]
        assert np.all(np.isfinite(g)), "dsinks: non-finite output"
        bound = t * np.maximum(mag, 1.0) + np.abs(m - w)  # per head
        report["dsinks/bound"] = (float((np.abs(g - w) / bound).max()), 1.0, float(np.abs(m - w).max()))
    bad = {k: v for k, v in report.items() if not v[0] <= v[1]}
    assert not bad, f"{case.shape_str}: parity violated {bad} (all: {report})"
    return report


def _group_mask(m, b, hs):
    """Batch b and query heads hs of a mask broadcastable to [B, Hq, Lq, Lkv] (size-1 axes kept)."""
    if m is None:
        return None
    m = m.reshape((1,) * (4 - m.ndim) + m.shape)
    return m[(slice(b, b + 1) if m.shape[0] > 1 else slice(0, 1)), (hs if m.shape[1] > 1 else slice(0, 1))]


def reference_group(case, out_dtype, b, hk, backward=True, mask=None, sinks=None):
    """Oracle and model values for the G query heads of KV group (b, hk) only.

    Used at full workload sizes, where the whole-tensor oracle would take minutes.
    Returns arrays shaped like the group's slices: o/lse/dq [G, Lq, ...], dk/dv [Lkv, D],
    and ``o_fed`` / ``lse_fed`` for the group (the backward model is driven by them, as in
    ``reference``). (dsinks sums over every batch, so a group cannot check it.)
    """
    G = case.Hq // case.Hkv
    hs = slice(hk * G, (hk + 1) * G)
    q = inp.as_float64(case.q[b:b + 1, hs], case.dtype)
    k = inp.as_float64(case.k[b:b + 1, hk:hk + 1], case.dtype)
    v = inp.as_float64(case.v[b:b + 1, hk:hk + 1], case.dtype)
    m = _group_mask(oracle_mask(case, mask), b, hs)
    sk = None if sinks is None else np.asarray(sinks, dtype=np.float64)[hs]
    o, lse = ref.attention_forward(q, k, v, case.scale, case.is_causal, mask=m, sinks=sk)
    op = case.dtype
    pn = path_name(case)
    o_pre = rf.emulate_forward(q, k, v, case.scale, case.is_causal, op, "f64", KV_BLOCK[pn], slack=SLACK[pn],
                               mask=m, sinks=sk)
    o_fed, lse_fed = rf.round_to(o, out_dtype), rf.round_to(lse, "f32")
    out = {"o": o[0], "lse": lse[0], "o_model": o_pre[0], "out_dtype": out_dtype, "o_fed": o_fed[0],
           "lse_fed": lse_fed[0]}
    if backward:
        do = inp.as_float64(case.do[b:b + 1, hs], case.dtype)
        dq, dk, dv = ref.group_backward(q, k, v, do, case.scale, case.is_causal, 0, 0, mask=m, sinks=sk)
        mdq, mdk, mdv = rf.emulate_backward_group(q, k, v, do, o_fed, lse_fed, case.scale, case.is_causal, op,
                                                  "f64", 0, 0, mask=m)
        out.update(dq=dq, dk=dk, dv=dv, dq_model=mdq, dk_model=mdk, dv_model=mdv)
    return out


def reference_rows(case, out_dtype, b, h, rows, mask=None, sinks=None):
    """Oracle and model values of query rows ``rows`` of head (b, h): O, LSE and dQ.

    dQ of a row depends only on that row's O and LSE (through Delta_i and P_i), so the
    backward model of these rows is driven by ``o_fed`` / ``lse_fed`` of the same rows."""
    G = case.Hq // case.Hkv
    hk = h // G
    rows = np.asarray(rows)
    qh = inp.as_float64(case.q[b, h], case.dtype)
    kh = inp.as_float64(case.k[b, hk], case.dtype)
    vh = inp.as_float64(case.v[b, hk], case.dtype)
    doh = inp.as_float64(case.do[b, h], case.dtype)
    mk = oracle_mask(case, mask)
    bias = None if mk is None else ref.head_bias(mk, case.B, case.Hq, case.Lq, case.Lkv, b, h)
    sink = None if sinks is None else float(sinks[h])
    o, lse, _ = ref.head_forward(qh, kh, vh, case.scale, case.is_causal, rows, bias=bias, sink=sink)
    dq, _, _, _ = ref.head_backward(qh, kh, vh, doh, case.scale, case.is_causal, rows, bias=bias, sink=sink)
    pn = path_name(case)
    o_pre = rf.emulate_forward_head(qh, kh, vh, case.scale, case.is_causal, case.dtype, "f64", KV_BLOCK[pn],
                                    rows=rows, slack=SLACK[pn], bias=bias, sink=sink)
    o_fed, lse_fed = rf.round_to(o, out_dtype), rf.round_to(lse, "f32")
    mdq = rf.emulate_dq_rows(qh, kh, vh, doh, o_fed, lse_fed, case.scale, case.is_causal, case.dtype, rows, bias=bias)
    return {"o": o, "lse": lse, "o_model": o_pre, "o_fed": o_fed, "lse_fed": lse_fed, "dq": dq, "dq_model": mdq,
            "out_dtype": out_dtype}


def compare_rows(case, got, want):
    """compare() for O, LSE and dQ of sampled rows (no dK/dV: those sum over every row)."""
    tol = TOL["stated"][case.dtype]
    odt = want["out_dtype"]
    report = {}
    for name in ("o", "dq"):
        t = tol["fwd"] if name == "o" else tol["bwd"]
        g, w, m = got[name], want[name], want[name + "_model"]
        assert np.all(np.isfinite(g)), f"{name}: non-finite output"
        floor = float(np.abs(m - w).max())
        bound = t + floor + half_ulp(np.maximum(np.abs(g), np.abs(w)), odt)
        report[name] = (float((np.abs(g - w) / bound).max()), 1.0, floor)
    fin = np.isfinite(want["lse"])
    assert np.array_equal(np.isneginf(got["lse"]), np.isneginf(want["lse"])), "lse: -inf rows differ"
    report["lse"] = (float(np.abs(got["lse"][fin] - want["lse"][fin]).max()) if fin.any() else 0.0,
                     TOL["lse"][case.dtype], 0.0)
    bad = {k: v for k, v in report.items() if not v[0] <= v[1]}
    assert not bad, f"{case.shape_str}: parity violated {bad} (all: {report})"
    return report


def slice_group(case, got, b, hk):
    G = case.Hq // case.Hkv
    hs = slice(hk * G, (hk + 1) * G)
    res = {"o": got["o"][b, hs], "lse": got["lse"][b, hs]}
    if "dq" in got:
        res.update(dq=got["dq"][b, hs], dk=got["dk"][b, hk], dv=got["dv"][b, hk])
    return res
