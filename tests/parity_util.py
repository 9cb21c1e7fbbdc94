"""Parity machinery shared by the GPU tests and ``smoke()``.

The GPU result is compared element by element with the fp64 oracle on the same
seeded inputs. Bound per output tensor X (tests/golden/tolerances.json):

    max|X_gpu - X_oracle| <= tol_X + F_X,    F_X = max|X_model - X_oracle|

where tol_X is the stated tolerance for the operand dtype and direction, and
X_model is the rounding-point model of the 16-bit kernels (oracle.rounding_floor)
evaluated on the same inputs with the kernels' key-block size. For fp32 operands
F is ~1e-7, so the fp32 bound is the literal 1e-5.
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
    return "vector" if (case.Lq <= 8 and not case.is_causal and G * case.Lq <= 32) else "tiled"


def run_gpu(case, out_dtype, device, backward=True):
    """Run sdpa_fwd (and sdpa_bwd) through the C ABI; returns float64 numpy arrays."""
    import torch

    import scaled_dot_product_online_amd as sd

    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out_dtype]
    q, k, v = (inp.to_torch(getattr(case, n), case.dtype, device) for n in ("q", "k", "v"))
    print(f"[gpu] fwd {case.shape_str} out={out_dtype}", flush=True)
    o, lse = sd.sdpa_fwd(q, k, v, scale=case.scale, is_causal=case.is_causal, out_dtype=tdt)
    torch.cuda.synchronize()
    res = {"o": inp.from_torch(o, out_dtype), "lse": inp.from_torch(lse, "f32")}
    if backward:
        do = inp.to_torch(case.do, case.dtype, device)
        print(f"[gpu] bwd {case.shape_str} out={out_dtype}", flush=True)
        dq, dk, dv = sd.sdpa_bwd(q, k, v, o, lse, do, scale=case.scale, is_causal=case.is_causal, out_dtype=tdt)
        torch.cuda.synchronize()
        res.update(dq=inp.from_torch(dq, out_dtype), dk=inp.from_torch(dk, out_dtype), dv=inp.from_torch(dv, out_dtype))
    return res


def reference(case, out_dtype, backward=True):
    """Oracle values and the rounding-model values for the whole case."""
    q, k, v = case.f64("q"), case.f64("k"), case.f64("v")
    o, lse = ref.attention_forward(q, k, v, case.scale, case.is_causal)
    op = case.dtype if case.dtype != "f32" else "f32"
    pn = path_name(case)
    o_model = rf.emulate_forward(q, k, v, case.scale, case.is_causal, op, out_dtype, KV_BLOCK[pn], slack=SLACK[pn])
    out = {"o": o, "lse": lse, "o_model": o_model}
    if backward:
        do = case.f64("do")
        dq, dk, dv = ref.attention_backward(q, k, v, do, case.scale, case.is_causal)
        mdq, mdk, mdv = rf.emulate_backward(q, k, v, do, o_model, lse, case.scale, case.is_causal, op, out_dtype)
        out.update(dq=dq, dk=dk, dv=dv, dq_model=mdq, dk_model=mdk, dv_model=mdv)
    return out


def compare(case, got, want, backward=True):
    """Per-tensor report {name: (err, bound, floor)}; raises AssertionError on a violation."""
    tol = TOL["stated"][case.dtype]
    report = {}
    names = ["o"] + (["dq", "dk", "dv"] if backward else [])
    for name in names:
        t = tol["fwd"] if name == "o" else tol["bwd"]
        g, w, m = got[name], want[name], want[name + "_model"]
        assert np.all(np.isfinite(g)), f"{name}: non-finite output"
        err = float(np.abs(g - w).max())
        floor = float(np.abs(m - w).max())
        report[name] = (err, t + floor, floor)
    lse_err = float(np.abs(got["lse"] - want["lse"]).max())
    report["lse"] = (lse_err, TOL["lse"][case.dtype], 0.0)
    bad = {k: v for k, v in report.items() if not v[0] <= v[1]}
    assert not bad, f"{case.shape_str}: parity violated {bad} (all: {report})"
    return report


def reference_group(case, out_dtype, b, hk, backward=True):
    """Oracle and model values for the G query heads of KV group (b, hk) only.

    Used at full workload sizes, where the whole-tensor oracle would take minutes.
    Returns arrays shaped like the group's slices: o/lse/dq [G, Lq, ...], dk/dv [Lkv, D].
    """
    G = case.Hq // case.Hkv
    hs = slice(hk * G, (hk + 1) * G)
    q = inp.as_float64(case.q[b:b + 1, hs], case.dtype)
    k = inp.as_float64(case.k[b:b + 1, hk:hk + 1], case.dtype)
    v = inp.as_float64(case.v[b:b + 1, hk:hk + 1], case.dtype)
    o, lse = ref.attention_forward(q, k, v, case.scale, case.is_causal)
    op = case.dtype
    pn = path_name(case)
    o_model = rf.emulate_forward(q, k, v, case.scale, case.is_causal, op, out_dtype, KV_BLOCK[pn], slack=SLACK[pn])
    out = {"o": o[0], "lse": lse[0], "o_model": o_model[0]}
    if backward:
        do = inp.as_float64(case.do[b:b + 1, hs], case.dtype)
        dq, dk, dv = ref.group_backward(q, k, v, do, case.scale, case.is_causal, 0, 0)
        mdq, mdk, mdv = rf.emulate_backward_group(q, k, v, do, o_model, lse, case.scale, case.is_causal, op,
                                                  out_dtype, 0, 0)
        out.update(dq=dq, dk=dk, dv=dv, dq_model=mdq, dk_model=mdk, dv_model=mdv)
    return out


def slice_group(case, got, b, hk):
    G = case.Hq // case.Hkv
    hs = slice(hk * G, (hk + 1) * G)
    res = {"o": got["o"][b, hs], "lse": got["lse"][b, hs]}
    if "dq" in got:
        res.update(dq=got["dq"][b, hs], dk=got["dk"][b, hk], dv=got["dv"][b, hk])
    return res
