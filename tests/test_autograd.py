"""The torch.autograd wrapper: eligibility checks (CPU) and its wiring to the C ABI (GPU).

The wrapper adds no arithmetic, so on the GPU its outputs and gradients must equal,
bit for bit, what sdpa_fwd / sdpa_bwd return for the same inputs (whose own parity
with the oracle is tested in test_parity_gpu.py). A float32 gradcheck on a tiny case
checks the backward against finite differences of the forward (the pages' test plan:
mps-flash-sdpa, "Testing"; MLX pull request "[Metal] Add Flash Attention VJP for
training", "Test Plan").
"""

import pytest
import torch

import scaled_dot_product_online_amd as sd
from scaled_dot_product_online_amd import inputs as inp


def _cpu(shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("shape,dtype,match", [((1, 2, 8, 64), torch.float32, "GPU only"),
                                               ((1, 2, 8, 64), torch.float64, "dtype"),
                                               ((2, 8, 64), torch.float16, r"\[B, H, L, D\]")])
def test_cpu_tensors_raise_before_any_call(shape, dtype, match):
    # No CPU fallback: host tensors are refused before the library is touched (an eligible
    # one for its device, the others for their dtype or rank, which are checked first).
    with pytest.raises(ValueError, match=match):
        sd.attention(_cpu(shape, dtype), _cpu(shape, dtype), _cpu(shape, dtype))


@pytest.mark.parametrize("dtype,match", [(torch.float64, "dtype"), (torch.int32, "dtype")])
def test_dtype_rules(monkeypatch, dtype, match):
    t = torch.empty((1, 2, 8, 64), dtype=dtype, device="meta")
    monkeypatch.setattr(torch.Tensor, "device", property(lambda self: torch.device("cuda", 0)))
    with pytest.raises(ValueError, match=match):
        sd.check_eligible(t, t, t)


@pytest.mark.parametrize(
    "shape_q,shape_k,causal,match",
    [
        ((1, 6, 8, 64), (1, 4, 8, 64), False, "not a multiple"),
        ((1, 4, 8, 80), (1, 2, 8, 80), False, "head size 80"),
        ((1, 4, 16, 64), (1, 2, 8, 64), True, "causal"),
        ((1, 4, 8, 64), (1, 2, 16, 64), True, None),  # causal, fewer queries than keys
        ((2, 4, 8, 64), (1, 2, 8, 64), False, "batch or head size"),
        ((1, 4, 8, 64), (1, 2, 8, 64), False, None),  # eligible
    ],
)
def test_shape_rules(monkeypatch, shape_q, shape_k, causal, match):
    q = torch.empty(shape_q, device="meta")
    k = torch.empty(shape_k, device="meta")
    # Pose meta tensors as GPU tensors so that only the shape rules decide.
    monkeypatch.setattr(torch.Tensor, "device", property(lambda self: torch.device("cuda", 0)))
    if match is None:
        sd.check_eligible(q, k, k.clone(), causal)
    else:
        with pytest.raises(ValueError, match=match):
            sd.check_eligible(q, k, k.clone(), causal)


CASES = [
    (1, 2, 2, 64, 64, 32, "f32", True),       # fp32 path
    (1, 8, 2, 150, 150, 128, "bf16", True),   # tiled, GQA 4:1, causal, ragged
    (2, 4, 1, 70, 200, 64, "f16", False),     # tiled, Lq != Lkv
    (2, 8, 2, 8, 300, 64, "bf16", False),     # short-query path
]


@pytest.mark.gpu
@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lkv,D,dt,causal", CASES)
def test_matches_c_abi_bitwise(device, B, Hq, Hkv, Lq, Lkv, D, dt, causal):
    case = inp.make_case(B, Hq, Hkv, Lq, Lkv, D, dt, is_causal=causal, seed=11)
    q, k, v, do = (inp.to_torch(getattr(case, n), dt, device) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = sd.sdpa_fwd(q, k, v, scale=case.scale, is_causal=causal)
    dq_ref, dk_ref, dv_ref = sd.sdpa_bwd(q, k, v, o_ref, lse_ref, do, scale=case.scale, is_causal=causal)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = sd.attention(qa, ka, va, scale=case.scale, is_causal=causal)
    o.backward(do)
    torch.cuda.synchronize()
    print(f"autograd {case.shape_str}", flush=True)
    assert torch.equal(o, o_ref)
    assert torch.equal(qa.grad, dq_ref)
    assert torch.equal(ka.grad, dk_ref)
    assert torch.equal(va.grad, dv_ref)


@pytest.mark.gpu
def test_no_grad_forward_skips_lse(device):
    case = inp.make_case(1, 4, 2, 64, 64, 64, "bf16", is_causal=False, seed=3)
    q, k, v = (inp.to_torch(getattr(case, n), "bf16", device) for n in ("q", "k", "v"))
    o_ref, _ = sd.sdpa_fwd(q, k, v, scale=case.scale, need_lse=False)
    with torch.no_grad():
        o = sd.attention(q, k, v, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert o.grad_fn is None


@pytest.mark.gpu
def test_gradcheck_fp32(device):
    """Backward against central finite differences of the forward (float32, tiny case)."""
    case = inp.make_case(1, 2, 1, 6, 9, 32, "f32", is_causal=False, seed=5)
    q, k, v = (inp.to_torch(getattr(case, n), "f32", device).requires_grad_(True) for n in ("q", "k", "v"))
    fn = lambda a, b, c: sd.attention(a, b, c, scale=case.scale)  # noqa: E731
    assert torch.autograd.gradcheck(fn, (q, k, v), eps=1e-2, atol=2e-3, rtol=2e-2, fast_mode=True)


def test_mask_and_sink_rules(monkeypatch):
    q = torch.empty((1, 4, 8, 64), device="meta")
    k = torch.empty((1, 2, 16, 64), device="meta")
    monkeypatch.setattr(torch.Tensor, "device", property(lambda self: torch.device("cuda", 0)))
    m = torch.empty((1, 1, 8, 16), dtype=torch.bool, device="meta")
    sd.check_eligible(q, k, k.clone(), False, m, torch.empty(4, device="meta"))
    with pytest.raises(ValueError, match="not combined"):
        sd.check_eligible(q, k, k.clone(), True, m)
    with pytest.raises(ValueError, match="bool or"):
        sd.check_eligible(q, k, k.clone(), False, torch.empty((8, 16), dtype=torch.float16, device="meta"))
    with pytest.raises(ValueError, match="broadcast"):
        sd.check_eligible(q, k, k.clone(), False, torch.empty((1, 3, 8, 16), dtype=torch.bool, device="meta"))
    with pytest.raises(ValueError, match="no gradient"):
        sd.check_eligible(q, k, k.clone(), False, torch.empty((8, 16), device="meta", requires_grad=True))
    with pytest.raises(ValueError, match="sinks"):
        sd.check_eligible(q, k, k.clone(), False, None, torch.empty(3, device="meta"))


@pytest.mark.gpu
@pytest.mark.parametrize("dt,Lq", [("bf16", 70), ("f16", 6), ("f32", 20)])
def test_mask_and_sinks_match_c_abi_bitwise(device, dt, Lq):
    case = inp.make_case(1, 4, 2, Lq, 90, 64, dt, seed=13)
    q, k, v, do = (inp.to_torch(getattr(case, n), dt, device) for n in ("q", "k", "v", "do"))
    mask = torch.from_numpy(inp.make_mask("bool", (1, 1, Lq, 90), dt, seed=1)).to(device)
    sinks = torch.from_numpy(inp.make_sinks(4, seed=2)).to(device)
    o_ref, lse_ref = sd.sdpa_fwd(q, k, v, scale=case.scale, attn_mask=mask, sinks=sinks)
    g_ref = sd.sdpa_bwd(q, k, v, o_ref, lse_ref, do, scale=case.scale, attn_mask=mask, sinks=sinks)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    sa = sinks.clone().requires_grad_(True)
    o = sd.attention(qa, ka, va, scale=case.scale, attn_mask=mask, sinks=sa)
    o.backward(do)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for got, want in zip((qa.grad, ka.grad, va.grad, sa.grad), g_ref):
        assert torch.equal(got, want)


@pytest.mark.gpu
def test_gradcheck_fp32_with_mask_and_sinks(device):
    """Backward (dq, dk, dv and dsinks) against finite differences of the masked forward."""
    case = inp.make_case(1, 2, 1, 6, 9, 32, "f32", seed=7)
    q, k, v = (inp.to_torch(getattr(case, n), "f32", device).requires_grad_(True) for n in ("q", "k", "v"))
    mask = torch.from_numpy(inp.make_mask("additive", (1, 2, 6, 9), "f32", seed=3)).to(device)
    sinks = torch.from_numpy(inp.make_sinks(2, seed=4)).to(device).requires_grad_(True)
    fn = lambda a, b, c, s: sd.attention(a, b, c, scale=case.scale, attn_mask=mask, sinks=s)  # noqa: E731
    assert torch.autograd.gradcheck(fn, (q, k, v, sinks), eps=1e-2, atol=2e-3, rtol=2e-2, fast_mode=True)
