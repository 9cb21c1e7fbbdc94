"""sdpa_bwd_noalloc through the C ABI against sdpa_bwd (GPU).

The entry point runs the same kernels as sdpa_bwd with the library's fixed per-GPU
scratch in place of the caller's workspace, so its outputs must be bit-identical. Two
calls in a row, the second with smaller sizes (the scratch keeps the first call's
contents), on each kernel family: tiled (causal GQA, and a small grid whose backward
splits into partials held in the scratch), short-query, float32.
"""

import ctypes

import numpy as np
import pytest

from scaled_dot_product_online_amd import inputs as inp

pytestmark = pytest.mark.gpu

PAIRS = [
    ((2, 8, 2, 300, 300, 128, "bf16", True), (1, 4, 1, 100, 130, 128, "bf16", True)),
    ((1, 8, 8, 2048, 2048, 64, "f16", False), (1, 2, 2, 640, 640, 64, "f16", True)),
    ((4, 32, 8, 8, 4099, 128, "bf16", False), (2, 8, 2, 4, 1000, 128, "bf16", False)),
    ((2, 8, 4, 100, 128, 64, "f32", True), (1, 2, 1, 37, 50, 64, "f32", False)),
]


def _run_pair(first, second, device):
    import torch

    import scaled_dot_product_online_amd as sd

    lib = sd.library()
    for case_def in (first, second):
        case = inp.make_case(*case_def, seed=3)
        print(f"[noalloc] {case.shape_str}", flush=True)
        q, k, v, do = (inp.to_torch(getattr(case, n), case.dtype, device) for n in ("q", "k", "v", "do"))
        o, lse = sd.sdpa_fwd(q, k, v, scale=case.scale, is_causal=case.is_causal)
        want = sd.sdpa_bwd(q, k, v, o, lse, do, scale=case.scale, is_causal=case.is_causal)
        got = [torch.full_like(t, float("nan")) for t in want]
        code = {torch.float32: sd.F32, torch.float16: sd.F16, torch.bfloat16: sd.BF16}[q.dtype]
        p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        st = lib.sdpa_bwd_noalloc(p(q), p(k), p(v), p(o), p(lse), p(do), p(got[0]), p(got[1]), p(got[2]),
                                  case.B, case.Hq, case.Hkv, case.Lq, case.Lkv, case.D, case.scale,
                                  int(case.is_causal), code, code,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, sd.status_str(st)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            assert torch.equal(a, b), f"{name} differs from sdpa_bwd"


@pytest.mark.parametrize("pair", PAIRS, ids=["tiled-causal", "tiled-split", "vector", "fp32"])
def test_noalloc_matches_workspace_backward(pair, device):
    _run_pair(*pair, device)


def test_noalloc_binding(device):
    import torch

    import scaled_dot_product_online_amd as sd

    case = inp.make_case(1, 4, 2, 70, 90, 64, "bf16", is_causal=True, seed=4)
    q, k, v, do = (inp.to_torch(getattr(case, n), "bf16", device) for n in ("q", "k", "v", "do"))
    o, lse = sd.sdpa_fwd(q, k, v, scale=case.scale, is_causal=True)
    want = sd.sdpa_bwd(q, k, v, o, lse, do, scale=case.scale, is_causal=True)
    got = sd.sdpa_bwd_noalloc(q, k, v, o, lse, do, *(torch.empty_like(t) for t in want), scale=case.scale,
                              is_causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(got, want))
