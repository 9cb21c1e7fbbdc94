"""GPU parity of masks and attention sinks: the HIP kernels (through sdpa_fwd_masked /
sdpa_bwd_masked) against the fp64 oracle.

Masks: boolean (nonzero keeps the key) or additive in the operand dtype (with -inf
entries), broadcast from [B, Hq, Lq, Lkv], [B, 1, 1, Lkv] (key padding), [1, 1, Lq, Lkv]
(one pattern for all heads) or [1, Hq, Lq, Lkv]; some cases leave query rows with no
key at all (O = 0, LSE = -inf). Sinks: one float32 logit per query head, one head with
-inf (no sink). Every kernel family is covered: tiled (16-bit), short-query (16-bit,
one or several key splits) and float32, at head dims 32 to 256. The bound is the one of
test_parity_gpu.py, plus dsinks per head within the stated backward tolerance of the
sum of its terms' magnitudes (tests/parity_util.py).
"""

import numpy as np
import pytest

from parity_util import compare, reference, run_gpu
from scaled_dot_product_online_amd import inputs as inp

pytestmark = pytest.mark.gpu


def _mask_shape(spec, B, Hq, Lq, Lkv):
    return {"full": (B, Hq, Lq, Lkv), "keypad": (B, 1, 1, Lkv), "shared": (1, 1, Lq, Lkv),
            "head": (1, Hq, Lq, Lkv)}[spec]


# B, Hq, Hkv, Lq, Lkv, D, dtype, causal, mask kind, mask shape, rows with no key, sinks
CASES = []
for _dt in ("f16", "bf16"):
    CASES += [
        (1, 4, 2, 200, 200, 64, _dt, False, "bool", "full", 3, False),       # tiled
        (2, 4, 1, 70, 300, 128, _dt, False, "additive", "shared", 0, True),
        (1, 8, 2, 130, 400, 128, _dt, False, "bool", "keypad", 0, True),
        (1, 4, 2, 150, 150, 96, _dt, False, "additive", "head", 2, False),
        (1, 2, 1, 100, 180, 256, _dt, False, "bool", "full", 0, True),
        (1, 4, 2, 200, 200, 64, _dt, False, None, None, 0, True),            # sinks only
        (1, 4, 2, 150, 170, 128, _dt, True, None, None, 0, True),            # causal + sinks
        (1, 4, 2, 130, 900, 128, _dt, False, "bool", "full", 2, True),       # tiled, 3 key splits
        # a boolean mask staged through LDS by the forward and (D <= 96) dQ kernels: ragged
        # query rows and keys (Lkv not a whole number of key tiles)
        (2, 4, 2, 150, 260, 96, _dt, False, "bool", "shared", 1, False),
        (2, 4, 2, 100, 132, 64, _dt, False, "bool", "head", 0, True),        # per-head block, staged
        (2, 4, 2, 90, 200, 128, _dt, False, "bool", "full", 0, False),       # per-(batch, head) block
        (1, 2, 1, 100, 800, 64, _dt, True, None, None, 0, True),             # causal + sinks, 3 key splits
        (1, 8, 2, 256, 300, 128, _dt, False, "bool", "keypad", 0, True),     # dK/dV in 2 splits
        # contiguous key padding (batch b keeps its first keys, one batch none): whole key
        # tiles and whole dK/dV waves are padding, which the tiled kernels skip
        (3, 4, 2, 130, 600, 128, _dt, False, "bool", "padded", 0, False),
        (3, 4, 1, 100, 700, 64, _dt, False, "bool", "padded", 0, True),
        (3, 4, 2, 80, 500, 256, _dt, False, "bool", "padded", 0, False),
        (2, 8, 2, 4, 1000, 64, _dt, False, "bool", "full", 1, True),         # short-query
        (2, 16, 4, 8, 4099, 128, _dt, False, "additive", "keypad", 0, True),  # several splits
        (2, 8, 2, 7, 333, 128, _dt, False, None, None, 0, True),
        (1, 8, 2, 8, 600, 256, _dt, False, "additive", "full", 0, True),
        (2, 8, 2, 8, 700, 32, _dt, True, None, None, 0, True),               # causal short-query + sinks
    ]
CASES += [
    (1, 4, 2, 37, 100, 64, "f32", False, "bool", "full", 2, True),          # float32 path
    (2, 4, 1, 20, 50, 32, "f32", False, "additive", "shared", 0, False),
    (1, 2, 1, 30, 30, 128, "f32", True, None, None, 0, True),
    (1, 2, 1, 24, 40, 256, "f32", False, "additive", "head", 1, True),
    # float32 rows of 32 lanes (D = 128) and of 16 two-element slices (D = 32)
    (1, 4, 2, 45, 70, 128, "f32", False, "bool", "keypad", 1, True),
    (2, 2, 1, 33, 90, 32, "f32", False, "bool", "full", 2, False),
]


def _id(c):
    B, Hq, Hkv, Lq, Lkv, D, dt, causal, kind, spec, empty, sinks = c
    m = f"{kind}-{spec}" + (f"-empty{empty}" if empty else "") if kind else "nomask"
    return f"{dt}-B{B}-H{Hq}x{Hkv}-L{Lq}x{Lkv}-D{D}-{'causal' if causal else 'full'}-{m}{'-sinks' if sinks else ''}"


def _inputs(c, seed):
    B, Hq, Hkv, Lq, Lkv, D, dt, causal, kind, spec, empty, sinks = c
    case = inp.make_case(B, Hq, Hkv, Lq, Lkv, D, dt, is_causal=causal, seed=seed)
    mask = None
    if spec == "padded":  # batch 0 keeps Lkv - 150 keys, batch 1 none, batch b > 1 Lkv - 150 - 97 b
        keep = [0 if b == 1 else max(0, Lkv - 150 - 97 * b) for b in range(B)]
        mask = ("bool", inp.make_key_padding_mask(B, Lkv, keep))
    elif kind is not None:
        mask = (kind, inp.make_mask(kind, _mask_shape(spec, B, Hq, Lq, Lkv), dt, seed=seed + 7, empty_rows=empty))
    sk = inp.make_sinks(Hq, seed=seed + 3, none_heads=(Hq - 1,)) if sinks else None
    return case, mask, sk


@pytest.mark.parametrize("case_def", CASES, ids=[_id(c) for c in CASES])
def test_mask_and_sink_parity(case_def, device):
    case, mask, sk = _inputs(case_def, seed=5)
    want = reference(case, case.dtype, mask=mask, sinks=sk)
    got = run_gpu(case, case.dtype, device, mask=mask, sinks=sk, fed=want)
    rep = compare(case, got, want)
    print(" ".join(f"{k}={v[0]:.2e}/{v[1]:.2e}" for k, v in rep.items()), flush=True)
    if mask is not None and case_def[10]:  # rows with no key: O = 0, LSE = -inf
        assert np.isneginf(got["lse"]).any()


@pytest.mark.parametrize("case_def", [c for c in CASES if c[6] != "f32"][1::3],
                         ids=[_id(c) for c in CASES if c[6] != "f32"][1::3])
def test_mask_and_sink_parity_fp32_out(case_def, device):
    case, mask, sk = _inputs(case_def, seed=9)
    want = reference(case, "f32", mask=mask, sinks=sk)
    compare(case, run_gpu(case, "f32", device, mask=mask, sinks=sk, fed=want), want)


@pytest.mark.parametrize("case_def", [c for c in CASES if c[6] != "f32"][2::4],
                         ids=[_id(c) for c in CASES if c[6] != "f32"][2::4])
def test_mask_and_sink_parity_end_to_end(case_def, device):
    """The backward fed by the GPU forward's own O and LSE (the bound then allows R, the
    spread that the forward output's rounding causes in Delta)."""
    case, mask, sk = _inputs(case_def, seed=11)
    want = reference(case, case.dtype, mask=mask, sinks=sk, end_to_end=True)
    compare(case, run_gpu(case, case.dtype, device, mask=mask, sinks=sk), want)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_all_true_mask_and_no_sink_equal_the_unmasked_call(dt, device):
    """An all-True boolean mask, and sinks that are all -inf, reproduce the plain call up to
    the rounding of a differently contracted product (the masked kernels add the bias to the
    scaled score, so the compiler fuses different multiply-adds)."""
    import torch

    import scaled_dot_product_online_amd as sd

    case = inp.make_case(1, 4, 2, 100, 130, 64, dt, seed=2)
    q, k, v, do = (inp.to_torch(getattr(case, n), dt, device) for n in ("q", "k", "v", "do"))
    o0, l0 = sd.sdpa_fwd(q, k, v, scale=case.scale)
    g0 = sd.sdpa_bwd(q, k, v, o0, l0, do, scale=case.scale)
    ones = torch.ones((1, 1, 100, 130), dtype=torch.bool, device=device)
    no_sink = torch.full((4,), float("-inf"), dtype=torch.float32, device=device)
    o1, l1 = sd.sdpa_fwd(q, k, v, scale=case.scale, attn_mask=ones, sinks=no_sink)
    g1 = sd.sdpa_bwd(q, k, v, o1, l1, do, scale=case.scale, attn_mask=ones, sinks=no_sink)
    torch.cuda.synchronize()
    assert torch.all(g1[3] == 0)
    assert torch.allclose(l0, l1, atol=2e-6, rtol=0)
    if dt == "f32":
        assert torch.allclose(o0, o1, atol=1e-6, rtol=0)
        for a, b in zip(g0, g1[:3]):
            assert torch.allclose(a, b, atol=1e-6, rtol=0)
    else:
        assert (o0.float() - o1.float()).abs().max().item() <= 2 ** -7
