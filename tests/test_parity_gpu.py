"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Cases follow the pages' test plan (MLX pull request "[Metal] Add Flash Attention
VJP for training", "Test Plan": vector path L = 1, 4, 7, 8; tiled L = 16 .. 256;
head dims 32/64/96/128 and 256; GQA 4:1, 8:1, 16:1 and MHA; fp16/bf16/fp32; L = 1,
non-power-of-two lengths, large batch, qL != kvL) at sizes the oracle finishes in
seconds but that span several tiles and a ragged tail. Full-size workloads are in
test_workloads_gpu.py.
"""

import numpy as np
import pytest

from parity_util import compare, reference, run_gpu
from scaled_dot_product_online_amd import inputs as inp

pytestmark = pytest.mark.gpu

CASES = [
    # fp32 operands (VALU path)
    (1, 2, 2, 64, 64, 32, "f32", False),
    (1, 4, 2, 100, 100, 64, "f32", True),
    (2, 4, 1, 37, 150, 128, "f32", False),
    (1, 2, 2, 1, 1, 64, "f32", True),
    (1, 4, 2, 37, 100, 32, "f32", True),   # causal, fewer queries than keys (ends aligned)
    (1, 4, 2, 70, 130, 96, "f32", True),   # head dim 96: four lanes of 24 per row
    (1, 2, 1, 45, 45, 96, "f32", False),
    (1, 4, 1, 50, 90, 256, "f32", True),   # head dim 256: eight lanes of 32 per row
]
for _dt in ("f16", "bf16"):
    for _d in (32, 64, 96, 128):
        CASES.append((1, 4, 2, 200, 200, _d, _dt, False))
        CASES.append((1, 4, 2, 200, 200, _d, _dt, True))
    CASES += [
        (1, 2, 1, 70, 300, 64, _dt, False),     # Lq != Lkv, ragged on both axes
        (2, 8, 1, 16, 16, 64, _dt, True),       # GQA 8:1, one partial tile
        (1, 16, 1, 32, 32, 128, _dt, False),    # GQA 16:1
        (1, 2, 2, 256, 256, 128, _dt, True),    # MHA, exact tiles
        (1, 2, 2, 1, 1, 64, _dt, True),         # L = 1 causal (tiled path)
        (1, 2, 2, 9, 9, 64, _dt, False),        # just above the vector cutoff
        (32, 2, 1, 8, 8, 32, _dt, True),        # large batch, causal short rows (vector path)
        # causal with Lq < Lkv: sequences aligned at their ends
        (1, 4, 2, 70, 300, 64, _dt, True),      # ragged on both axes
        (1, 8, 2, 130, 400, 128, _dt, True),    # GQA 4:1, several tiles each way
        (2, 2, 2, 9, 200, 32, _dt, True),       # just above the vector cutoff
        # vector path (Lq <= 8)
        (2, 8, 2, 1, 1000, 64, _dt, False),
        (2, 8, 2, 4, 1000, 64, _dt, False),
        (2, 8, 2, 7, 333, 128, _dt, False),
        (1, 8, 1, 4, 2085, 128, _dt, False),    # 32 packed rows, ragged keys
        (3, 4, 4, 8, 1, 32, _dt, False),        # single key
        (2, 16, 4, 8, 4099, 64, _dt, False),    # several splits
        (2, 8, 2, 8, 1000, 64, _dt, True),      # causal decode rows against a longer cache
        (2, 8, 2, 4, 333, 128, _dt, True),
        (1, 4, 1, 1, 200, 64, _dt, True),       # one causal query sees every key
        (2, 16, 4, 8, 4099, 64, _dt, True),     # causal, several splits
        # head dim 96 (12 16-byte chunks per row)
        (1, 8, 2, 130, 400, 96, _dt, True),     # tiled, causal, Lq < Lkv
        (2, 4, 1, 70, 300, 96, _dt, False),     # tiled, ragged
        (2, 8, 2, 7, 1000, 96, _dt, False),     # vector
        (2, 16, 4, 8, 4099, 96, _dt, True),     # vector, causal, several splits
        # keys split over workgroups on small grids: tiled forward and dQ (and dK/dV where noted)
        (1, 2, 1, 150, 1100, 64, _dt, False),   # 4 splits, ragged last tile
        (1, 4, 2, 200, 1000, 128, _dt, True),   # 4 splits, causal with Lq < Lkv
        (1, 2, 2, 640, 640, 64, _dt, True),     # 2 splits, the second empty for the first query blocks
        (1, 2, 1, 96, 700, 96, _dt, False),     # 2 splits, head dim 96
        # backward splits on small grids: dK/dV over its (query head, query tile) sequence
        (1, 8, 1, 512, 256, 64, _dt, False),    # 8 splits, GQA 8:1
        (1, 4, 1, 256, 200, 256, _dt, False),   # 2 splits, head dim 256
        (1, 4, 1, 512, 512, 128, _dt, True),    # causal, 4 splits
        (1, 4, 1, 500, 512, 64, _dt, True),     # causal, 4 splits, ragged last query tile
        # head dim 256 (32-key forward / dQ tiles, 16-row dQ waves, dK/dV with K rows in LDS and
        # 32-query tiles, 2-wave short-query kernels)
        (1, 4, 2, 200, 200, 256, _dt, True),    # tiled, causal
        (1, 4, 1, 70, 300, 256, _dt, False),    # tiled, ragged
        (1, 8, 2, 130, 400, 256, _dt, True),    # tiled, causal, Lq < Lkv
        (2, 8, 1, 33, 129, 256, _dt, False),    # tiled: one key past a 128-key block, one query past a 32-query tile
        (1, 4, 4, 96, 96, 256, _dt, True),      # tiled, MHA, causal: three 32-query tiles
        (2, 8, 2, 7, 1000, 256, _dt, False),    # vector
        (1, 8, 1, 4, 2085, 256, _dt, True),     # vector, causal, 32 packed rows
        (2, 16, 4, 8, 4099, 256, _dt, False),   # vector, several splits
        # head dim 256, forward and dQ keys split over 8 workgroups (16-row dQ waves)
        (1, 2, 1, 128, 1024, 256, _dt, False),  # 8 splits
        (1, 2, 2, 300, 1000, 256, _dt, True),   # 8 splits, causal with Lq < Lkv, last split empty
        # head dim 128 without a mask: 8-wave forward workgroups of 256 rows, 128-key tiles,
        # keys split over workgroups (ragged, causal with Lq < Lkv)
        (1, 4, 2, 128, 2048, 128, _dt, False),
        (1, 2, 1, 200, 1100, 128, _dt, True),
        # head dim 64 without a mask: 128-key forward tiles and 128-query dK/dV tiles
        (1, 4, 2, 200, 700, 64, _dt, True),     # causal with Lq < Lkv (tile starts rounded to 128)
        (2, 4, 4, 330, 330, 32, _dt, False),    # ragged last tiles, head dim 32
    ]
# A causal dQ on a small grid: one key split per 2048 keys binds (3 splits where one workgroup
# per CU would take 2).
CASES += [(1, 4, 4, 4100, 4100, 32, "bf16", True)]


def _id(c):
    B, Hq, Hkv, Lq, Lkv, D, dt, causal = c
    return f"{dt}-B{B}-H{Hq}x{Hkv}-L{Lq}x{Lkv}-D{D}-{'causal' if causal else 'full'}"


@pytest.mark.parametrize("case_def", CASES, ids=[_id(c) for c in CASES])
def test_parity_native_out(case_def, device):
    case = inp.make_case(*case_def, seed=0)
    want = reference(case, case.dtype)
    compare(case, run_gpu(case, case.dtype, device, fed=want), want)


@pytest.mark.parametrize("case_def", [c for c in CASES if c[6] != "f32"][::2],
                         ids=[_id(c) for c in CASES if c[6] != "f32"][::2])
def test_parity_fp32_out(case_def, device):
    case = inp.make_case(*case_def, seed=1)
    want = reference(case, "f32")
    compare(case, run_gpu(case, "f32", device, fed=want), want)


@pytest.mark.parametrize("case_def", CASES[1::3], ids=[_id(c) for c in CASES[1::3]])
def test_parity_end_to_end(case_def, device):
    """Forward then backward on the GPU's own O and LSE, as a training step runs: the bound
    allows R, the spread that the rounding of the stored O causes in Delta_i."""
    case = inp.make_case(*case_def, seed=2)
    want = reference(case, case.dtype, end_to_end=True)
    compare(case, run_gpu(case, case.dtype, device), want)


# Scale of zero (every visible key weighs the same) and negative scales, on every path:
# tiled causal and ragged, short-query causal and with split keys, float32.
SCALE_CASES = [
    (1, 4, 2, 150, 150, 64, "bf16", True),
    (1, 2, 1, 70, 300, 128, "f16", False),
    (1, 4, 2, 100, 260, 96, "bf16", True),
    (2, 8, 2, 4, 1000, 64, "bf16", True),
    (2, 16, 4, 8, 4099, 128, "f16", False),
    (1, 4, 2, 37, 100, 64, "f32", True),
]


@pytest.mark.parametrize("scale", [0.0, -0.125, -0.3])
@pytest.mark.parametrize("case_def", SCALE_CASES, ids=[_id(c) for c in SCALE_CASES])
def test_parity_zero_and_negative_scale(case_def, scale, device):
    case = inp.make_case(*case_def, seed=6, scale=scale)
    want = reference(case, case.dtype)
    got = run_gpu(case, case.dtype, device, fed=want)
    compare(case, got, want)
    if scale == 0.0:  # uniform weights: the gradients of Q and K vanish
        assert np.all(got["dq"] == 0) and np.all(got["dk"] == 0)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_large_logits_and_rising_scores(dt, device):
    """Scores ~N(0, 100), and keys whose norm grows along the sequence so the running max
    moves in every tile; both stress the exp2-domain rescaling."""
    case = inp.make_case(1, 4, 2, 300, 300, 64, dt, is_causal=True, seed=3)
    case.q = inp.from_f32(inp.as_float64(case.q, dt).astype(np.float32) * 10.0, dt)
    want = reference(case, "f32")
    compare(case, run_gpu(case, "f32", device, fed=want), want)
    case2 = inp.make_case(1, 2, 2, 64, 700, 64, dt, is_causal=False, seed=4)
    k = inp.as_float64(case2.k, dt)
    k *= np.linspace(0.2, 3.0, k.shape[2])[None, None, :, None]
    case2.k = inp.from_f32(k.astype(np.float32), dt)
    want2 = reference(case2, "f32")
    compare(case2, run_gpu(case2, "f32", device, fed=want2), want2)


@pytest.mark.parametrize("case_def", [(2, 8, 2, 200, 200, 64, "bf16", True), (2, 8, 2, 4, 3000, 128, "f16", False),
                                      (1, 4, 2, 100, 100, 64, "f32", True)])
def test_forward_without_lse_matches(case_def, device):
    import torch

    import scaled_dot_product_online_amd as sd

    case = inp.make_case(*case_def)
    q, k, v = (inp.to_torch(getattr(case, n), case.dtype, device) for n in ("q", "k", "v"))
    o1, lse = sd.sdpa_fwd(q, k, v, scale=case.scale, is_causal=case.is_causal)
    o2, none = sd.sdpa_fwd(q, k, v, scale=case.scale, is_causal=case.is_causal, need_lse=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("case_def", [(1, 8, 2, 333, 333, 128, "bf16", True), (2, 8, 2, 8, 5000, 64, "f16", False),
                                      (1, 2, 1, 70, 300, 32, "bf16", False)])
def test_deterministic_and_canaries(case_def, device):
    """Bitwise-identical repeats (no atomics anywhere) and no writes outside the outputs."""
    import torch

    import scaled_dot_product_online_amd as sd

    case = inp.make_case(*case_def)
    q, k, v, do = (inp.to_torch(getattr(case, n), case.dtype, device) for n in ("q", "k", "v", "do"))
    tdt = q.dtype
    pad = 4096
    B, Hq, Lq, D = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]

    def padded(shape, dtype):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * pad,), 7.0, dtype=dtype, device=device)
        return buf, buf[pad:pad + n].view(shape)

    runs = []
    for _ in range(2):
        ob, o = padded((B, Hq, Lq, D), tdt)
        lb, lse = padded((B, Hq, Lq), torch.float32)
        qb, dq = padded((B, Hq, Lq, D), tdt)
        kb, dk = padded((B, Hkv, Lkv, D), tdt)
        vb, dv = padded((B, Hkv, Lkv, D), tdt)
        sd.sdpa_fwd(q, k, v, scale=case.scale, is_causal=case.is_causal, out=o, lse=lse)
        sd.sdpa_bwd(q, k, v, o, lse, do, scale=case.scale, is_causal=case.is_causal, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        for buf in (ob, lb, qb, kb, vb):
            assert torch.all(buf[:pad] == 7.0) and torch.all(buf[-pad:] == 7.0), "write outside an output"
        runs.append([t.clone() for t in (o, lse, dq, dk, dv)])
    for a, b in zip(*runs):
        assert torch.equal(a, b), "repeat differs"
