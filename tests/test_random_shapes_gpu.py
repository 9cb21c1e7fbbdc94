"""GPU parity on seeded random shapes: the HIP kernels (through the C ABI) against the
fp64 oracle, with the bound of test_parity_gpu.py.

The shapes are drawn once from a fixed generator: operand type, head dim (32 to 256),
GQA group size (1 to 8), causal or not, query lengths from 1 (short-query path) to a
few hundred, and key lengths up to about 1200, so that most cases have ragged tails and
many run on grids small enough for the kernels to split their keys or query tiles
across workgroups. A second draw adds long causal shapes on small grids. Sizes stay where
the oracle finishes in a few seconds.
"""

import numpy as np
import pytest

from parity_util import compare, reference, run_gpu
from scaled_dot_product_online_amd import inputs as inp

pytestmark = pytest.mark.gpu


def _draw_cases(n, seed=2026, max_work=1.5e8):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dt = str(rng.choice(["f16", "bf16", "f32"], p=[0.4, 0.4, 0.2]))
        D = int(rng.choice([32, 64, 96, 128, 256]))
        Hkv = int(rng.integers(1, 3))
        G = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 3))
        causal = bool(rng.integers(0, 2))
        Lq = int(rng.integers(1, 9)) if rng.random() < 0.3 else int(rng.integers(9, 320))
        Lkv = int(rng.integers(Lq if causal else 1, (Lq if causal else 0) + 1200))
        if B * Hkv * G * Lq * Lkv * D > max_work:
            continue
        cases.append((B, Hkv * G, Hkv, Lq, Lkv, D, dt, causal))
    return cases


CASES = _draw_cases(32)


def _draw_long_causal(n, seed=2027, max_work=6e8):
    """Causal 16-bit shapes of 600-2600 queries against up to 1500 more keys on one batch of
    1-8 heads: small grids where the forward and dQ split their keys (the causal dQ at least
    once per 2048 keys) and dK/dV its query tiles, with long and short causal triangles."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dt = str(rng.choice(["f16", "bf16"]))
        D = int(rng.choice([32, 64, 128]))
        Hkv = int(rng.integers(1, 3))
        G = int(rng.choice([1, 2, 4]))
        Lq = int(rng.integers(600, 2600))
        Lkv = int(rng.integers(Lq, Lq + 1500))
        if Hkv * G * Lq * Lkv * D > max_work:
            continue
        cases.append((1, Hkv * G, Hkv, Lq, Lkv, D, dt, True))
    return cases


CASES += _draw_long_causal(12)


def _id(c):
    B, Hq, Hkv, Lq, Lkv, D, dt, causal = c
    return f"{dt}-B{B}-H{Hq}x{Hkv}-L{Lq}x{Lkv}-D{D}-{'causal' if causal else 'full'}"


@pytest.mark.parametrize("case_def", CASES, ids=[_id(c) for c in CASES])
def test_random_shape_parity(case_def, device):
    case = inp.make_case(*case_def, seed=7)
    want = reference(case, case.dtype)
    compare(case, run_gpu(case, case.dtype, device, fed=want), want)
