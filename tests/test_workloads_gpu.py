"""GPU parity at the full sizes of the workloads (scaled_dot_product_online_amd/workloads.py).

Each workload runs forward + backward through the C ABI at its real shape, in the
launch configuration bench.py times. The fp64 oracle then checks whole KV groups
(all G query heads, every row and every key) sampled from the output, with the
same bound as the small-size tests (tol + rounding floor, tests/golden/tolerances.json).
Properties that hold at any size are checked on the whole output: finiteness, and
dV column sums over each group equal to the summed dO (sum_j dV_j = sum_i dO_i; not
with sinks, which take a share of each row's probability). Workloads with a mask or
sinks (workloads.MASKED) run through the masked entry points with them.
"""

import numpy as np
import pytest

from parity_util import compare, reference_group, run_gpu, slice_group
from scaled_dot_product_online_amd import inputs as inp
from scaled_dot_product_online_amd.workloads import WORKLOADS, mask_and_sinks

pytestmark = pytest.mark.gpu


def _groups(case, n):
    """n (b, hk) groups spread over the batch and the KV heads (first and last included)."""
    allg = [(b, hk) for b in range(case.B) for hk in range(case.Hkv)]
    idx = np.unique(np.linspace(0, len(allg) - 1, num=min(n, len(allg))).round().astype(int))
    return [allg[i] for i in idx]


@pytest.mark.parametrize("wl", WORKLOADS, ids=[w[0] for w in WORKLOADS])
def test_workload_full_size(wl, device):
    name, B, Hq, Hkv, Lq, Lkv, D, dt, causal = wl
    print(f"[workload] {name}", flush=True)
    case = inp.make_case(B, Hq, Hkv, Lq, Lkv, D, dt, is_causal=causal, seed=0)
    mask, sinks = mask_and_sinks(name)
    got = run_gpu(case, dt, device, mask=mask, sinks=sinks)
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert np.all(np.isfinite(got[key])), key
    # Any size: sum_j dV_j over a group's keys equals the sum of dO over its heads and rows.
    G = Hq // Hkv
    do = inp.as_float64(case.do, dt).reshape(B, Hkv, G * Lq, D).sum(axis=2)
    col = got["dv"].sum(axis=2)
    tol = 1e-3 * np.abs(do).max() + (0.05 if dt != "f32" else 1e-3) * np.sqrt(Lkv)
    if sinks is None:
        assert np.abs(col - do).max() <= tol
    # About 2^26 score elements of fp64 oracle work (seconds on the host), at least one group.
    n_groups = max(1, min(B * Hkv, 8, (1 << 26) // (G * Lq * Lkv)))
    for b, hk in _groups(case, n_groups):
        print(f"[workload] {name} oracle on group b={b} hk={hk}", flush=True)
        want = reference_group(case, dt, b, hk, mask=mask, sinks=sinks)
        rep = compare(case, slice_group(case, got, b, hk), want)
        print(f"[workload] {name} b={b} hk={hk} " +
              " ".join(f"{k}={v[0]:.2e}/{v[1]:.2e}" for k, v in rep.items()), flush=True)
