"""GPU parity at the full sizes of the workloads (scaled_dot_product_online_amd/workloads.py).

Each workload runs forward + backward through the C ABI at its real shape, in the
launch configuration bench.py times, and the fp64 oracle checks, with the bound of the
small-size tests (tol + rounding floor, tests/golden/tolerances.json):
* every (batch, query head): O, LSE and dQ on sampled query rows (the first and last
  rows, the first and last row of each causal quarter, and seeded random rows);
* the first and the last (batch, KV-head) group whole: O, LSE, dQ of all its query
  heads and rows, and its dK, dV.
The backward is checked on decoupled inputs, as in tests/parity_util.py: wherever the
oracle checks a result, the backward receives the oracle's O (rounded to the output
dtype) and LSE (fp32) in place of the GPU forward's: for the whole of the two checked
groups, and for every sampled row (dQ of a row depends only on that row's O and LSE).
Elsewhere it takes the GPU forward's. Properties that hold at any size are checked on
the whole output: finiteness, and dV column sums over each group equal to the summed
dO (sum_j dV_j = sum_i dO_i; not with sinks, which take a share of each row's
probability). Workloads with a mask or sinks (workloads.MASKED) run through the masked
entry points with them.
"""

import time

import numpy as np
import pytest

from parity_util import compare, compare_rows, reference_group, reference_rows, slice_group
from scaled_dot_product_online_amd import inputs as inp
from scaled_dot_product_online_amd.workloads import WORKLOADS, mask_and_sinks

pytestmark = pytest.mark.gpu

ROWS_PER_HEAD = 12


def sample_rows(Lq, seed):
    """Sorted distinct query rows: the ends, quarter boundaries, and seeded random rows."""
    fixed = {0, Lq - 1} | {min(Lq - 1, (Lq * k) // 4) for k in range(1, 4)}
    rng = np.random.default_rng(seed)
    extra = set(rng.integers(0, Lq, size=ROWS_PER_HEAD).tolist())
    return np.array(sorted(fixed | extra))


def end_groups(B, Hkv):
    return sorted({(0, 0), (B - 1, Hkv - 1)})


@pytest.mark.parametrize("wl", WORKLOADS, ids=[w[0] for w in WORKLOADS])
def test_workload_full_size(wl, device):
    import torch

    import scaled_dot_product_online_amd as sd
    from parity_util import _torch_mask

    name, B, Hq, Hkv, Lq, Lkv, D, dt, causal = wl
    G = Hq // Hkv
    print(f"[workload] {name}", flush=True)
    case = inp.make_case(B, Hq, Hkv, Lq, Lkv, D, dt, is_causal=causal, seed=0)
    mask, sinks = mask_and_sinks(name)
    tm = _torch_mask(case, mask, device)
    ts = None if sinks is None else torch.from_numpy(sinks).to(device)
    q, k, v, do = (inp.to_torch(getattr(case, n), dt, device) for n in ("q", "k", "v", "do"))
    kw = dict(scale=case.scale, is_causal=causal, attn_mask=tm, sinks=ts)
    o, lse = sd.sdpa_fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    got_o, got_lse = inp.from_torch(o, dt), inp.from_torch(lse, "f32")

    # Oracle values of the two whole groups and of sampled rows of every head.
    t0 = time.perf_counter()
    groups = end_groups(B, Hkv)
    want_g = {}
    for b, hk in groups:
        print(f"[workload] {name} oracle on group b={b} hk={hk}", flush=True)
        want_g[(b, hk)] = reference_group(case, dt, b, hk, mask=mask, sinks=sinks)
    rows, want_r = {}, {}
    for b in range(B):
        for h in range(Hq):
            rows[(b, h)] = sample_rows(Lq, seed=1000 * b + h)
            want_r[(b, h)] = reference_rows(case, dt, b, h, rows[(b, h)], mask=mask, sinks=sinks)
    print(f"[workload] {name} oracle: {len(groups)} groups + {sum(len(r) for r in rows.values())} rows of "
          f"{B * Hq} heads in {time.perf_counter() - t0:.1f} s", flush=True)

    # The backward's O and LSE: the GPU forward's, with the oracle's wherever it checks.
    o_fed, lse_fed = o.clone(), lse.clone()
    for (b, hk), w in want_g.items():
        ot, lt = _fed_torch(w, dt, device)
        o_fed[b, hk * G:(hk + 1) * G] = ot
        lse_fed[b, hk * G:(hk + 1) * G] = lt
    for (b, h), w in want_r.items():
        ot, lt = _fed_torch(w, dt, device)
        idx = torch.from_numpy(rows[(b, h)]).to(device)
        o_fed[b, h, idx] = ot
        lse_fed[b, h, idx] = lt
    g = sd.sdpa_bwd(q, k, v, o_fed, lse_fed, do, **kw)
    torch.cuda.synchronize()
    got = {"o": got_o, "lse": got_lse, "dq": inp.from_torch(g[0], dt), "dk": inp.from_torch(g[1], dt),
           "dv": inp.from_torch(g[2], dt)}
    for key, val in got.items():
        assert np.all(np.isfinite(val)), key

    # Any size: sum_j dV_j over a group's keys equals the sum of dO over its heads and rows.
    dosum = inp.as_float64(case.do, dt).reshape(B, Hkv, G * Lq, D).sum(axis=2)
    col = got["dv"].sum(axis=2)
    tol = 1e-3 * np.abs(dosum).max() + 0.05 * np.sqrt(Lkv)
    if sinks is None:
        assert np.abs(col - dosum).max() <= tol

    worst = {}
    for (b, h), w in want_r.items():
        r = rows[(b, h)]
        rep = compare_rows(case, {"o": got["o"][b, h, r], "lse": got["lse"][b, h, r], "dq": got["dq"][b, h, r]}, w)
        for key, val in rep.items():
            worst[key] = max(worst.get(key, 0.0), val[0])
    print(f"[workload] {name} sampled rows of all {B * Hq} heads, worst err/bound: " +
          " ".join(f"{k}={v:.2e}" for k, v in worst.items()), flush=True)
    for b, hk in groups:
        rep = compare(case, slice_group(case, got, b, hk), want_g[(b, hk)])
        print(f"[workload] {name} group b={b} hk={hk} " +
              " ".join(f"{k}={v[0]:.2e}/{v[1]:.2e}" for k, v in rep.items()), flush=True)


def _fed_torch(want, dt, device):
    import torch

    o = inp.to_torch(inp.from_f32(np.asarray(want["o_fed"], dtype=np.float32), dt), dt, device)
    lse = torch.from_numpy(np.asarray(want["lse_fed"], dtype=np.float32)).to(device)
    return o, lse
