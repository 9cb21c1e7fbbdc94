"""Parity at the largest key length the C ABI admits for one head (bf16, D = 128).

sdpa.h admits one head's rows while (Lkv + 256) * D * 2 bytes fit 2 GiB, so that the
kernels' 32-bit buffer offsets reach nearly their limit: Lkv = 8,388,351 here. An fp64
oracle over 8M keys would take minutes, so the test uses a property that holds at any
size: K and V are R = 2047 copies of one 4096-key block (Lkv = 8,384,512). Each copy
then gets 1/R of the block's probabilities, so

    O = O_block,  LSE = LSE_block + ln R,  dQ = dQ_block,
    dK, dV of every copy = dK_block / R, dV_block / R,

and the block problem is checked against the oracle with the usual bound
(tests/parity_util.py). Every copy's dK / dV must also be bit-identical to the
first copy's (a key's gradients depend only on its own row and the query rows).
Both kernel families run: the short-query path (Lq = 4) and the tiled path (Lq = 16).
The last test takes the query side to the same length (Q and dO repeated), where the
dK / dV accumulations run over all 8.4M queries.
"""

import math

import numpy as np
import pytest

from parity_util import compare, reference
from scaled_dot_product_online_amd import inputs as inp

pytestmark = pytest.mark.gpu

BLOCK, R, D = 4096, 2047, 128


@pytest.mark.parametrize("Lq", [4, 16], ids=["short-query", "tiled"])
def test_repeated_keys_at_max_length(device, Lq):
    import torch

    import scaled_dot_product_online_amd as sd

    assert (BLOCK * R + 256) * D * 2 <= (1 << 31) - 1  # inside the ABI's per-head limit
    case = inp.make_case(1, 2, 1, Lq, BLOCK, D, "bf16", seed=3)
    q, kb, vb, do = (inp.to_torch(getattr(case, n), "bf16", device) for n in ("q", "k", "v", "do"))
    k = kb.repeat(1, 1, R, 1).contiguous()
    v = vb.repeat(1, 1, R, 1).contiguous()
    print(f"[max-size] Lq={Lq} Lkv={k.shape[2]} path={sd.PATH_NAMES[sd.select_path(2, 1, Lq, k.shape[2], D, 0, sd.BF16)]}",
          flush=True)
    o, lse = sd.sdpa_fwd(q, k, v, scale=case.scale, out_dtype=torch.float32)
    dq, dk, dv = sd.sdpa_bwd(q, k, v, o, lse, do, scale=case.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    del k, v
    dkr, dvr = dk.view(R, BLOCK, D), dv.view(R, BLOCK, D)
    assert bool((dkr == dkr[:1]).all()) and bool((dvr == dvr[:1]).all()), "copies' dK / dV differ"
    got = {"o": inp.from_torch(o, "f32"), "lse": inp.from_torch(lse, "f32") - math.log(R),
           "dq": inp.from_torch(dq, "f32"), "dk": inp.from_torch(dkr[0], "f32")[None, None] * R,
           "dv": inp.from_torch(dvr[0], "f32")[None, None] * R}
    del dk, dv, dkr, dvr
    rep = compare(case, got, reference(case, "f32", end_to_end=True))
    print(" ".join(f"{n}={e:.2e}/{b:.2e}" for n, (e, b, _) in rep.items()), flush=True)
    assert np.all(np.isfinite(got["lse"]))


def test_repeated_queries_at_max_length(device):
    """The other side of the limit: Lq = R * 4096 queries (Q and dO are R copies of one
    block) against one 4096-key block. Every copy's O, LSE and dQ equal the block's, and
    dK, dV (accumulated over all 8.4M queries) are R times the block's."""
    import torch

    import scaled_dot_product_online_amd as sd

    case = inp.make_case(1, 2, 1, BLOCK, BLOCK, D, "bf16", seed=4)
    qb, k, v, dob = (inp.to_torch(getattr(case, n), "bf16", device) for n in ("q", "k", "v", "do"))
    q = qb.repeat(1, 1, R, 1).contiguous()
    do = dob.repeat(1, 1, R, 1).contiguous()
    print(f"[max-size] Lq={q.shape[2]} Lkv={BLOCK}", flush=True)
    o, lse = sd.sdpa_fwd(q, k, v, scale=case.scale, out_dtype=torch.float32)
    dq, dk, dv = sd.sdpa_bwd(q, k, v, o, lse, do, scale=case.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    del q, do
    o_r, l_r, dq_r = (t.view(1, 2, R, BLOCK, *t.shape[3:]) for t in (o, lse, dq))
    for t in (o_r, l_r, dq_r):  # every query copy computes the same rows
        assert bool((t == t[:, :, :1]).all()), "query copies differ"
    got = {"o": inp.from_torch(o_r[:, :, 0], "f32"), "lse": inp.from_torch(l_r[:, :, 0], "f32"),
           "dq": inp.from_torch(dq_r[:, :, 0], "f32"), "dk": inp.from_torch(dk, "f32") / R,
           "dv": inp.from_torch(dv, "f32") / R}
    del o, lse, dq, o_r, l_r, dq_r
    rep = compare(case, got, reference(case, "f32", end_to_end=True))
    print(" ".join(f"{n}={e:.2e}/{b:.2e}" for n, (e, b, _) in rep.items()), flush=True)
