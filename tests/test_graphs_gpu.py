"""HIP-graph capture of the C-ABI calls.

The library only enqueues kernels on the caller's stream (no allocation, no
synchronisation, no memset), so a caller can capture sdpa_fwd / sdpa_bwd (and the
masked entry points) in a graph and replay it. Each case captures one forward +
backward with static buffers, replays the graph several times with unrelated eager
work and a synchronisation between the replays, and checks every replay bit for bit
against the eager call on the same inputs. Covers the tiled, short-query and float32
paths, causal and masked with sinks, and head dim 256.
"""

import pytest

from scaled_dot_product_online_amd import inputs as inp

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, Lq, Lkv, D, dtype, causal, masked (key padding + sinks)
    (1, 8, 2, 200, 200, 128, "bf16", True, False),   # tiled
    (2, 8, 2, 8, 3000, 64, "bf16", False, True),      # short-query, several splits
    (1, 4, 2, 70, 130, 64, "f16", False, True),       # tiled with a mask
    (1, 4, 1, 256, 1024, 64, "f16", False, True),     # tiled, small grid: forward and dQ split 4 ways, dK/dV 2
    (1, 2, 2, 40, 60, 32, "f32", True, False),        # float32 path
    (1, 4, 2, 130, 260, 256, "f16", True, False),     # head dim 256: two-wave forward, 16-row dQ
    (1, 4, 2, 150, 300, 256, "bf16", False, True),    # head dim 256 with a mask (the forward spills registers)
]


def _id(c):
    return f"{c[6]}-L{c[3]}x{c[4]}-D{c[5]}-{'causal' if c[7] else 'full'}{'-mask-sinks' if c[8] else ''}"


@pytest.mark.parametrize("c", CASES, ids=[_id(c) for c in CASES])
def test_graph_replays_equal_eager(device, c):
    import torch

    import scaled_dot_product_online_amd as sd

    B, Hq, Hkv, Lq, Lkv, D, dt, causal, masked = c
    case = inp.make_case(B, Hq, Hkv, Lq, Lkv, D, dt, is_causal=causal, seed=21)
    q, k, v, do = (inp.to_torch(getattr(case, n), dt, device) for n in ("q", "k", "v", "do"))
    extra = {}
    if masked:
        keep = [Lkv - 7 * b for b in range(B)]
        extra = {"attn_mask": torch.from_numpy(inp.make_key_padding_mask(B, Lkv, keep)).to(device),
                 "sinks": torch.from_numpy(inp.make_sinks(Hq, seed=1)).to(device)}
    code = {"f32": sd.F32, "f16": sd.F16, "bf16": sd.BF16}[dt]
    o, lse = torch.empty_like(q), torch.empty((B, Hq, Lq), dtype=torch.float32, device=device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsinks = torch.empty(Hq, dtype=torch.float32, device=device) if masked else None
    wf = torch.empty(max(sd.workspace_bytes(0, B, Hq, Hkv, Lq, Lkv, D, causal, code), 256), dtype=torch.uint8,
                     device=device)
    wb = torch.empty(max(sd.workspace_bytes(1, B, Hq, Hkv, Lq, Lkv, D, causal, code), 256), dtype=torch.uint8,
                     device=device)

    def step():
        sd.sdpa_fwd(q, k, v, scale=case.scale, is_causal=causal, out=o, lse=lse, workspace=wf, **extra)
        sd.sdpa_bwd(q, k, v, o, lse, do, scale=case.scale, is_causal=causal, dq=dq, dk=dk, dv=dv, workspace=wb,
                    dsinks=dsinks, **extra)

    outs = lambda: [t.clone() for t in (o, lse, dq, dk, dv) + ((dsinks,) if masked else ())]  # noqa: E731
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager, on the stream the graph is captured on
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    want = outs()
    for t in (o, lse, dq, dk, dv):
        t.zero_()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        got = outs()
        print(f"[graph] {_id(c)} replay {r}", flush=True)
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs from the eager call"
        # unrelated eager work between replays
        junk = torch.randn(1 << 20, device=device)
        (junk * 2).sum().item()
        for t in (o, dq):
            t.zero_()
