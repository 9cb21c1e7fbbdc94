"""The attention workloads that the tests and the benchmark run (shapes only).

Each entry is (name, B, Hq, Hkv, Lq, Lkv, D, dtype, is_causal). Sources:
* ``fp32_tiny`` and ``fp32_b8h8s128`` — PyTensor issue "PERF: detect
  scaled-dot-product-attention pattern ...", section "Reproducer + metrics"
  (B, H, S, hd = 8, 8, 128, 64, float32, seed 0); the tiny case is a reduced copy
  of it for an oracle that finishes in well under a second.
* ``fp16_h8_*`` — mps-flash-sdpa 0.1.0, sections "Quick Start" ([1, 8, 2048, 64]
  fp16, causal on and off) and "Benchmarks" (sequence 2048 and 4096).
* ``bf16_gqa8_causal_4k_d128`` — grouped-query attention with causal masking
  (MLX pull request "[Metal] Add Flash Attention VJP for training", sections
  "Key Features" and "Test Plan": GQA 8:1) at a long-context training shape.
* ``vec_*`` — the short-query path (same pull request, "Implementation Notes",
  vector VJP for L <= 8) with Lq != Lkv ("Test Plan", edge cases); the ``_causal``
  one is causal decode rows against an 8192-key cache (sequences aligned at their
  ends).
* ``bf16_gqa8_causal_q1k_kv4k_d128`` — a causal 1024-query chunk against 4096 keys
  (Lq != Lkv, "Test Plan"), the GQA shape above.
* ``*_d96`` and ``*_d256`` — the GQA and short-query shapes above at head dims 96
  (listed in the same pull request's "Test Plan") and 256 (which that pull request's
  vector VJP leaves out for lack of threadgroup memory, "Limitations").
* ``*_keypad*`` and ``*_sinks*`` — the GQA and short-query shapes with a boolean
  key-padding mask (batch b keeps its first Lkv - (b mod 4)*Lkv/8 keys) and/or one sink logit
  per query head (N(0, 1)): the masks and sinks that mps-flash-sdpa ("When MFA
  Dispatches vs. Falls Back") and the MLX pull request ("Limitations") hand back to
  unfused attention. Their work is counted like the unmasked shape's (the kernels
  visit every key tile; a mask removes no tile).
"""

from __future__ import annotations

WORKLOADS = [
    ("fp32_tiny", 1, 2, 2, 64, 64, 32, "f32", False),
    ("fp32_b8h8s128", 8, 8, 8, 128, 128, 64, "f32", False),
    ("fp16_h8_2k", 1, 8, 8, 2048, 2048, 64, "f16", False),
    ("fp16_h8_2k_causal", 1, 8, 8, 2048, 2048, 64, "f16", True),
    ("fp16_h8_4k", 1, 8, 8, 4096, 4096, 64, "f16", False),
    ("fp16_h8_4k_causal", 1, 8, 8, 4096, 4096, 64, "f16", True),
    ("bf16_gqa8_causal_4k_d128", 4, 32, 4, 4096, 4096, 128, "bf16", True),
]
for _dt in ("f16", "bf16"):
    for _lq in (1, 4, 8):
        for _d in (64, 128):
            WORKLOADS.append((f"vec_{_dt}_lq{_lq}_d{_d}", 16, 32, 8, _lq, 8192, _d, _dt, False))
WORKLOADS += [
    ("vec_bf16_lq8_d128_causal", 16, 32, 8, 8, 8192, 128, "bf16", True),
    ("bf16_gqa8_causal_q1k_kv4k_d128", 4, 32, 4, 1024, 4096, 128, "bf16", True),
    ("bf16_gqa8_causal_4k_d96", 4, 32, 4, 4096, 4096, 96, "bf16", True),
    ("bf16_gqa8_causal_4k_d256", 4, 32, 4, 4096, 4096, 256, "bf16", True),
    ("vec_bf16_lq8_d96", 16, 32, 8, 8, 8192, 96, "bf16", False),
    ("vec_bf16_lq8_d256", 16, 32, 8, 8, 8192, 256, "bf16", False),
    ("bf16_gqa8_keypad_4k_d128", 4, 32, 4, 4096, 4096, 128, "bf16", False),
    ("bf16_gqa8_causal_sinks_4k_d128", 4, 32, 4, 4096, 4096, 128, "bf16", True),
    ("vec_bf16_lq8_d128_keypad_sinks", 16, 32, 8, 8, 8192, 128, "bf16", False),
]

# Masks and sinks of the workloads that have them: "keypad" = inputs.make_key_padding_mask
# with keep[b] = Lkv - (b % 4) * Lkv // 8; sinks = inputs.make_sinks(Hq, seed=0).
MASKED = {
    "bf16_gqa8_keypad_4k_d128": {"mask": "keypad", "sinks": False},
    "bf16_gqa8_causal_sinks_4k_d128": {"mask": None, "sinks": True},
    "vec_bf16_lq8_d128_keypad_sinks": {"mask": "keypad", "sinks": True},
}


def mask_and_sinks(name):
    """(mask, sinks) for a workload: mask None or ("bool", array), sinks None or float32 [Hq]."""
    from . import inputs as inp

    spec = MASKED.get(name)
    if spec is None:
        return None, None
    _, B, Hq, Hkv, Lq, Lkv, D, dt, causal = BY_NAME[name]
    mask = None
    if spec["mask"] == "keypad":
        mask = ("bool", inp.make_key_padding_mask(B, Lkv, [Lkv - (b % 4) * Lkv // 8 for b in range(B)]))
    sinks = inp.make_sinks(Hq, seed=0) if spec["sinks"] else None
    return mask, sinks

BY_NAME = {w[0]: w for w in WORKLOADS}

# The workload the headline throughput is quoted on.
HEADLINE = "bf16_gqa8_causal_4k_d128"


def flops(B, Hq, Lq, Lkv, D, is_causal, backward=False):
    """Counted FLOPs: 4*B*Hq*D per (query, key) pair forward, 2.5x that for the backward.

    Pairs: Lq*Lkv; causal (sequences aligned at their ends) Lq*Lkv - Lq*Lq/2, which is
    half of Lq*Lkv when the lengths are equal (the usual "halved for causal")."""
    pairs = Lq * Lkv - (Lq * Lq / 2.0 if is_causal else 0.0)
    f = 4.0 * B * Hq * pairs * D
    return f * 2.5 if backward else f
