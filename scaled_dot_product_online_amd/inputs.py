"""Seeded synthetic inputs for attention (no attention arithmetic in this module).

Both the HIP path (through the tests, ``bench.py`` and ``smoke()``) and the CPU
oracle consume exactly the arrays built here, so the two sides see bit-identical
operands.

Recipe (PyTensor issue "PERF: detect scaled-dot-product-attention pattern and
lower to mx.fast.scaled_dot_product_attention", section "Reproducer + metrics"):
``numpy.random.default_rng(seed)`` draws standard normals in float64, which are
cast to float32; Q, K, V, dO are drawn in that order. 16-bit operands are then
rounded from float32 to the target format with round-to-nearest-even; the
scale is the float32 value of 1/sqrt(D).

Storage: float32 arrays for "f32", numpy float16 for "f16", and uint16 bit
patterns for "bf16" (numpy has no bfloat16).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DTYPES = ("f32", "f16", "bf16")


def f32_to_bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (finite inputs and
    infinities; no NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def from_f32(x32, dtype):
    """Convert a float32 array to the storage form of ``dtype``."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x32.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"dtype must be one of {DTYPES}")


def as_float64(arr, dtype):
    """Exact widening of a storage array to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr).astype(np.float64)


def default_scale(D):
    """float32(1/sqrt(D)), the scale every workload on the pages uses."""
    return float(np.float32(1.0 / np.sqrt(np.float64(D))))


@dataclass
class Case:
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lkv: int
    D: int
    dtype: str
    is_causal: bool
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray | None

    def f64(self, name):
        return as_float64(getattr(self, name), self.dtype)

    @property
    def shape_str(self):
        return (f"B={self.B} Hq={self.Hq} Hkv={self.Hkv} Lq={self.Lq} Lkv={self.Lkv} D={self.D} "
                f"{self.dtype} causal={int(self.is_causal)}")


def make_case(B, Hq, Hkv, Lq, Lkv, D, dtype, is_causal=False, seed=0, with_grad=True, scale=None):
    """Draw Q, K, V (and dO) for one workload."""
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}")
    rng = np.random.default_rng(seed)

    def draw(shape):
        return from_f32(rng.standard_normal(shape).astype(np.float32), dtype)

    q = draw((B, Hq, Lq, D))
    k = draw((B, Hkv, Lkv, D))
    v = draw((B, Hkv, Lkv, D))
    do = draw((B, Hq, Lq, D)) if with_grad else None
    return Case(B, Hq, Hkv, Lq, Lkv, D, dtype, bool(is_causal),
                default_scale(D) if scale is None else float(np.float32(scale)), q, k, v, do)


def make_mask(kind, shape, dtype, seed=0, p_keep=0.7, empty_rows=0):
    """A seeded synthetic attention mask of ``shape`` (broadcastable to [B, Hq, Lq, Lkv]).

    kind "bool": each key kept with probability ``p_keep``; every row keeps at least
    its first key except the first ``empty_rows`` query rows, which keep none.
    kind "additive": N(0, 4) values in the storage form of ``dtype``, with about 1 in 8
    entries set to -inf (the first key of each row stays finite unless the row is one
    of the ``empty_rows``, which are all -inf).
    Returns a numpy bool array, or a storage array of ``dtype`` (bf16 as bit patterns)."""
    rng = np.random.default_rng(seed)
    if kind == "bool":
        m = rng.random(shape) < p_keep
        m[..., 0] = True
        m[..., :empty_rows, :] = False
        return m
    if kind == "additive":
        x = (rng.standard_normal(shape) * 2.0).astype(np.float32)
        x[rng.random(shape) < 0.125] = -np.inf
        x[..., 0] = (rng.standard_normal(x[..., 0].shape) * 2.0).astype(np.float32)  # finite
        x[..., :empty_rows, :] = -np.inf
        return from_f32(x, dtype)
    raise ValueError("kind must be 'bool' or 'additive'")


def make_key_padding_mask(B, Lkv, keep):
    """Boolean [B, 1, 1, Lkv]: batch b keeps its first keep[b] keys (a padded batch)."""
    keep = np.asarray(keep).reshape(B, 1, 1, 1)
    return np.arange(Lkv)[None, None, None, :] < keep


def make_sinks(Hq, seed=0, none_heads=()):
    """Seeded float32 sink logits, N(0, 1) per query head; heads in ``none_heads`` get -inf."""
    s = np.random.default_rng(seed).standard_normal(Hq).astype(np.float32)
    s[list(none_heads)] = -np.inf
    return s


def to_torch(arr, dtype, device):
    """Move a storage array to a torch tensor of the matching dtype on ``device``."""
    import torch

    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def from_torch(t, dtype):
    """Bring a device tensor back as float64 numpy (exact widening)."""
    import torch

    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    return t.numpy().astype(np.float64)
