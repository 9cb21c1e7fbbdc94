"""Fused scaled-dot-product attention for AMD Instinct MI355X (gfx950).

The computation lives in libsdpa_mi355x.so (hand-written HIP kernels behind the C
ABI of include/sdpa.h); this package is its Python binding:

    sdpa_fwd(q, k, v, scale=None, is_causal=False, out_dtype=None, need_lse=True,
             attn_mask=None, sinks=None) -> (o, lse)
    sdpa_bwd(q, k, v, o, lse, dO, scale=None, is_causal=False, out_dtype=None,
             attn_mask=None, sinks=None) -> (dq, dk, dv[, dsinks])
    attention(q, k, v, scale=None, is_causal=False, attn_mask=None, sinks=None) -> o
        differentiable (torch.autograd) wrapper over the two calls above

Tensors are contiguous [B, H, L, D] torch tensors on the GPU in float32, float16
or bfloat16; K/V may have fewer heads than Q (grouped-query attention).
"""

from ._lib import (  # noqa: F401
    BF16,
    F16,
    F32,
    MASK_ADDITIVE,
    MASK_BOOL,
    MASK_NONE,
    PATH_FP32,
    PATH_NAMES,
    PATH_TILED,
    PATH_VECTOR,
    SdpaError,
    library,
    sdpa_bwd,
    sdpa_bwd_noalloc,
    sdpa_fwd,
    select_path,
    status_str,
    workspace_bytes,
)

from .autograd import attention, check_eligible  # noqa: F401,E402
