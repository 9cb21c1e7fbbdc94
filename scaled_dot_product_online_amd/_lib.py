"""ctypes binding of libsdpa_mi355x.so: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI declared
in include/sdpa.h. This module turns torch tensors into device pointers, allocates
outputs and the workspace with torch (device memory is plumbing here), passes
torch's current HIP stream, and raises ``SdpaError`` on a non-zero status. There
is no fallback: if the library is missing, loading it raises.
"""

from __future__ import annotations

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libsdpa_mi355x.so")

F32, F16, BF16 = 0, 1, 2
PATH_TILED, PATH_VECTOR, PATH_FP32 = 0, 1, 2
PATH_NAMES = {PATH_TILED: "tiled", PATH_VECTOR: "vector", PATH_FP32: "fp32"}
MASK_NONE, MASK_BOOL, MASK_ADDITIVE = 0, 1, 2
SYMBOLS = ("sdpa_select_path", "sdpa_workspace_bytes", "sdpa_fwd", "sdpa_bwd", "sdpa_bwd_stage", "sdpa_fwd_masked",
           "sdpa_bwd_masked", "sdpa_bwd_masked_stage", "sdpa_bwd_noalloc", "sdpa_status_str")
NOALLOC_SCRATCH_BYTES = 64 << 20  # SDPA_NOALLOC_SCRATCH_BYTES in include/sdpa.h

_lib = None


class SdpaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"sdpa status {status}: {msg}")
        self.status = status


def library():
    """Load the shared library once (raises OSError/RuntimeError when it is absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m scaled_dot_product_online_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, c_int, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.sdpa_select_path.argtypes = [i64, i64, i64, i64, i64, c_int, c_int]
    lib.sdpa_select_path.restype = c_int
    lib.sdpa_workspace_bytes.argtypes = [c_int, i64, i64, i64, i64, i64, i64, c_int, c_int]
    lib.sdpa_workspace_bytes.restype = ctypes.c_size_t
    lib.sdpa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, c_int, c_int, c_int, vp,
                             ctypes.c_size_t, vp]
    lib.sdpa_fwd.restype = c_int
    lib.sdpa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, c_int, c_int,
                             c_int, vp, ctypes.c_size_t, vp]
    lib.sdpa_bwd.restype = c_int
    lib.sdpa_bwd_stage.argtypes = [c_int] + lib.sdpa_bwd.argtypes
    lib.sdpa_bwd_stage.restype = c_int
    mask_args = [c_int, vp, i64, i64, i64]
    lib.sdpa_fwd_masked.argtypes = lib.sdpa_fwd.argtypes[:13] + mask_args + [vp] + lib.sdpa_fwd.argtypes[13:]
    lib.sdpa_fwd_masked.restype = c_int
    lib.sdpa_bwd_masked.argtypes = lib.sdpa_bwd.argtypes[:17] + mask_args + [vp, vp] + lib.sdpa_bwd.argtypes[17:]
    lib.sdpa_bwd_masked.restype = c_int
    lib.sdpa_bwd_masked_stage.argtypes = [c_int] + lib.sdpa_bwd_masked.argtypes
    lib.sdpa_bwd_masked_stage.restype = c_int
    lib.sdpa_bwd_noalloc.argtypes = lib.sdpa_bwd.argtypes[:19] + [vp]
    lib.sdpa_bwd_noalloc.restype = c_int
    lib.sdpa_status_str.argtypes = [c_int]
    lib.sdpa_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_str(status):
    return library().sdpa_status_str(int(status)).decode()


def _check(status):
    if status != 0:
        raise SdpaError(status, status_str(status))


def select_path(Hq, Hkv, Lq, Lkv, D, is_causal, dtype):
    return library().sdpa_select_path(Hq, Hkv, Lq, Lkv, D, int(bool(is_causal)), dtype)


def workspace_bytes(backward, B, Hq, Hkv, Lq, Lkv, D, is_causal, dtype):
    n = library().sdpa_workspace_bytes(int(bool(backward)), B, Hq, Hkv, Lq, Lkv, D, int(bool(is_causal)), dtype)
    if n == ctypes.c_size_t(-1).value:
        raise SdpaError(2, "invalid sizes")
    return n


# ---- torch-facing wrappers -------------------------------------------------------------

def _torch_code(t):
    import torch

    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t not in codes:
        raise TypeError(f"unsupported dtype {t}")
    return codes[t]


def _torch_dtype(code):
    import torch

    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[code]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(dev, stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return ctypes.c_void_p(stream.cuda_stream)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, L, D]")


_HEAD_DIMS = (32, 64, 96, 128, 256)


def check_eligible(q, k, v, is_causal=False, attn_mask=None, sinks=None):
    """Raise ValueError naming the first reason the library cannot take these inputs.

    Types, shapes and dtypes are checked first, the devices last (every tensor on the GPU
    of q), so that nothing reaches the C ABI that could make a kernel read or write
    outside a buffer."""
    import torch

    dtypes = (torch.float32, torch.float16, torch.bfloat16)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} is not a tensor")
        if t.dtype not in dtypes:
            raise ValueError(f"{name} has dtype {t.dtype}; supported: float32, float16, bfloat16")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, L, D], got shape {tuple(t.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError(f"q, k, v dtypes differ: {q.dtype}, {k.dtype}, {v.dtype}")
    B, Hq, Lq, D = q.shape
    if k.shape != v.shape:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} differ")
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k/v {tuple(k.shape)} do not match q {tuple(q.shape)} in batch or head size")
    Hkv = k.shape[1]
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"query heads {Hq} are not a multiple of key/value heads {Hkv}")
    if D not in _HEAD_DIMS:
        raise ValueError(f"head size {D} is not supported (supported: {_HEAD_DIMS})")
    if is_causal and Lq > k.shape[2]:
        raise ValueError("causal attention needs Lq <= Lkv (sequences aligned at their ends)")
    if attn_mask is not None:
        if is_causal:
            raise ValueError("attn_mask and is_causal are not combined")
        if not isinstance(attn_mask, torch.Tensor):
            raise ValueError("attn_mask must be a tensor")
        if attn_mask.dtype not in (torch.bool, q.dtype):
            raise ValueError(f"attn_mask must be bool or {q.dtype}, got {attn_mask.dtype}")
        if attn_mask.requires_grad:
            raise ValueError("no gradient is formed for attn_mask")
        try:
            torch.broadcast_shapes(tuple(attn_mask.shape), (B, Hq, Lq, k.shape[2]))
        except RuntimeError:
            raise ValueError(f"attn_mask {tuple(attn_mask.shape)} does not broadcast to {(B, Hq, Lq, k.shape[2])}")
    if sinks is not None:
        if not isinstance(sinks, torch.Tensor):
            raise ValueError("sinks must be a tensor")
        if sinks.dtype != torch.float32 or tuple(sinks.shape) != (Hq,):
            raise ValueError(f"sinks must be float32 of shape ({Hq},)")
    for name, t in (("q", q), ("k", k), ("v", v), ("attn_mask", attn_mask), ("sinks", sinks)):
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} is on {t.device}; the library runs on the GPU only")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")


def check_buffer(name, t, shape, dtype, device):
    """Raise ValueError unless ``t`` is a contiguous tensor of exactly this shape and dtype on ``device``."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} is not a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _workspace_arg(workspace, need, device):
    """(pointer, size in bytes) of a caller's workspace, checked against the size the call needs."""
    if workspace is None:
        return None
    if not workspace.is_contiguous() or workspace.device != device:
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes; this call needs {need}")
    return nbytes


def mask_args(attn_mask, B, Hq, Lq, Lkv, dtype_code):
    """(kind, tensor, stride_b, stride_h, stride_q) for a torch mask broadcastable to [B,Hq,Lq,Lkv].

    A boolean mask keeps the keys where it is True; any other mask must have the
    operand dtype and is added to the scaled scores. Broadcast dimensions are passed
    as stride 0 (no copy); only a mask whose key dimension is broadcast or strided is
    copied, along that dimension."""
    import torch

    if attn_mask is None:
        return MASK_NONE, None, 0, 0, 0
    m = attn_mask
    if m.device.type != "cuda":
        raise ValueError("attn_mask must be on the GPU")
    if m.dtype == torch.bool:
        kind = MASK_BOOL
    elif m.dtype == _torch_dtype(dtype_code):
        kind = MASK_ADDITIVE
    else:
        raise TypeError(f"attn_mask must be bool or {_torch_dtype(dtype_code)}, got {m.dtype}")
    if m.dim() > 4:
        raise ValueError(f"attn_mask has {m.dim()} dimensions; at most 4 ([B, Hq, Lq, Lkv])")
    m = m.reshape((1,) * (4 - m.dim()) + tuple(m.shape))
    if m.shape[3] != Lkv or m.stride(3) != 1:
        m = m.expand(m.shape[0], m.shape[1], m.shape[2], Lkv).contiguous()
    e = m.expand(B, Hq, Lq, Lkv)  # raises if not broadcastable
    return kind, m, e.stride(0), e.stride(1), e.stride(2)


def _sinks_arg(sinks, Hq):
    import torch

    if sinks is None:
        return None
    if sinks.dtype != torch.float32 or tuple(sinks.shape) != (Hq,) or not sinks.is_contiguous():
        raise ValueError(f"sinks must be a contiguous float32 tensor of shape ({Hq},)")
    if sinks.device.type != "cuda":
        raise ValueError("sinks must be on the GPU")
    return sinks


def sdpa_fwd(q, k, v, scale=None, is_causal=False, out_dtype=None, need_lse=True, out=None, lse=None,
             workspace=None, stream=None, attn_mask=None, sinks=None):
    """O (and LSE when ``need_lse``) for BHLD tensors q [B,Hq,Lq,D], k/v [B,Hkv,Lkv,D].

    ``attn_mask`` (bool, or the operand dtype: added to the scaled scores) broadcasts to
    [B,Hq,Lq,Lkv]; ``sinks`` is a float32 [Hq] tensor of per-head sink logits."""
    import torch

    check_eligible(q, k, v, is_causal, attn_mask, sinks)
    _contig(q, k, v)
    B, Hq, Lq, D = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    dt = _torch_code(q.dtype)
    odt = dt if out_dtype is None else _torch_code(out_dtype)
    if scale is None:
        scale = float(torch.tensor(1.0 / D ** 0.5, dtype=torch.float32))
    if out is None:
        out = torch.empty((B, Hq, Lq, D), dtype=_torch_dtype(odt), device=q.device)
    check_buffer("out", out, (B, Hq, Lq, D), _torch_dtype(odt), q.device)
    if need_lse and lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if not need_lse:
        lse = None
    if lse is not None:
        check_buffer("lse", lse, (B, Hq, Lq), torch.float32, q.device)
    nws = workspace_bytes(0, B, Hq, Hkv, Lq, Lkv, D, is_causal, dt)
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    ws_len = _workspace_arg(workspace, nws, q.device) or 0
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Lq, Lkv, D, scale, int(bool(is_causal)))
    tail = (dt, odt, _ptr(workspace), ws_len, _stream(q.device, stream))
    if attn_mask is None and sinks is None:
        st = library().sdpa_fwd(*head, *tail)
    else:
        kind, m, sb, sh, sq = mask_args(attn_mask, B, Hq, Lq, Lkv, dt)
        st = library().sdpa_fwd_masked(*head, kind, _ptr(m), sb, sh, sq, _ptr(_sinks_arg(sinks, Hq)), *tail)
    _check(st)
    return out, lse


def sdpa_bwd(q, k, v, o, lse, dO, scale=None, is_causal=False, out_dtype=None, dq=None, dk=None, dv=None,
             workspace=None, stream=None, stage=None, attn_mask=None, sinks=None, dsinks=None):
    """dQ, dK, dV of sum(O * dO); ``o`` and ``lse`` are what sdpa_fwd returned.

    ``stage`` None runs the whole backward; 0 or 1 runs one stage (sdpa_bwd_stage, or
    sdpa_bwd_masked_stage with a mask or sinks), in which case the same ``workspace``
    (and, with sinks, ``dsinks``) must be passed to both stages. With ``attn_mask`` or
    ``sinks`` (as given to sdpa_fwd) the result is (dq, dk, dv, dsinks), dsinks None
    without sinks."""
    import torch

    check_eligible(q, k, v, is_causal, attn_mask, sinks)
    _contig(q, k, v)
    B, Hq, Lq, D = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    dt = _torch_code(q.dtype)
    odt = dt if out_dtype is None else _torch_code(out_dtype)
    if scale is None:
        scale = float(torch.tensor(1.0 / D ** 0.5, dtype=torch.float32))
    tdt = _torch_dtype(odt)
    check_buffer("o", o, (B, Hq, Lq, D), tdt, q.device)
    check_buffer("lse", lse, (B, Hq, Lq), torch.float32, q.device)
    check_buffer("dO", dO, (B, Hq, Lq, D), q.dtype, q.device)
    dq = torch.empty((B, Hq, Lq, D), dtype=tdt, device=q.device) if dq is None else dq
    dk = torch.empty((B, Hkv, Lkv, D), dtype=tdt, device=q.device) if dk is None else dk
    dv = torch.empty((B, Hkv, Lkv, D), dtype=tdt, device=q.device) if dv is None else dv
    check_buffer("dq", dq, (B, Hq, Lq, D), tdt, q.device)
    check_buffer("dk", dk, (B, Hkv, Lkv, D), tdt, q.device)
    check_buffer("dv", dv, (B, Hkv, Lkv, D), tdt, q.device)
    if sinks is not None and dsinks is not None:
        check_buffer("dsinks", dsinks, (Hq,), torch.float32, q.device)
    nws = workspace_bytes(1, B, Hq, Hkv, Lq, Lkv, D, is_causal, dt)
    if workspace is None:
        workspace = torch.empty(max(nws, 256), dtype=torch.uint8, device=q.device)
    ws_len = _workspace_arg(workspace, nws, q.device)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv),
            B, Hq, Hkv, Lq, Lkv, D, scale, int(bool(is_causal)))
    tail = (dt, odt, _ptr(workspace), ws_len, _stream(q.device, stream))
    if attn_mask is None and sinks is None:
        st = library().sdpa_bwd(*head, *tail) if stage is None else library().sdpa_bwd_stage(int(stage), *head, *tail)
        _check(st)
        return dq, dk, dv
    kind, m, sb, sh, sq = mask_args(attn_mask, B, Hq, Lq, Lkv, dt)
    sk = _sinks_arg(sinks, Hq)
    if sk is not None and dsinks is None:
        dsinks = torch.empty(Hq, dtype=torch.float32, device=q.device)
    masked = (kind, _ptr(m), sb, sh, sq, _ptr(sk), _ptr(dsinks if sk is not None else None))
    if stage is None:
        st = library().sdpa_bwd_masked(*head, *masked, *tail)
    else:
        st = library().sdpa_bwd_masked_stage(int(stage), *head, *masked, *tail)
    _check(st)
    return dq, dk, dv, (dsinks if sk is not None else None)


def sdpa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, scale=None, is_causal=False, stream=None):
    """sdpa_bwd_noalloc: the backward into caller-provided dq, dk, dv (out dtype = their
    dtype), with the library's fixed per-GPU scratch instead of a workspace. Allocates
    nothing; calls that may overlap on one GPU race on the scratch (include/sdpa.h)."""
    import torch

    check_eligible(q, k, v, is_causal)
    _contig(q, k, v)
    B, Hq, Lq, D = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    dt = _torch_code(q.dtype)
    odt = _torch_code(dq.dtype)
    tdt = _torch_dtype(odt)
    if scale is None:
        scale = float(torch.tensor(1.0 / D ** 0.5, dtype=torch.float32))
    check_buffer("o", o, (B, Hq, Lq, D), tdt, q.device)
    check_buffer("lse", lse, (B, Hq, Lq), torch.float32, q.device)
    check_buffer("dO", dO, (B, Hq, Lq, D), q.dtype, q.device)
    check_buffer("dq", dq, (B, Hq, Lq, D), tdt, q.device)
    check_buffer("dk", dk, (B, Hkv, Lkv, D), tdt, q.device)
    check_buffer("dv", dv, (B, Hkv, Lkv, D), tdt, q.device)
    st = library().sdpa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk),
                                    _ptr(dv), B, Hq, Hkv, Lq, Lkv, D, scale, int(bool(is_causal)), dt, odt,
                                    _stream(q.device, stream))
    _check(st)
    return dq, dk, dv
