"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/sdpa.h declares, and rejects bad arguments before touching memory."""

import ctypes
import os
import re

import pytest

import scaled_dot_product_online_amd as sd
from scaled_dot_product_online_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "sdpa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sdpa_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_lib.SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = sd.library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(8):
        assert sd.status_str(code)
    assert sd.status_str(99) == "unknown status"


def test_select_path():
    assert sd.select_path(32, 4, 4096, 4096, 128, True, sd.BF16) == sd.PATH_TILED
    assert sd.select_path(32, 8, 8, 8192, 128, False, sd.BF16) == sd.PATH_VECTOR
    assert sd.select_path(32, 8, 1, 8192, 64, False, sd.F16) == sd.PATH_VECTOR
    assert sd.select_path(32, 8, 8, 8, 64, True, sd.F16) == sd.PATH_VECTOR     # causal short queries stream too
    assert sd.select_path(32, 8, 8, 4096, 64, True, sd.F16) == sd.PATH_VECTOR  # decode against a long cache
    assert sd.select_path(32, 8, 9, 8192, 64, False, sd.F16) == sd.PATH_TILED
    assert sd.select_path(64, 4, 8, 8192, 64, False, sd.F16) == sd.PATH_TILED  # 16*8 rows exceed one block
    assert sd.select_path(8, 8, 128, 128, 64, False, sd.F32) == sd.PATH_FP32
    assert sd.select_path(8, 8, 128, 128, 96, False, sd.F16) == sd.PATH_TILED
    assert sd.select_path(8, 8, 128, 128, 80, False, sd.F16) == -1           # unsupported head dim
    assert sd.select_path(8, 8, 128, 64, 64, True, sd.F16) == -1             # causal needs Lq <= Lkv
    assert sd.select_path(8, 8, 64, 128, 64, True, sd.F16) == sd.PATH_TILED  # Lq < Lkv causal: ends aligned
    assert sd.select_path(8, 3, 128, 128, 64, False, sd.F16) == -1           # Hq % Hkv


def test_workspace_sizes():
    # the tiled forward needs none on grids that fill the chip, the fp32 forward none at all;
    # backward keeps Delta (fp32 per query row)
    assert sd.workspace_bytes(0, 4, 32, 4, 4096, 4096, 128, True, sd.BF16) == 0
    assert sd.workspace_bytes(0, 8, 8, 8, 128, 128, 64, False, sd.F32) == 0
    # small tiled grids split the keys: fp32 partials O [nsplit, B*Hq*Lq, D] and (m, l), with
    # enough splits for one 128-row workgroup per CU at D = 64 (8 heads of 2048 rows: 2)
    assert sd.workspace_bytes(0, 1, 8, 8, 2048, 2048, 64, False, sd.F16) == 2 * 8 * 2048 * (64 + 2) * 4
    assert sd.workspace_bytes(0, 1, 8, 8, 4096, 4096, 64, True, sd.F16) == 0  # 256 workgroups: no split
    # a causal dQ on a small grid keeps one split per 2048 keys (here 2), and causal dK/dV aims for
    # two workgroups per CU: L = 4096 splits its query tiles 2 ways
    rows = 8 * 4096
    assert sd.workspace_bytes(1, 1, 8, 8, 4096, 4096, 64, True, sd.F16) == rows * 8 + 2 * rows * 64 * 4 + 2 * (
        2 * rows * 64 * 4)
    assert sd.workspace_bytes(1, 1, 8, 8, 4096, 4096, 64, False, sd.F16) == rows * 8
    assert sd.workspace_bytes(0, 1, 2, 2, 200, 200, 64, True, sd.F16) == 0  # too few key tiles to split
    # ... and so does the backward: {LSE*log2e, Delta} pairs, dQ partials (2 key splits), dK and dV
    # partials (2 splits of the query tiles)
    rows, kv = 8 * 2048, 8 * 2048
    assert sd.workspace_bytes(1, 1, 8, 8, 2048, 2048, 64, False, sd.F16) == rows * 8 + 2 * rows * 64 * 4 + 2 * (
        2 * kv * 64 * 4)
    # a causal dQ on a small grid keeps one key split per 2048 keys: 4 heads of 4100 rows (132
    # workgroups) take 3 splits, not the 2 of one workgroup per CU; dK/dV aims for two workgroups
    # per CU there (2 Lq > Lkv): 4 splits of its 65 query tiles
    rows = 4 * 4100
    assert sd.workspace_bytes(1, 1, 4, 4, 4100, 4100, 32, True, sd.BF16) == 4 * 4160 * 8 + 3 * rows * 32 * 4 + 2 * (
        4 * rows * 32 * 4)
    # ... and only one per CU where the causal triangle is short (1024 queries against 4096
    # keys): dQ 4 splits, dK/dV 8 of its 32 workgroups
    assert sd.workspace_bytes(1, 1, 8, 1, 1024, 4096, 128, True, sd.BF16) == 8 * 1024 * 8 + 4 * 8 * 1024 * 128 * 4 + 2 * (
        8 * 4096 * 128 * 4)
    assert sd.workspace_bytes(1, 4, 32, 4, 4096, 4096, 128, True, sd.BF16) >= 4 * 32 * 4096 * 4
    assert sd.workspace_bytes(1, 8, 8, 8, 128, 128, 64, False, sd.F32) >= 8 * 8 * 128 * 4
    # vector path: split partials
    assert sd.workspace_bytes(0, 16, 32, 8, 8, 8192, 128, False, sd.BF16) > 0
    assert sd.workspace_bytes(1, 16, 32, 8, 8, 8192, 128, False, sd.BF16) >= 16 * 32 * 8 * 128 * 4
    with pytest.raises(sd.SdpaError):
        sd.workspace_bytes(0, 0, 1, 1, 1, 1, 64, False, sd.F16)


def _no_device():
    """The validation tests pass fake, never-dereferenced pointers; they only run where no
    GPU is visible, so that a validation slip cannot turn into a launch on real memory."""
    from conftest import gpu_available

    if gpu_available():
        pytest.skip("fake-pointer validation tests run only without a GPU")


def _fwd(lib, q=1, k=1, v=1, o=1, lse=0, B=1, Hq=1, Hkv=1, Lq=16, Lkv=16, D=64, scale=0.125, causal=0, dt=1,
         odt=1, ws=0, wsb=0):
    p = lambda x: ctypes.c_void_p(x * 256 if x else 0)  # noqa: E731  (aligned fake addresses, never dereferenced)
    return lib.sdpa_fwd(p(q), p(k), p(v), p(o), p(lse), B, Hq, Hkv, Lq, Lkv, D, scale, causal, dt, odt, p(ws), wsb,
                        None)


def test_forward_validation_rejects_before_launch():
    _no_device()
    lib = sd.library()
    assert _fwd(lib, q=0) == 1                        # NULL
    assert _fwd(lib, B=0) == 2                        # shape
    assert _fwd(lib, Hq=3, Hkv=2) == 2                # Hq % Hkv
    assert _fwd(lib, D=80) == 3                       # head dim
    assert _fwd(lib, Lq=32, Lkv=16, causal=1) == 3    # causal needs Lq <= Lkv
    assert _fwd(lib, dt=1, odt=2) == 3                # out dtype must be dtype or f32
    assert _fwd(lib, dt=0, odt=1) == 3                # f32 operands need f32 outputs
    assert _fwd(lib, dt=5) == 3
    assert _fwd(lib, scale=float("inf")) == 7
    assert _fwd(lib, scale=float("nan")) == 7
    assert _fwd(lib, B=1 << 40, Hq=1 << 20) == 2      # overflow
    assert _fwd(lib, Lq=4, Lkv=8192, Hq=8, Hkv=2) == 4  # vector path needs its workspace
    misaligned = lib.sdpa_fwd(ctypes.c_void_p(258), ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256),
                              None, 1, 1, 1, 16, 16, 64, 0.125, 0, 1, 1, None, 0, None)
    assert misaligned == 5


def test_backward_requires_lse_and_workspace():
    _no_device()
    lib = sd.library()
    p = lambda x: ctypes.c_void_p(x * 256 if x else 0)  # noqa: E731
    args = [p(1), p(1), p(1), p(1), p(0), p(1), p(1), p(1), p(1), 1, 1, 1, 16, 16, 64, 0.125, 0, 1, 1, p(1), 1 << 20,
            None]
    assert lib.sdpa_bwd(*args) == 1                    # lse is required
    args[4] = p(1)
    args[19], args[20] = p(0), 0
    assert lib.sdpa_bwd(*args) == 4                    # workspace required
    args[19], args[20] = ctypes.c_void_p(256 + 16), 1 << 20
    assert lib.sdpa_bwd(*args) == 5                    # workspace alignment


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.library()


def _fwdm(lib, kind=1, mask=1, sb=0, sh=0, sq=16, sinks=0, causal=0, dt=1, mask_addr=None, sinks_addr=None):
    p = lambda x: ctypes.c_void_p(x * 256 if x else 0)  # noqa: E731  (aligned fake addresses, never dereferenced)
    m = ctypes.c_void_p(mask_addr) if mask_addr is not None else p(mask)
    sk = ctypes.c_void_p(sinks_addr) if sinks_addr is not None else p(sinks)
    return lib.sdpa_fwd_masked(p(1), p(1), p(1), p(1), p(0), 1, 2, 1, 16, 16, 64, 0.125, causal, kind, m, sb, sh, sq,
                               sk, dt, dt, p(0), 0, None)


def _bwdm(lib, kind=1, sinks=0, dsinks=0):
    p = lambda x: ctypes.c_void_p(x * 256 if x else 0)  # noqa: E731
    return lib.sdpa_bwd_masked(p(1), p(1), p(1), p(1), p(1), p(1), p(1), p(1), p(1), 1, 2, 1, 16, 16, 64, 0.125, 0,
                               kind, p(1), 0, 0, 16, p(sinks), p(dsinks), 1, 1, p(1), 1 << 20, None)


def test_masked_validation_rejects_before_launch():
    _no_device()
    lib = sd.library()
    assert _fwdm(lib, kind=3) == 7                    # unknown mask kind
    assert _fwdm(lib, mask=0) == 1                    # mask kind set, no mask
    assert _fwdm(lib, causal=1) == 3                  # a mask with the causal flag
    assert _fwdm(lib, sq=-1) == 2                     # negative stride
    assert _fwdm(lib, sh=1 << 62) == 2                # (Hq-1)*sh beyond int64 / 8
    assert _fwdm(lib, kind=2, mask_addr=257) == 5     # additive 16-bit mask on an odd address
    assert _fwdm(lib, kind=1, sinks_addr=258) == 5    # sinks not 4-byte aligned
    assert _bwdm(lib, sinks=1, dsinks=0) == 1         # sinks without dsinks


def test_mask_kind_none_ignores_the_mask_arguments():
    _no_device()
    lib = sd.library()
    # NONE with garbage strides and no pointer validates like sdpa_fwd (here: bad head dim).
    p = lambda x: ctypes.c_void_p(x * 256 if x else 0)  # noqa: E731
    st = lib.sdpa_fwd_masked(p(1), p(1), p(1), p(1), p(0), 1, 2, 1, 16, 16, 80, 0.125, 1, 0, p(0), -5, -5, -5, p(0),
                             1, 1, p(0), 0, None)
    assert st == 3


# ---- the Python binding checks every tensor before any call into the library -------------

def _meta(shape, dtype=None):
    import torch

    names = {"f16": torch.float16, "f32": torch.float32, "bf16": torch.bfloat16, "u8": torch.uint8,
             "bool": torch.bool}
    return torch.empty(shape, dtype=names.get(dtype, dtype) if dtype is not None else torch.bfloat16, device="meta")


@pytest.fixture
def as_gpu(monkeypatch):
    """Pose meta tensors (no memory behind them) as tensors on cuda:0, so that only the
    shape, dtype and layout rules decide; a check that let one through would go on to ask
    the library for a workspace size and then fail on the missing stream, never launching."""
    import torch

    monkeypatch.setattr(torch.Tensor, "device", property(lambda self: torch.device("cuda", 0)))


B, HQ, HKV, LQ, LKV, D = 2, 4, 2, 16, 24, 64


def _fwd_args():
    return dict(q=_meta((B, HQ, LQ, D)), k=_meta((B, HKV, LKV, D)), v=_meta((B, HKV, LKV, D)),
                out=_meta((B, HQ, LQ, D)), lse=_meta((B, HQ, LQ), "f32"))


@pytest.mark.parametrize("change,match", [
    (dict(k=_meta((B + 1, HKV, LKV, D)), v=_meta((B + 1, HKV, LKV, D))), "batch or head size"),
    (dict(k=_meta((B, HKV, LKV, 32)), v=_meta((B, HKV, LKV, 32))), "batch or head size"),
    (dict(v=_meta((B, HKV, LKV + 1, D))), "differ"),
    (dict(k=_meta((B, HKV, LKV, D), "f16")), "dtypes differ"),
    (dict(q=_meta((B, 3, LQ, D)), ), "not a multiple"),
    (dict(out=_meta((B, HQ, LQ + 1, D))), "out has shape"),
    (dict(out=_meta((B, HQ, LQ, D), "f32")), "out has dtype"),
    (dict(lse=_meta((B, HQ, LQ), "bf16")), "lse has dtype"),
    (dict(lse=_meta((B, HQ, LQ + 1), "f32")), "lse has shape"),
    (dict(workspace=_meta((16,), "u8"), q=_meta((B, HQ, 4, D)), k=_meta((B, HKV, 8192, D)),
          v=_meta((B, HKV, 8192, D)), out=_meta((B, HQ, 4, D)), lse=_meta((B, HQ, 4), "f32")), "workspace holds"),
    (dict(attn_mask=_meta((B, 1, LQ, LKV + 1), "bool")), "does not broadcast"),
    (dict(attn_mask=_meta((B, 1, LQ, LKV), "f16")), "attn_mask must be bool"),
    (dict(sinks=_meta((HQ + 1,), "f32")), "sinks must be float32"),
])
def test_binding_forward_rejects_mismatched_tensors(as_gpu, change, match):
    args = _fwd_args()
    args.update(change)
    q, k, v = args.pop("q"), args.pop("k"), args.pop("v")
    with pytest.raises(ValueError, match=match):
        sd.sdpa_fwd(q, k, v, **args)


@pytest.mark.parametrize("which,shape,dt,match", [
    ("o", (B, HQ, LQ, D + 1), None, "o has shape"),
    ("o", (B, HQ, LQ, D), "f32", "o has dtype"),
    ("lse", (B, HQ), "f32", "lse has shape"),
    ("dO", (B, HQ, LQ, D), "f16", "dO has dtype"),
    ("dO", (B, HQ, LQ - 1, D), None, "dO has shape"),
    ("dq", (B, HQ, LQ, D), "f32", "dq has dtype"),
    ("dk", (B, HQ, LKV, D), None, "dk has shape"),
    ("dv", (B, HKV, LKV - 1, D), None, "dv has shape"),
    ("workspace", (8,), "u8", "workspace holds"),
])
def test_binding_backward_rejects_mismatched_tensors(as_gpu, which, shape, dt, match):
    import torch

    dtypes = {None: torch.bfloat16, "f16": torch.float16, "f32": torch.float32, "u8": torch.uint8}
    args = dict(o=_meta((B, HQ, LQ, D)), lse=_meta((B, HQ, LQ), torch.float32), dO=_meta((B, HQ, LQ, D)),
                dq=_meta((B, HQ, LQ, D)), dk=_meta((B, HKV, LKV, D)), dv=_meta((B, HKV, LKV, D)))
    args[which] = _meta(shape, dtypes[dt])
    q, k, v = _meta((B, HQ, LQ, D)), _meta((B, HKV, LKV, D)), _meta((B, HKV, LKV, D))
    o, lse, dO = args.pop("o"), args.pop("lse"), args.pop("dO")
    with pytest.raises(ValueError, match=match):
        sd.sdpa_bwd(q, k, v, o, lse, dO, **args)


def test_binding_refuses_host_tensors():
    import torch

    q = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU only"):
        sd.sdpa_fwd(q, q, q)
    with pytest.raises(ValueError, match="GPU only"):
        sd.sdpa_bwd(q, q, q, q, torch.zeros((1, 2, 8)), q)


def test_noalloc_rejects_sizes_beyond_its_scratch_before_any_device_call():
    _no_device()
    lib = sd.library()
    p = lambda x: ctypes.c_void_p(x * 256 if x else 0)  # noqa: E731  (never dereferenced)
    ptrs = [p(1)] * 9
    # 2 x 64 x 16384 query rows of {LSE, Delta} pairs (8 bytes) = 16 MiB fits the 64 MiB scratch;
    # with small-grid partials a tiny-grid shape can need more. 16 x 64 x 65536 rows: 512 MiB.
    assert lib.sdpa_bwd_noalloc(*ptrs, 16, 64, 8, 65536, 65536, 128, 0.125, 1, 2, 2, None) == 4
    assert lib.sdpa_bwd_noalloc(*ptrs, 0, 64, 8, 64, 64, 128, 0.125, 1, 2, 2, None) == 2  # shape checks first
    ptrs[4] = p(0)
    assert lib.sdpa_bwd_noalloc(*ptrs, 1, 8, 8, 64, 64, 64, 0.125, 0, 1, 1, None) == 1  # lse is required
    assert sd.workspace_bytes(1, 16, 64, 8, 65536, 65536, 128, True, sd.BF16) > _lib.NOALLOC_SCRATCH_BYTES
