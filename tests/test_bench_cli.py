"""bench.py on the CPU: the FLOP convention, the kernel names its traffic lookup uses, and
the one-GPU refusal (no GPU needed)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from scaled_dot_product_online_amd.workloads import BY_NAME, HEADLINE, flops  # noqa: E402


def test_flop_convention():
    # forward 4*B*Hq*Lq*Lkv*D, halved for causal with equal lengths; backward 2.5x
    assert flops(4, 32, 4096, 4096, 128, False) == 4 * 4 * 32 * 4096 * 4096 * 128
    assert flops(4, 32, 4096, 4096, 128, True) == 4 * 4 * 32 * 4096 * 4096 * 128 / 2
    assert flops(4, 32, 4096, 4096, 128, True, backward=True) == 2.5 * flops(4, 32, 4096, 4096, 128, True)
    # causal with fewer queries than keys (ends aligned): Lq*Lkv - Lq^2/2 visible pairs
    assert flops(1, 1, 2, 5, 1, True) == 4 * (2 * 5 - 2)
    # the headline: 549.8 GFLOP forward, 1374.4 backward
    _, B, Hq, Hkv, Lq, Lkv, D, dt, causal = BY_NAME[HEADLINE]
    assert abs(flops(B, Hq, Lq, Lkv, D, causal) / 1e9 - 549.76) < 0.01
    assert abs(flops(B, Hq, Lq, Lkv, D, causal, backward=True) / 1e9 - 1374.39) < 0.01


class _Case:
    def __init__(self, dtype, causal, D):
        self.dtype, self.is_causal, self.D = dtype, causal, D


class _Runner:
    def __init__(self, path, dtype, causal, D, masked=False):
        self.path, self.case, self.mask = path, _Case(dtype, causal, D), (object() if masked else None)


def test_kernel_symbols():
    r = _Runner("tiled", "bf16", True, 128)
    assert bench.kernel_symbol(r, "fwd") == "fwd_tiled_kernel<bf16_t, 128, true, false, bf16_t>"
    assert bench.kernel_symbol(r, "bwd_stage0") == "dq_kernel<bf16_t, 128, true, false, bf16_t>"
    assert bench.kernel_symbol(r, "bwd_stage1") == "dkv_kernel<bf16_t, 128, true, false, bf16_t>"
    v = _Runner("vector", "f16", False, 64, masked=True)
    assert bench.kernel_symbol(v, "bwd_stage0") == "vec_bwd_kernel<f16_t, 64, false, true, f16_t>"
    assert bench.kernel_symbol(v, "bwd_stage1") == "vec_dq_reduce_kernel<64, f16_t>"
    assert bench.kernel_symbol(_Runner("fp32", "f32", False, 64), "fwd") is None


def test_traffic_lookup_ignores_other_sources(tmp_path, monkeypatch):
    # A summary taken on other kernel sources is never reported.
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "x.traffic.json").write_text(
        '{"source_sha256": "0", "kernels": {"dkv_kernel<bf16_t, 128, true, false, bf16_t, false>": '
        '{"read_bytes": 1, "write_bytes": 2}}}')
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic(_Runner("tiled", "bf16", True, 128), "bwd_stage1") is None


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_traffic_lookup_without_a_kernel_name(monkeypatch):
    # The fp32 path has no kernel name in the lookup: no traffic, and no error, even when a
    # summary of the current sources exists.
    monkeypatch.setattr(bench, "kernel_symbol", lambda r, label: None)
    assert bench.measured_traffic(_Runner("fp32", "f32", False, 64), "fwd") is None
