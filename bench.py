#!/usr/bin/env python3
"""Throughput of the fused attention hot path on one MI355X.

A step is one pass of the whole path on one batch of synthetic input: the forward
(O and the logsumexp) followed by the backward's two stages (dQ, then dK/dV), on
the workload the headline metric is quoted on (bf16, GQA 8:1, causal, B=4,
Hq=32, Hkv=4, L=4096, D=128; inputs i.i.d. N(0,1) from seed 0, resident in HBM
before timing starts). FLOPs are counted as 4*B*Hq*D per visible (query, key) pair
for the forward and 2.5x that for the backward: Lq*Lkv pairs, halved for causal
masking when Lq == Lkv (Lq*Lkv - Lq*Lq/2 when causal with fewer queries).

Prints ONE JSON line (rank 0, N=1). Besides the contract fields it carries:
  roofline      the dominant kernel's algorithmic FLOPs per launch over its mean
                launch time (HIP events on the launch stream) against dense MFMA peak
  cpu_baseline  the fp64 oracle timed on this host on whole GQA groups of the workload
  vector_path   the short-query path (Lq = 8, D = 128, Lkv = 8192) in HBM GB/s: forward,
                backward end to end (both stages), and the backward's streaming kernel
                (stage 0) alone
  graph         device times from HIP graph replays (no host launch gaps): a whole step
                from a graph of R steps, and each stage from a graph of R launches of it
                (--graph-reps R, 0 turns it off)
Options: --sweep prints one line per workload instead.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from scaled_dot_product_online_amd import inputs as inp  # noqa: E402
from scaled_dot_product_online_amd.workloads import BY_NAME, HEADLINE, MASKED, WORKLOADS, flops, mask_and_sinks  # noqa: E402

METRIC = "SDPA TFLOP/s fwd & fwd+bwd (bf16/fp16, causal) and % of MFMA peak, 1 GPU"
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}  # AMD's published MI355X figures: dense MFMA (16-bit), fp32 vector FMA (the fp32 path)
PEAK_HBM_GBS = 8000.0
VECTOR_WORKLOAD = "vec_bf16_lq8_d128"
# GEMMs each kernel executes, in units of the forward's two (S and P.V):
KERNEL_GEMMS = {"fwd": 2, "bwd_stage0": 3, "bwd_stage1": 4}  # dQ kernel: S, dP, dQ; dK/dV kernel: S, dP, dV, dK


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(BY_NAME))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-vector", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="one JSON line per workload")
    ap.add_argument("--graph-reps", type=int, default=10, metavar="R",
                    help="also time each stage as R launches replayed from a HIP graph (0: off)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run 3 plain device copies of MIB MiB (reference for HBM traffic counters)")
    return ap.parse_args()


class Runner:
    """Device buffers for one workload and a step() that runs fwd + bwd stage 0 + stage 1."""

    def __init__(self, name, device, rotate=False):
        import torch

        import scaled_dot_product_online_amd as sd

        self.sd, self.torch = sd, torch
        self.name = name
        _, B, Hq, Hkv, Lq, Lkv, D, dt, causal = BY_NAME[name]
        self.case = inp.make_case(B, Hq, Hkv, Lq, Lkv, D, dt, is_causal=causal, seed=0)
        c = self.case
        self.q, self.k, self.v, self.do = (inp.to_torch(getattr(c, n), dt, device) for n in ("q", "k", "v", "do"))
        # rotate: two copies of K and V used in turn, so that no call finds the other's
        # operands in the 256 MB memory-side cache (short-query shapes whose K and V are
        # about that size).
        self.kv = [(self.k, self.v)] + ([(self.k.clone(), self.v.clone())] if rotate else [])
        self.turn = 0
        mask, sinks = mask_and_sinks(name)
        self.mask = None if mask is None else torch.from_numpy(mask[1]).to(device)
        self.sinks = None if sinks is None else torch.from_numpy(sinks).to(device)
        self.dsinks = None if sinks is None else torch.empty(Hq, dtype=torch.float32, device=device)
        tdt = self.q.dtype
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=device)
        self.dq = torch.empty_like(self.q)
        self.dk, self.dv = torch.empty_like(self.k), torch.empty_like(self.v)
        code = {"f32": sd.F32, "f16": sd.F16, "bf16": sd.BF16}[dt]
        self.path = sd.PATH_NAMES[sd.select_path(Hq, Hkv, Lq, Lkv, D, causal, code)]
        wf = sd.workspace_bytes(0, B, Hq, Hkv, Lq, Lkv, D, causal, code)
        wb = sd.workspace_bytes(1, B, Hq, Hkv, Lq, Lkv, D, causal, code)
        self.ws_f = torch.empty(max(wf, 256), dtype=torch.uint8, device=device)
        self.ws_b = torch.empty(max(wb, 256), dtype=torch.uint8, device=device)
        # A stream of its own (default priority), so that the stages can also be captured
        # in HIP graphs (capture needs a stream other than the null stream).
        self.stream = torch.cuda.Stream(device)
        self.tdt = tdt
        self.fwd_flops = flops(B, Hq, Lq, Lkv, D, causal)
        self.bwd_flops = flops(B, Hq, Lq, Lkv, D, causal, backward=True)
        e = 2 if dt != "f32" else 4
        qb, kb = B * Hq * Lq * D * e, B * Hkv * Lkv * D * e
        lse_b = B * Hq * Lq * 4
        # Algorithmic HBM bytes: each operand read once, each result written once.
        self.fwd_bytes = qb + 2 * kb + qb + lse_b
        self.bwd_bytes = (qb + 2 * kb + qb + qb + lse_b) + (qb + 2 * kb)

    def fwd(self):
        self.turn = (self.turn + 1) % len(self.kv)
        k, v = self.kv[self.turn]
        self.sd.sdpa_fwd(self.q, k, v, scale=self.case.scale, is_causal=self.case.is_causal, out=self.o,
                         lse=self.lse, workspace=self.ws_f, stream=self.stream, attn_mask=self.mask,
                         sinks=self.sinks)

    def bwd(self, stage):
        k, v = self.kv[self.turn]
        self.sd.sdpa_bwd(self.q, k, v, self.o, self.lse, self.do, scale=self.case.scale,
                         is_causal=self.case.is_causal, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws_b,
                         stream=self.stream, stage=stage, attn_mask=self.mask, sinks=self.sinks, dsinks=self.dsinks)

    def timed(self, steps, warmup):
        """Wall time of `steps` steps (synchronised on both sides) and per-kernel event times."""
        torch = self.torch
        for _ in range(warmup):
            self.fwd()
            self.bwd(0)
            self.bwd(1)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record(self.stream)
            self.fwd()
            ev[i][1].record(self.stream)
            self.bwd(0)
            ev[i][2].record(self.stream)
            self.bwd(1)
            ev[i][3].record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = {"fwd": 0.0, "bwd_stage0": 0.0, "bwd_stage1": 0.0}
        for e in ev:
            ms["fwd"] += e[0].elapsed_time(e[1]) / steps
            ms["bwd_stage0"] += e[1].elapsed_time(e[2]) / steps
            ms["bwd_stage1"] += e[2].elapsed_time(e[3]) / steps
        return wall, ms

    def graph_times(self, reps, rounds):
        """Device times without host launch gaps, from HIP graphs replayed between two events on
        the launch stream (median over `rounds` replays): `step` is one whole step (forward,
        dQ stage, dK/dV stage) from a graph of `reps` steps; each stage's entry is one launch
        from a graph of `reps` launches of that stage alone (so it runs after itself, with
        its own operands still in the caches). Where a stage's device time is shorter than a
        host call through the binding, the eager times above include the host's gaps."""
        torch = self.torch
        stages = (("fwd", self.fwd), ("bwd_stage0", lambda: self.bwd(0)), ("bwd_stage1", lambda: self.bwd(1)))

        def whole_step():
            for _, fn in stages:
                fn()

        graphs = {}
        for key, fn in stages + (("step", whole_step),):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream):
                for _ in range(reps):
                    fn()
            graphs[key] = g
        torch.cuda.synchronize()
        times = {key: [] for key in graphs}
        with torch.cuda.stream(self.stream):
            for _ in range(rounds):
                for key, g in graphs.items():
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(self.stream)
                    g.replay()
                    e1.record(self.stream)
                    torch.cuda.synchronize()
                    times[key].append(e0.elapsed_time(e1) / reps)
        del graphs
        return {key: float(np.median(v)) for key, v in times.items()}


def blas_info():
    """(threads, library and version) of the BLAS that NumPy calls, after loading it."""
    import numpy as np

    np.ones((64, 64)) @ np.ones((64, 64))
    try:
        import threadpoolctl

        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return int(info[0].get("num_threads", 1)), f"{info[0].get('internal_api')} {info[0].get('version')}"
    except Exception:  # pragma: no cover
        pass
    return len(os.sched_getaffinity(0)), "unknown"


def cpu_baseline(case, budget_s=10.0, mask=None, sinks=None):
    """fp64 oracle on whole GQA groups of the same inputs, timed on host cores.

    Each group (b, hk) runs the forward alone, then forward + backward (the backward
    recomputes the forward), in order until ~budget_s seconds of CPU work (at least one
    group). Reports fwd+bwd TFLOP/s, and the mean seconds per group of both."""
    from oracle import sdpa_reference as ref

    threads, blas = blas_info()
    G = case.Hq // case.Hkv
    groups = [(b, hk) for b in range(case.B) for hk in range(case.Hkv)]
    om = None
    if mask is not None:
        om = np.asarray(mask[1], dtype=bool) if mask[0] == "bool" else inp.as_float64(mask[1], case.dtype)
    done, t_fwd, t_all = 0, 0.0, 0.0
    for b, hk in groups:
        hs = slice(hk * G, (hk + 1) * G)
        q = case.f64("q")[b:b + 1, hs]
        k = case.f64("k")[b:b + 1, hk:hk + 1]
        v = case.f64("v")[b:b + 1, hk:hk + 1]
        do = case.f64("do")[b:b + 1, hs]
        m = None
        if om is not None:
            m4 = om.reshape((1,) * (4 - om.ndim) + om.shape)
            m = m4[(slice(b, b + 1) if m4.shape[0] > 1 else slice(0, 1)), (hs if m4.shape[1] > 1 else slice(0, 1))]
        sk = None if sinks is None else np.asarray(sinks, dtype=np.float64)[hs]
        t0 = time.perf_counter()
        ref.attention_forward(q, k, v, case.scale, case.is_causal, mask=m, sinks=sk)
        t1 = time.perf_counter()
        ref.group_backward(q, k, v, do, case.scale, case.is_causal, 0, 0, mask=m, sinks=sk)
        t2 = time.perf_counter()
        t_fwd += t1 - t0
        t_all += t2 - t1
        done += 1
        if t_fwd + t_all >= budget_s:
            break
    f = done * (flops(1, G, case.Lq, case.Lkv, case.D, case.is_causal)
                + flops(1, G, case.Lq, case.Lkv, case.D, case.is_causal, backward=True))
    return {"value": f / t_all / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "fwd_s_per_group": t_fwd / done, "fwdbwd_s_per_group": t_all / done, "groups": done,
            "groups_total": len(groups), "blas": blas,
            "sample": f"fp64 numpy oracle of {done} of {len(groups)} GQA groups ({G} query heads each, Lq={case.Lq}, "
                      f"Lkv={case.Lkv}, D={case.D}, causal={case.is_causal}) of the same workload: forward alone, then "
                      f"forward+backward ({t_all:.1f} s); value = fwd+bwd FLOPs counted as for the GPU / fwd+bwd time"}


def measure(runner, steps, warmup, graph_reps=0):
    wall, ms = runner.timed(steps, warmup)
    total = runner.fwd_flops + runner.bwd_flops
    value = total * steps / wall / 1e12
    dt = runner.case.dtype
    out = {"value": value, "ms_per_step": wall / steps * 1e3, "kernel_ms": ms,
           "fwd_tflops": runner.fwd_flops / (ms["fwd"] * 1e-3) / 1e12,
           "bwd_tflops": runner.bwd_flops / ((ms["bwd_stage0"] + ms["bwd_stage1"]) * 1e-3) / 1e12}
    out["fwd_frac_of_peak"] = out["fwd_tflops"] / PEAK_TFLOPS[dt]
    out["fwdbwd_frac_of_peak"] = value / PEAK_TFLOPS[dt]
    if graph_reps > 0:
        try:
            g = runner.graph_times(graph_reps, max(3, min(steps, 10)))
        except Exception as e:  # the contract's fields above stand without it
            out["graph"] = {"error": f"{type(e).__name__}: {e}"}
        else:
            step = g.pop("step")
            out["graph"] = {"reps": graph_reps, "step_ms": step, "fwdbwd_tflops": total / (step * 1e-3) / 1e12,
                            "kernel_ms": g, "fwd_tflops": runner.fwd_flops / (g["fwd"] * 1e-3) / 1e12}
    dom = max(ms, key=ms.get)
    if runner.path == "vector":
        algo = {"fwd": runner.fwd_bytes, "bwd_stage0": runner.bwd_bytes, "bwd_stage1": 0}[dom]
        ach = algo / (ms[dom] * 1e-3) / 1e9
        out["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": ach / PEAK_HBM_GBS, "traffic": measured_traffic(runner, dom)}
    else:
        # The tiled kernels run on the matrix cores; the fp32 path on the vector ALUs (fp32 FMA
        # peak: 256 CUs x 256 flop/clock x 2.4 GHz = 157.3 TFLOP/s).
        algo = runner.fwd_flops * KERNEL_GEMMS[dom] / 2
        ach = algo / (ms[dom] * 1e-3) / 1e12
        out["roofline"] = {"kernel": dom, "bound": "alu" if runner.path == "fp32" else "mfma", "achieved": ach,
                           "peak": PEAK_TFLOPS[dt],
                           "unit": "TFLOP/s", "frac": ach / PEAK_TFLOPS[dt],
                           "traffic": measured_traffic(runner, dom)}
    return out


def kernel_symbol(runner, label):
    """Short kernel name (as rocprofv3 summaries print it) behind a bench label."""
    c = runner.case
    t = {"bf16": "bf16_t", "f16": "f16_t", "f32": "float"}[c.dtype]
    causal = "true" if c.is_causal else "false"
    masked = "true" if runner.mask is not None else "false"
    if runner.path == "tiled":
        base = {"fwd": "fwd_tiled_kernel", "bwd_stage0": "dq_kernel", "bwd_stage1": "dkv_kernel"}[label]
        return f"{base}<{t}, {c.D}, {causal}, {masked}, {t}>"
    if runner.path == "vector":
        if label == "bwd_stage1":
            return f"vec_dq_reduce_kernel<{c.D}, {t}>"
        base = {"fwd": "vec_fwd_kernel", "bwd_stage0": "vec_bwd_kernel"}[label]
        return f"{base}<{t}, {c.D}, {causal}, {masked}, {t}>"
    return None


def measured_traffic(runner, label):
    """HBM bytes per launch from committed counter summaries, if taken on the current kernel sources."""
    import glob

    from scaled_dot_product_online_amd.rocprof_summary import sources_sha256

    sym = kernel_symbol(runner, label)
    if sym is None:
        return None
    sha = sources_sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.traffic.json"))):
        with open(path) as f:
            t = json.load(f)
        if t.get("source_sha256") != sha:
            continue
        # The dK/dV kernel has a split and an unsplit instantiation (one more template
        # argument); a profiled run launches one of them.
        names = [n for n in t.get("kernels", {}) if n == sym or n.startswith(sym[:-1] + ", ")]
        if len(names) == 1:
            k = t["kernels"][names[0]]
            return k["read_bytes"] + k["write_bytes"]
    return None


def vector_line(device, steps, warmup, graph_reps=0):
    r = Runner(VECTOR_WORKLOAD, device)
    _, ms = r.timed(steps, warmup)
    fwd_gbs = r.fwd_bytes / (ms["fwd"] * 1e-3) / 1e9
    bwd_gbs = r.bwd_bytes / ((ms["bwd_stage0"] + ms["bwd_stage1"]) * 1e-3) / 1e9
    main_gbs = r.bwd_bytes / (ms["bwd_stage0"] * 1e-3) / 1e9  # the streaming kernel alone (stage 0)
    out = {"workload": VECTOR_WORKLOAD, "kernel_ms": ms, "fwd_GBps": fwd_gbs, "bwd_GBps": bwd_gbs,
           "fwd_frac_of_hbm_peak": fwd_gbs / PEAK_HBM_GBS, "bwd_frac_of_hbm_peak": bwd_gbs / PEAK_HBM_GBS,
           "bwd_stage0_frac_of_hbm_peak": main_gbs / PEAK_HBM_GBS}
    if graph_reps > 0:
        try:
            g = r.graph_times(graph_reps, max(3, min(steps, 10)))
        except Exception as e:
            out["graph"] = {"error": f"{type(e).__name__}: {e}"}
            return out
        step = g.pop("step")
        out["graph"] = {"reps": graph_reps, "step_ms": step, "kernel_ms": g,
                        "fwd_frac_of_hbm_peak": r.fwd_bytes / (g["fwd"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "bwd_frac_of_hbm_peak": r.bwd_bytes / ((g["bwd_stage0"] + g["bwd_stage1"]) * 1e-3) / 1e9
                        / PEAK_HBM_GBS}
    return out


def config_of(name):
    _, B, Hq, Hkv, Lq, Lkv, D, dt, causal = BY_NAME[name]
    cfg = {"workload": name, "B": B, "Hq": Hq, "Hkv": Hkv, "Lq": Lq, "Lkv": Lkv, "D": D, "causal": causal,
           "scale": "1/sqrt(D)", "inputs": "iid N(0,1), numpy default_rng(0)"}
    if name in MASKED:
        cfg["mask"] = MASKED[name]["mask"]
        cfg["sinks"] = MASKED[name]["sinks"]
    return cfg


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (the (b, kv-head) groups are "
              "independent, so a run would shard them across GPUs with no communication). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    device = "cuda:0"
    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy << 20, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    names = [w[0] for w in WORKLOADS] if args.sweep else [args.workload]
    for name in names:
        r = Runner(name, device, rotate=args.sweep and BY_NAME[name][4] <= 8)
        m = measure(r, args.steps, args.warmup, args.graph_reps)
        line = {"metric": METRIC, "value": m["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": m["ms_per_step"], "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": r.case.dtype, "data": "synthetic",
                "config": config_of(name), "path": r.path, "fwd_tflops": m["fwd_tflops"],
                "bwd_tflops": m["bwd_tflops"], "fwd_frac_of_peak": m["fwd_frac_of_peak"],
                "fwdbwd_frac_of_peak": m["fwdbwd_frac_of_peak"], "kernel_ms": m["kernel_ms"],
                "roofline": m["roofline"]}
        if "graph" in m:
            line["graph"] = m["graph"]
        if not args.sweep and not args.no_vector:
            line["vector_path"] = vector_line(device, args.steps, args.warmup, args.graph_reps)
        if args.sweep:
            line["kv_copies"] = len(r.kv)
        mask, sinks = mask_and_sinks(name)
        line["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(
            r.case, budget_s=2.0 if args.sweep else 10.0, mask=mask, sinks=sinks)
        print(json.dumps(line), flush=True)
        del r
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
