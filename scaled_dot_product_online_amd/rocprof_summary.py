"""Summarise rocprofv3 CSV output into the short text files kept under profiles/.

    python -m scaled_dot_product_online_amd.rocprof_summary --name NAME --command "CMD" \
        [--trace DIR] [--fetch DIR --write DIR --calib-bytes N] [--sq DIR [DIR ...]]

--trace    directory of a `rocprofv3 --kernel-trace --stats --output-format csv` run
--fetch    directory of a `rocprofv3 --pmc FETCH_SIZE` run of the same program
--write    directory of a `rocprofv3 --pmc WRITE_SIZE` run of the same program
--calib-bytes  size of the plain device copy the program ran (bench.py --calibrate-copy):
           the counters' KiB for that copy, against its true bytes read and written,
           give the factors that turn FETCH_SIZE / WRITE_SIZE into bytes.
--bench-log    stdout of the traced bench.py run: its own HIP-event times per stage (timed
           steps only; the trace's averages also hold the warm-up calls) are listed beside
           the durations.
--sq       directories of `rocprofv3 --pmc` runs of the same program with SQ (shader
           sequencer) and GRBM counters, at most 8 SQ counters per run; their per-dispatch
           means are merged by kernel name into one table of instruction mix, matrix-core
           occupancy, waits and the shader clock (counters.json keeps the raw means).

Writes profiles/NAME.md (per-kernel durations, and per-dispatch HBM traffic and
instruction counters when those runs are given) and, for the traffic and the counters,
profiles/NAME.traffic.json and profiles/NAME.counters.json keyed by the sha256 of the HIP
sources, so that bench.py reports `traffic` only for the kernel build the counters were
taken on.

Counter arithmetic (MI355X: 256 CUs of 4 SIMDs in 8 XCDs, each XCD with its own GRBM):
  clock           GRBM_GUI_ACTIVE / 8 XCDs / kernel duration (dispatch timestamps of the
                  same run)
  matrix busy     SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8): the share
                  of SIMD cycles in which the matrix core works (the busy count equals the
                  instructions' issue cycles: 32 per 32x32x16, 16 per 16x16x32 16-bit MFMA)
  per MFMA        SQ_INSTS_{VALU - MFMA, LDS, SALU} / SQ_INSTS_MFMA (SQ_INSTS_VALU counts
                  the MFMA instructions too)
  waits           SQ_WAIT_INST_LDS, SQ_WAIT_ANY, SQ_WAIT_INST_ANY as shares of SQ_WAVE_CYCLES
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)


def sources_sha256():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()


def short(name):
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0].replace("sdpa::", "")


def read_csv(d, suffix):
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def counter_means(d):
    agg = collections.defaultdict(list)
    for r in read_csv(d, "counter_collection.csv"):
        agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def sq_means(dirs):
    """{kernel: {counter: mean per dispatch}} over several --pmc runs, with each run's mean
    dispatch duration in ns as duration_ns@<run> (for the clock of that run's GRBM counts)."""
    out = collections.defaultdict(dict)
    for run, d in enumerate(dirs):
        vals = collections.defaultdict(lambda: collections.defaultdict(list))
        durs = collections.defaultdict(dict)
        for r in read_csv(d, "counter_collection.csv"):
            k = short(r["Kernel_Name"])
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            durs[k][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        for k, cs in vals.items():
            for c, v in cs.items():
                out[k][c if c not in out[k] else f"{c}@{run}"] = sum(v) / len(v)
                if c == "GRBM_GUI_ACTIVE":
                    out[k][f"duration_ns@{run}"] = sum(durs[k].values()) / len(durs[k])
                    out[k][f"GRBM_GUI_ACTIVE@{run}"] = sum(v) / len(v)
    return out


def sq_derived(c):
    """Derived per-kernel figures from the merged SQ / GRBM means (None where a counter is missing)."""
    g = lambda n: c.get(n)  # noqa: E731
    clocks = [c[k] / 8.0 / c["duration_ns@" + k.split("@")[1]] for k in c
              if k.startswith("GRBM_GUI_ACTIVE@") and c.get("duration_ns@" + k.split("@")[1])]
    cycles = g("GRBM_GUI_ACTIVE") / 8.0 if g("GRBM_GUI_ACTIVE") else None
    mfma = g("SQ_INSTS_MFMA")
    d = {"clock_GHz": sum(clocks) / len(clocks) if clocks else None}
    d["mfma_busy"] = (g("SQ_VALU_MFMA_BUSY_CYCLES") / (1024.0 * cycles)
                      if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None and cycles else None)
    if mfma:
        d["valu_per_mfma"] = (g("SQ_INSTS_VALU") - mfma) / mfma if g("SQ_INSTS_VALU") is not None else None
        d["lds_per_mfma"] = g("SQ_INSTS_LDS") / mfma if g("SQ_INSTS_LDS") is not None else None
        d["salu_per_mfma"] = g("SQ_INSTS_SALU") / mfma if g("SQ_INSTS_SALU") is not None else None
    wc = g("SQ_WAVE_CYCLES")
    for n, key in (("SQ_WAIT_INST_LDS", "wait_lds"), ("SQ_WAIT_ANY", "wait_any"), ("SQ_WAIT_INST_ANY", "wait_issue")):
        d[key] = g(n) / wc if wc and g(n) is not None else None
    d["lds_bank_conflict_cycles"] = g("SQ_LDS_BANK_CONFLICT")
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--name", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--trace")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--calib-bytes", type=int, default=0)
    ap.add_argument("--bench-log")
    ap.add_argument("--sq", nargs="+")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args()

    stats = read_csv(a.trace, "kernel_stats.csv") if a.trace else []
    lines = [f"# {a.name}", "", "Command (run from the repository root on one MI355X):", "", "```", a.command, "```", ""]
    if stats:
        lines += ["## Kernel durations (rocprofv3 --kernel-trace --stats)", "",
                  "| kernel | calls | average us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    if a.bench_log:
        with open(a.bench_log) as f:
            runs = [json.loads(l) for l in f if l.startswith("{")]
        lines += ["", "HIP-event times that bench.py measured in the same traced run (timed steps only; the "
                      "averages above also hold the warm-up calls):", "",
                  "| workload | stage | ms per call |", "|---|---|---|"]
        for r in runs:
            for stage, ms in r["kernel_ms"].items():
                lines.append(f"| {r['config']['workload']} | {stage} | {ms:.4f} |")
            vp = r.get("vector_path")
            if vp:
                for stage, ms in vp["kernel_ms"].items():
                    lines.append(f"| {vp['workload']} | {stage} | {ms:.4f} |")
    traffic = None
    if a.fetch and a.write:
        fetch, write = counter_means(a.fetch), counter_means(a.write)
        copy = [k for k in fetch if "copyBuffer" in k]
        if not copy or not a.calib_bytes:
            raise SystemExit("counter runs need the calibration copy (bench.py --calibrate-copy MIB)")
        kib = a.calib_bytes / 1024.0
        f_scale, w_scale = kib / fetch[copy[0]], kib / write[copy[0]]
        lines += ["", "## HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
                  f"Calibration: a plain copy of {a.calib_bytes} bytes reads {fetch[copy[0]]:.0f} KiB of FETCH_SIZE "
                  f"and {write[copy[0]]:.0f} KiB of WRITE_SIZE; factors {f_scale:.4f} (fetch) and {w_scale:.4f} "
                  f"(write) turn the counters into bytes.", "",
                  "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | bytes read | bytes written |", "|---|---|---|---|---|"]
        traffic = {"source_sha256": sources_sha256(), "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
        for k in fetch:
            if "copyBuffer" in k:
                continue
            rd, wr = fetch[k] * f_scale * 1024, write.get(k, 0.0) * w_scale * 1024
            lines.append(f"| `{short(k)}` | {fetch[k]:.0f} | {write.get(k, 0.0):.0f} | {rd:.4g} | {wr:.4g} |")
            traffic["kernels"][short(k)] = {"read_bytes": rd, "write_bytes": wr}
    counters = None
    if a.sq:
        merged = sq_means(a.sq)
        fmt = lambda x, f: "—" if x is None else format(x, f)  # noqa: E731
        lines += ["", "## Instruction counters per dispatch (rocprofv3 --pmc, SQ and GRBM blocks)", "",
                  "| kernel | clock GHz | matrix busy | VALU / MFMA | LDS / MFMA | SALU / MFMA | waiting on LDS | "
                  "waiting (s_waitcnt) | waiting to issue | LDS bank-conflict cycles |",
                  "|---|---|---|---|---|---|---|---|---|---|"]
        counters = {"source_sha256": sources_sha256(), "kernels": {}}
        for k in sorted(merged):
            dv = sq_derived(merged[k])
            if not merged[k].get("SQ_INSTS_MFMA") and not merged[k].get("SQ_INSTS_VALU"):
                continue
            lines.append(f"| `{k}` | {fmt(dv['clock_GHz'], '.2f')} | {fmt(dv['mfma_busy'], '.1%')} | "
                         f"{fmt(dv.get('valu_per_mfma'), '.2f')} | {fmt(dv.get('lds_per_mfma'), '.2f')} | "
                         f"{fmt(dv.get('salu_per_mfma'), '.2f')} | {fmt(dv['wait_lds'], '.1%')} | "
                         f"{fmt(dv['wait_any'], '.1%')} | {fmt(dv['wait_issue'], '.1%')} | "
                         f"{fmt(dv['lds_bank_conflict_cycles'], '.3g')} |")
            counters["kernels"][k] = {"means": merged[k], "derived": dv}
    os.makedirs(a.out, exist_ok=True)
    with open(os.path.join(a.out, f"{a.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if traffic is not None:
        with open(os.path.join(a.out, f"{a.name}.traffic.json"), "w") as f:
            json.dump(traffic, f, indent=1)
    if counters is not None:
        with open(os.path.join(a.out, f"{a.name}.counters.json"), "w") as f:
            json.dump(counters, f, indent=1)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
