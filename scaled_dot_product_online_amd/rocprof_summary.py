"""Summarise rocprofv3 CSV output into the short text files kept under profiles/.

    python -m scaled_dot_product_online_amd.rocprof_summary --name NAME --command "CMD" \
        --trace DIR [--fetch DIR --write DIR --calib-bytes N]

--trace    directory of a `rocprofv3 --kernel-trace --stats --output-format csv` run
--fetch    directory of a `rocprofv3 --pmc FETCH_SIZE` run of the same program
--write    directory of a `rocprofv3 --pmc WRITE_SIZE` run of the same program
--calib-bytes  size of the plain device copy the program ran (bench.py --calibrate-copy):
           the counters' KiB for that copy, against its true bytes read and written,
           give the factors that turn FETCH_SIZE / WRITE_SIZE into bytes.
--bench-log    stdout of the traced bench.py run: its own HIP-event times per stage (timed
           steps only; the trace's averages also hold the warm-up calls) are listed beside
           the durations.

Writes profiles/NAME.md (per-kernel durations, and per-dispatch HBM traffic when
counter runs are given) and, for the traffic, profiles/NAME.traffic.json keyed by
the sha256 of the HIP sources, so that bench.py reports `traffic` only for the
kernel build the counters were taken on.
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--name", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--calib-bytes", type=int, default=0)
    ap.add_argument("--bench-log")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args()

    stats = read_csv(a.trace, "kernel_stats.csv")
    lines = [f"# {a.name}", "", "Command (run from the repository root on one MI355X):", "", "```", a.command, "```", "",
             "## Kernel durations (rocprofv3 --kernel-trace --stats)", "",
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
    os.makedirs(a.out, exist_ok=True)
    with open(os.path.join(a.out, f"{a.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if traffic is not None:
        with open(os.path.join(a.out, f"{a.name}.traffic.json"), "w") as f:
            json.dump(traffic, f, indent=1)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
