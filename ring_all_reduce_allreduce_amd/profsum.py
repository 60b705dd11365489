"""Summarises rocprofv3 CSV output of a bench run into a short text report.

Inputs: the kernel_stats.csv of a `--kernel-trace --stats` run, and the
counter_collection.csv files of separate `--pmc FETCH_SIZE` and
`--pmc WRITE_SIZE` runs, for the benchmark and for the copy-calibration run
(`bench.py --copy-calibration`, a copy kernel that reads and writes 1 GiB per
launch). The counters report KiB per dispatch; each is scaled by
known bytes / counted bytes of the copy kernel, so that counter quirks of the
part (e.g. a fetch counter that counts half the bytes) cancel.

Writes a markdown report and a `key: value` traffic record that bench.py reads
to fill roofline.traffic (only while the kernel source hash still matches).

  python -m ring_all_reduce_allreduce_amd.profsum --name ar8x64 --kernel ring_bulk_kernel \\
      --stats S.csv --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv \\
      --hash H --algorithmic-bytes B --report profiles/X.md --traffic profiles/traffic_ar8x64.txt \\
      --command "..." [--command "..."]
"""
from __future__ import annotations

import argparse
import csv
import statistics

COPY_BYTES = 1 << 30


def per_dispatch(path: str, kernel_substr: str, counter: str) -> list[float]:
    vals = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals.append(float(r["Counter_Value"]) * 1024.0)
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_substr} in {path}")
    return vals


def kernel_stats(path: str) -> list[dict]:
    with open(path) as f:
        return list(csv.DictReader(f))


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--name", required=True)
    ap.add_argument("--kernel", required=True, help="substring of the kernel name to summarise")
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--hash", required=True)
    ap.add_argument("--algorithmic-bytes", type=int, required=True)
    ap.add_argument("--report", required=True)
    ap.add_argument("--traffic", required=True)
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--title", default="")
    a = ap.parse_args()

    fetch = per_dispatch(a.fetch, a.kernel, "FETCH_SIZE")
    write = per_dispatch(a.write, a.kernel, "WRITE_SIZE")
    cfetch = per_dispatch(a.copy_fetch, "copy_kernel", "FETCH_SIZE")
    cwrite = per_dispatch(a.copy_write, "copy_kernel", "WRITE_SIZE")
    f_scale = COPY_BYTES / statistics.median(cfetch)
    w_scale = COPY_BYTES / statistics.median(cwrite)
    fetch_b = statistics.median(fetch) * f_scale
    write_b = statistics.median(write) * w_scale
    traffic = fetch_b + write_b

    rows = kernel_stats(a.stats)
    lines = [f"# {a.title or a.name}", ""]
    lines.append("Commands (run from /tmp with TMPDIR=/tmp; R = repository root):")
    lines.append("")
    for c in a.command:
        lines.append(f"    {c}")
    lines.append("")
    lines.append("## Kernel trace statistics")
    lines.append("")
    lines.append("| kernel | calls | avg us | min us | max us | share |")
    lines.append("|---|---|---|---|---|---|")
    for r in rows:
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    target = [r for r in rows if a.kernel in r["Name"]]
    avg_ns = float(target[0]["AverageNs"]) if target else float("nan")
    lines.append("")
    lines.append("## HBM-side bytes per launch (L2 to fabric)")
    lines.append("")
    lines.append(f"- copy calibration: FETCH_SIZE reads {statistics.median(cfetch) / 2**20:.1f} MiB and "
                 f"WRITE_SIZE {statistics.median(cwrite) / 2**20:.1f} MiB for a copy that reads and writes "
                 f"1024 MiB: scale factors fetch x{f_scale:.4f}, write x{w_scale:.4f}")
    lines.append(f"- `{a.kernel}`: FETCH_SIZE {statistics.median(fetch) / 2**20:.1f} MiB raw -> "
                 f"{fetch_b / 2**20:.1f} MiB; WRITE_SIZE {statistics.median(write) / 2**20:.1f} MiB raw -> "
                 f"{write_b / 2**20:.1f} MiB ({len(fetch)} / {len(write)} dispatches, medians)")
    lines.append(f"- traffic {traffic / 1e9:.4f} GB per launch vs algorithmic {a.algorithmic_bytes / 1e9:.4f} GB "
                 f"(ratio {traffic / a.algorithmic_bytes:.3f})")
    lines.append(f"- average launch {avg_ns / 1e3:.1f} us -> algorithmic {a.algorithmic_bytes / avg_ns:.0f} GB/s, "
                 f"counted {traffic / avg_ns:.0f} GB/s")
    lines.append(f"- kernel source hash `{a.hash}`")
    lines.append("")
    with open(a.report, "w") as f:
        f.write("\n".join(lines))
    with open(a.traffic, "w") as f:
        f.write(f"workload: {a.name}\nkernel: {a.kernel}\nkernel_source_hash: {a.hash}\n"
                f"bytes_per_launch: {int(round(traffic))}\nfetch_bytes: {int(round(fetch_b))}\n"
                f"write_bytes: {int(round(write_b))}\nfetch_scale: {f_scale:.6f}\nwrite_scale: {w_scale:.6f}\n"
                f"launch_avg_ns: {avg_ns:.0f}\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
