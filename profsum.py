"""Summarises rocprofv3 CSV output of a bench run into a short text report.

Inputs: the kernel_stats.csv of a `--kernel-trace --stats` run, and the
counter_collection.csv files of separate `--pmc FETCH_SIZE` and
`--pmc WRITE_SIZE` runs (optionally also one `--pmc
TCC_EA0_RDREQ_DRAM_32B_sum TCC_EA0_WRREQ_WRITE_DRAM_32B_sum` run), for the
benchmark and for the copy-calibration run (`bench.py --copy-calibration`, a
copy kernel that reads and writes 1 GiB per launch). FETCH_SIZE and
WRITE_SIZE report KiB per dispatch, the DRAM-request counters 32-byte units;
each is scaled by known bytes / counted bytes of the copy kernel, so that
counter quirks of the part (e.g. a fetch counter that counts half the bytes)
cancel. All of them count requests that leave the L2 for the memory side of
the fabric: the 256 MB Infinity Cache sits there, in front of HBM, and its
hits are counted the same as HBM accesses.

Writes a markdown report (with this summariser's own command line) and a
`key: value` traffic record that bench.py reads to fill roofline.traffic
(only while the kernel source hash still matches).

  python profsum.py --name ar8x64 --kernel ring_bulk_kernel \\
      --stats S.csv --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv \\
      [--dram D.csv --copy-dram CD.csv] \\
      --hash H --algorithmic-bytes B --report profiles/X.md --traffic profiles/traffic_ar8x64.txt \\
      --command "..." [--command "..."]
"""
from __future__ import annotations

import argparse
import csv
import shlex
import statistics
import sys

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


def trace_report(a) -> None:
    """The kernel trace statistics of one run (no counters), with the
    average of the kernel named by --kernel."""
    rows = kernel_stats(a.stats)
    argv = [x.replace(a.out_dir, "OUT") if a.out_dir else x for x in sys.argv[1:]]
    lines = [f"# {a.title or a.name}", "", "Commands (run from /tmp with TMPDIR=/tmp; R = repository root):", ""]
    lines += [f"    {c}" for c in a.command]
    lines += ["", "Summarised with (OUT = the directory of the run above):", "",
              "    python3 profsum.py " + " ".join(shlex.quote(x) for x in argv), "",
              "## Kernel trace statistics", "", "| kernel | calls | avg us | min us | max us | share |",
              "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    target = [r for r in rows if a.kernel in r["Name"]]
    if target:
        lines += ["", f"- `{a.kernel}`: {target[0]['Calls']} launches, average "
                      f"{float(target[0]['AverageNs']) / 1e3:.1f} us"]
    lines.append("")
    with open(a.report, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def markers_report(a) -> None:
    """The kernel trace statistics and the roctx ranges (count, mean and
    maximum host duration per name) of one run."""
    rows = kernel_stats(a.stats)
    ranges: dict[str, list[float]] = {}
    with open(a.markers) as f:
        for r in csv.DictReader(f):
            ranges.setdefault(r["Function"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    argv = [x.replace(a.out_dir, "OUT") if a.out_dir else x for x in sys.argv[1:]]
    lines = [f"# {a.title or a.name}", "", "Commands (run from /tmp with TMPDIR=/tmp; R = repository root):", ""]
    lines += [f"    {c}" for c in a.command]
    lines += ["", "Summarised with (OUT = the directory of the run above):", "",
              "    python3 profsum.py " + " ".join(shlex.quote(x) for x in argv), "",
              "## roctx ranges (host time of each library call)", "",
              "| range | calls | mean us | max us |", "|---|---|---|---|"]
    for name, d in sorted(ranges.items()):
        lines.append(f"| `{name}` | {len(d)} | {statistics.mean(d):.1f} | {max(d):.1f} |")
    lines += ["", "## Kernel trace statistics", "", "| kernel | calls | avg us | min us | max us | share |",
              "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    lines.append("")
    with open(a.report, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--name", required=True)
    ap.add_argument("--kernel", required=True, help="substring of the kernel name to summarise")
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch", default="")
    ap.add_argument("--write", default="")
    ap.add_argument("--copy-fetch", default="")
    ap.add_argument("--copy-write", default="")
    ap.add_argument("--dram", default="", help="counter_collection.csv of the DRAM-request counter run")
    ap.add_argument("--copy-dram", default="", help="the same run of the copy calibration")
    ap.add_argument("--out-dir", default="", help="shown as OUT in the report's copy of this command line")
    ap.add_argument("--hash", default="")
    ap.add_argument("--algorithmic-bytes", type=int, default=0)
    ap.add_argument("--report", required=True)
    ap.add_argument("--traffic", default="")
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--title", default="")
    ap.add_argument("--markers", default="", help="marker_api_trace.csv of a --marker-trace run: report the "
                                                  "roctx ranges instead of the traffic")
    a = ap.parse_args()
    if a.markers:
        return markers_report(a)
    if not a.fetch:
        return trace_report(a)

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
    lines.append("Summarised with (OUT = the directory of the runs above):")
    lines.append("")
    argv = [x.replace(a.out_dir, "OUT") if a.out_dir else x for x in sys.argv[1:]]
    lines.append("    python3 profsum.py " + " ".join(shlex.quote(x) for x in argv))
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
    lines.append("## Bytes per launch between the L2 and the memory side (HBM and Infinity Cache together)")
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
    dram_b = None
    if a.dram and a.copy_dram:
        rd = per_dispatch(a.dram, a.kernel, "TCC_EA0_RDREQ_DRAM_32B_sum")
        wr = per_dispatch(a.dram, a.kernel, "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")
        crd = per_dispatch(a.copy_dram, "copy_kernel", "TCC_EA0_RDREQ_DRAM_32B_sum")
        cwr = per_dispatch(a.copy_dram, "copy_kernel", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")
        # per_dispatch scales by 1024 (KiB); these counters are 32-byte units
        unit = 32.0 / 1024.0
        rd_s, wr_s = COPY_BYTES / (statistics.median(crd) * unit), COPY_BYTES / (statistics.median(cwr) * unit)
        rd_b = statistics.median(rd) * unit * rd_s
        wr_b = statistics.median(wr) * unit * wr_s
        dram_b = rd_b + wr_b
        lines.append(f"- requests destined for DRAM (TCC_EA0_RDREQ_DRAM_32B_sum, TCC_EA0_WRREQ_WRITE_DRAM_32B_sum; "
                     f"copy scale x{rd_s:.4f} / x{wr_s:.4f}): read {rd_b / 2**20:.1f} MiB, write "
                     f"{wr_b / 2**20:.1f} MiB, {dram_b / 1e9:.4f} GB per launch. These classify requests by "
                     f"their target (device memory), before the Infinity Cache: they bound HBM bytes from above "
                     f"like FETCH_SIZE + WRITE_SIZE, and no counter here separates cache hits from HBM")
    lines.append(f"- kernel source hash `{a.hash}`")
    lines.append("")
    with open(a.report, "w") as f:
        f.write("\n".join(lines))
    with open(a.traffic, "w") as f:
        f.write(f"workload: {a.name}\nkernel: {a.kernel}\nkernel_source_hash: {a.hash}\n"
                f"bytes_per_launch: {int(round(traffic))}\nfetch_bytes: {int(round(fetch_b))}\n"
                f"write_bytes: {int(round(write_b))}\nfetch_scale: {f_scale:.6f}\nwrite_scale: {w_scale:.6f}\n"
                f"launch_avg_ns: {avg_ns:.0f}\n" + (f"dram_request_bytes: {int(round(dram_b))}\n" if dram_b else ""))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
