"""Summaries of rocprofv3 output for this library's kernels.

  python -m block_drafter_amd.profsum stats KERNEL_STATS_CSV [--top N]
      Markdown table of a ``--kernel-trace --stats --output-format csv`` run.

  python -m block_drafter_amd.profsum sequence KERNEL_TRACE_CSV --start REGEX [--nth N] [--until REGEX]
      The kernels of one call in launch order (start, duration, gap to the
      previous kernel's end, workgroups): from the N-th dispatch matching
      --start (negative N counts from the end) up to the next match, or to
      the first dispatch matching --until.

  python -m block_drafter_amd.profsum traffic --fetch CSV --write CSV
        --fetch-copy CSV --write-copy CSV --kernel REGEX --algorithmic BYTES
      [--min-fetch-kib KIB]
      HBM traffic per launch of the kernels whose name matches REGEX (and,
      with --min-fetch-kib, whose fetch reaches KIB), from two
      ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs (KiB per dispatch).
      Each counter is scaled by the factor that turns its reading on a plain
      device copy of known size into the copy's true bytes (the copy runs
      come from ``bench.py --copy-probe BYTES``).  The summary records a hash
      of the kernel sources, so a reader can tell when it has gone stale.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
# sources whose change invalidates a traffic figure of the streamed GEMM
# (the kernel, and the launcher that picks its configuration and operands)
GEMM_SOURCES = ["csrc/gemm_stream.hip", "csrc/dspine_device.hpp", "csrc/dspine_internal.hpp", "csrc/dspine_api.cpp"]


def source_hash(paths=GEMM_SOURCES) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(HERE, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = name.split("(")[0]
    return name.replace("void ", "").replace("dspine::", "")


def stats_table(path: str, top: int = 20) -> str:
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["| kernel | calls | avg µs | min µs | max µs | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows[:top]:
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out)


def sequence_table(path: str, start: str, nth: int = -1, until: str = "") -> str:
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    idx = [i for i, r in enumerate(rows) if re.search(start, r["Kernel_Name"])]
    if not idx:
        raise SystemExit("no dispatch matches --start")
    k = nth if nth >= 0 else len(idx) + nth
    i0 = idx[k]
    i1 = idx[k + 1] if k + 1 < len(idx) else len(rows)
    if until:
        for i in range(i0 + 1, len(rows)):
            if re.search(until, rows[i]["Kernel_Name"]):
                i1 = i + 1
                break
    t0 = int(rows[i0]["Start_Timestamp"])
    prev = t0
    total = 0.0
    out = ["| start µs | kernel | µs | gap µs | workgroups |", "|---:|---|---:|---:|---:|"]
    for r in rows[i0:i1]:
        st, en = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        wg = (int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])) // max(
            1, int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]))
        total += (en - st) / 1e3
        out.append(f"| {(st - t0) / 1e3:.1f} | `{short_name(r['Kernel_Name'])}` | {(en - st) / 1e3:.2f} | "
                   f"{(st - prev) / 1e3:.1f} | {wg} |")
        prev = en
    out.append(f"\n{i1 - i0} kernels, {total:.1f} µs of kernel time in a {(prev - t0) / 1e3:.1f} µs span")
    return "\n".join(out)


def _counter(path: str, regex: str):
    vals = []
    for r in csv.DictReader(open(path)):
        if re.search(regex, r["Kernel_Name"]):
            vals.append(float(r["Counter_Value"]))
    return vals


def copy_factor(path: str, copy_bytes: int) -> float:
    vals = _counter(path, r"copyBuffer|elementwise_kernel.*copy|CopyKernel|copy_kernel")
    if not vals:
        raise SystemExit(f"no copy dispatch in {path}")
    return copy_bytes / (statistics.median(vals) * 1024.0)


def traffic(args) -> str:
    fetch = _counter(args.fetch, args.kernel)
    write = _counter(args.write, args.kernel)
    if not fetch or not write:
        raise SystemExit("kernel regex matched no dispatch")
    if args.min_fetch_kib > 0:
        # one instantiation can serve several GEMMs: keep the dispatches whose
        # fetch reaches the given size, and the same ordinals of the write run
        # (both runs launch the same kernels in the same order)
        if len(fetch) != len(write):
            raise SystemExit("the two runs dispatched the kernel a different number of times")
        keep = [i for i, v in enumerate(fetch) if v >= args.min_fetch_kib]
        if not keep:
            raise SystemExit("no dispatch reaches --min-fetch-kib")
        fetch = [fetch[i] for i in keep]
        write = [write[i] for i in keep]
    ff = copy_factor(args.fetch_copy, args.copy_bytes)
    wf = copy_factor(args.write_copy, args.copy_bytes)
    fb = statistics.median(fetch) * 1024.0 * ff
    wb = statistics.median(write) * 1024.0 * wf
    t = fb + wb
    lines = [
        f"kernel regex: `{args.kernel}`" + (f", dispatches fetching >= {args.min_fetch_kib:.0f} KiB"
                                            if args.min_fetch_kib > 0 else ""),
        f"dispatches: {len(fetch)} (FETCH_SIZE run), {len(write)} (WRITE_SIZE run)",
        f"copy calibration: FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {wf:.4f} (plain copy of {args.copy_bytes} bytes)",
        f"fetched bytes per launch: {fb:.0f}",
        f"written bytes per launch: {wb:.0f}",
        f"algorithmic bytes per launch: {args.algorithmic}",
        f"traffic / algorithmic: {t / args.algorithmic:.4f}",
        f"traffic_bytes_per_launch: {t:.0f}",
        f"source_hash: {source_hash()}",
    ]
    return "\n".join(lines)


def read_traffic(md_path: str):
    """(traffic bytes per launch, source hash) recorded in a traffic summary,
    or None when the file is missing or names other sources."""
    if not os.path.exists(md_path):
        return None
    txt = open(md_path).read()
    m = re.search(r"traffic_bytes_per_launch: (\d+)", txt)
    h = re.search(r"source_hash: ([0-9a-f]+)", txt)
    if not m or not h:
        return None
    return int(m.group(1)), h.group(1)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--top", type=int, default=20)
    q = sub.add_parser("sequence")
    q.add_argument("csv")
    q.add_argument("--start", required=True)
    q.add_argument("--nth", type=int, default=-1)
    q.add_argument("--until", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--fetch-copy", required=True)
    t.add_argument("--write-copy", required=True)
    t.add_argument("--copy-bytes", type=int, default=1 << 30)
    t.add_argument("--kernel", required=True)
    t.add_argument("--algorithmic", type=int, required=True)
    t.add_argument("--min-fetch-kib", type=float, default=0.0)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.csv, a.top))
    elif a.cmd == "sequence":
        print(sequence_table(a.csv, a.start, a.nth, a.until))
    else:
        print(traffic(a))


if __name__ == "__main__":
    sys.exit(main())
