"""Condense rocprofv3 CSV output (``-f csv``) into the short text summaries
kept under profiles/.

    python -m gated_linear_recurrence_history_amd.rocprof_summary stats DIR OUT --command "..."
    python -m gated_linear_recurrence_history_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR OUT \
        --kernel gscan_bwd_kernel --workload prod_fp32 --copy-bytes N --command "..."

    python -m gated_linear_recurrence_history_amd.rocprof_summary counters OUT DIR [DIR ...] \
        --kernel NAME [--kernel NAME ...] --command "..."

``stats`` keeps rocprofv3's own per-kernel statistics (kernel_stats.csv).
``counters`` gives, for each named kernel, the mean per dispatch of every
counter or derived metric the given ``--pmc`` runs collected (rows of one
dispatch summed, as rocprofv3 writes one row per instance).
``traffic`` turns two counter runs (FETCH_SIZE, then WRITE_SIZE; both in KiB
per dispatch) into HBM bytes per launch of one kernel.  Each counter is
scaled by what it reads for a plain device-to-device copy of ``copy-bytes``
bytes recorded at the end of the same run (the last ``copies`` dispatches of
the runtime's copy kernel; each reads and writes exactly that many bytes),
and the result carries the SHA-256 of the kernel source so a
reader can tell when the counters no longer describe the code.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(HERE, "csrc", "gscan_kernels.hip")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_source_sha256() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def short_name(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("gscan::", "")
    if n.startswith("void "):
        n = n[5:]
    return n.split("(")[0].strip()


def _find(directory: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    return hits[0]


def _col(header, *keys):
    low = [h.lower() for h in header]
    for k in keys:
        if k in low:
            return low.index(k)
    raise KeyError(f"none of {keys} in {header}")


def stats(directory: str):
    """[(kernel, calls, avg_ns, min_ns, max_ns, total_ns, percent)] from kernel_stats.csv."""
    path = _find(directory, "kernel_stats.csv")
    with open(path, newline="") as f:
        rows = list(csv.reader(f))
    h = rows[0]
    iname, icalls = _col(h, "name"), _col(h, "calls")
    iavg, imin, imax = _col(h, "averagens"), _col(h, "minns"), _col(h, "maxns")
    itot, ipct = _col(h, "totaldurationns"), _col(h, "percentage")
    out = []
    for r in rows[1:]:
        out.append((short_name(r[iname]), int(r[icalls]), float(r[iavg]), float(r[imin]),
                    float(r[imax]), float(r[itot]), float(r[ipct])))
    return out


def counter_per_dispatch(directory: str, counter: str):
    """{kernel: [value per dispatch]} for one counter (rows of a dispatch summed)."""
    path = _find(directory, "counter_collection.csv")
    with open(path, newline="") as f:
        rows = list(csv.reader(f))
    h = rows[0]
    idisp, iname = _col(h, "dispatch_id"), _col(h, "kernel_name")
    icn, icv = _col(h, "counter_name"), _col(h, "counter_value")
    per = {}
    for r in rows[1:]:
        if r[icn] != counter:
            continue
        key = (short_name(r[iname]), int(r[idisp]))
        per[key] = per.get(key, 0.0) + float(r[icv])
    out = {}
    for (k, _), v in sorted(per.items(), key=lambda kv: kv[0][1]):
        out.setdefault(k, []).append(v)
    return out


def write_stats(directory, out_path, command):
    lines = ["rocprofv3 kernel statistics (from its kernel_stats.csv)", "",
             f"command: {command}", "",
             f"{'kernel':<56} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'share':>7}"]
    for name, calls, avg, mn, mx, tot, pct in stats(directory):
        lines.append(f"{name[:56]:<56} {calls:>6} {avg / 1e3:>9.3f} {mn / 1e3:>9.3f} "
                     f"{mx / 1e3:>9.3f} {pct:>6.2f}%")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_traffic(fetch_dir, write_dir, out_path, kernel, workload, copy_bytes, copies, command):
    fetch = counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = counter_per_dispatch(write_dir, "WRITE_SIZE")
    kf, kw = statistics.mean(fetch[kernel]), statistics.mean(write[kernel])
    cf = statistics.mean(fetch[COPY_KERNEL][-copies:])
    cw = statistics.mean(write[COPY_KERNEL][-copies:])
    fetch_scale = copy_bytes / (cf * 1024.0)
    write_scale = copy_bytes / (cw * 1024.0)
    rec = {
        "kernel": kernel, "workload": workload, "source_sha256": kernel_source_sha256(),
        "fetch_kib_per_dispatch": round(kf, 1), "write_kib_per_dispatch": round(kw, 1),
        "dispatches": [len(fetch[kernel]), len(write[kernel])],
        "copy_bytes": copy_bytes, "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
        "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
        "traffic_bytes": int(round(kf * 1024.0 * fetch_scale + kw * 1024.0 * write_scale)),
    }
    lines = [f"HBM traffic of {kernel} on {workload} from rocprofv3 FETCH_SIZE and WRITE_SIZE", "",
             f"commands: {command}", "",
             f"{kernel}: FETCH_SIZE {kf:.1f} KiB, WRITE_SIZE {kw:.1f} KiB per dispatch "
             f"(means over {len(fetch[kernel])} and {len(write[kernel])} dispatches)",
             f"calibration: device copy of {copy_bytes} bytes reads FETCH_SIZE {cf:.1f} KiB and "
             f"WRITE_SIZE {cw:.1f} KiB -> scale {fetch_scale:.4f} (fetch), {write_scale:.4f} (write)",
             f"traffic per launch: {rec['traffic_bytes']} bytes", "",
             "record: " + json.dumps(rec)]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return rec


def counter_names(directory: str):
    """Counter and metric names present in one counter_collection.csv, in file order."""
    path = _find(directory, "counter_collection.csv")
    with open(path, newline="") as f:
        rows = list(csv.reader(f))
    icn = _col(rows[0], "counter_name")
    seen = []
    for r in rows[1:]:
        if r[icn] not in seen:
            seen.append(r[icn])
    return seen


def write_counters(dirs, out_path, kernels, command):
    """Mean per dispatch of every collected counter for each kernel; returns {kernel: {counter: v}}."""
    table = {k: {} for k in kernels}
    counts = {k: {} for k in kernels}
    for d in dirs:
        for c in counter_names(d):
            per = counter_per_dispatch(d, c)
            for k in kernels:
                if k in per:
                    table[k][c] = statistics.mean(per[k])
                    counts[k][c] = len(per[k])
    lines = ["rocprofv3 counters per dispatch (mean over dispatches)", "",
             f"commands: {command}", ""]
    for k in kernels:
        lines.append(k)
        for c, v in table[k].items():
            lines.append(f"  {c:<34} {v:>18.4f}   ({counts[k][c]} dispatches)")
        lines.append("")
    lines.append("record: " + json.dumps(table))
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return table


def read_traffic(path):
    """The record of a traffic summary, or None if absent or unparsable."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("record: "):
                    return json.loads(line[len("record: "):])
    except OSError:
        return None
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("out")
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--copies", type=int, default=4)
    t.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("out")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", action="append", required=True)
    c.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.mode == "stats":
        write_stats(a.dir, a.out, a.command)
    elif a.mode == "counters":
        print(json.dumps(write_counters(a.dirs, a.out, a.kernel, a.command)))
    else:
        print(json.dumps(write_traffic(a.fetch_dir, a.write_dir, a.out, a.kernel, a.workload,
                                       a.copy_bytes, a.copies, a.command)))


if __name__ == "__main__":
    main()
