"""Summaries of rocprofv3 output for the verify-round kernels.

Two jobs, both on CSV files that rocprofv3 writes with --output-format csv:

  stats    per-kernel dispatch count and duration from a --kernel-trace
           --stats run (the *_kernel_stats.csv file), as a short text table;
  traffic  HBM bytes per dispatch of selected kernels from two --pmc runs
           (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled by
           the factor that makes the same counter read the known size of a
           plain device-to-device copy (the calibration runs of
           ``bench.py --copy-calibration``).

Usage (after the rocprofv3 runs):
  python -m target_verification_amd.profiling stats  --csv K.csv [--top 20] [--match RE]
  python -m target_verification_amd.profiling traffic --fetch F.csv --write W.csv
      --cal-fetch CF.csv --cal-write CW.csv --cal-bytes B --kernel 'k_qgemm<2, 4, 1, 3>'
      [--kernel ...] --out profiles/gemm_traffic.json
"""

import argparse
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_SOURCES = ("sv_gemm.hip", "sv_gemm_body.h", "sv_epi.h", "sv_device.h", "sv_internal.h")


def _code_only(text):
    """Source text without comments and with whitespace collapsed, so that a
    change of comments alone keeps the hash."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def gemm_source_hash():
    """Hash of the code the quantized GEMM kernel is built from (comments
    and layout ignored); counter readings taken on other code are stale."""
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "target_verification_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def kernel_stats(path):
    """[(name, calls, total_ns, avg_ns, min_ns, max_ns)] sorted by total."""
    out = []
    for r in _rows(path):
        out.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]),
                    float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"])))
    out.sort(key=lambda t: -t[2])
    return out


def stats_table(path, top=20, match=None):
    rows = kernel_stats(path)
    if match:
        rx = re.compile(match)
        rows = [r for r in rows if rx.search(r[0])]
    total = sum(r[2] for r in rows) or 1.0
    lines = [f"{'kernel':70s} {'calls':>7s} {'total ms':>10s} {'avg us':>9s} "
             f"{'min us':>9s} {'max us':>9s} {'share':>6s}"]
    for name, calls, tot, avg, mn, mx in rows[:top]:
        short = name if len(name) <= 70 else name[:67] + "..."
        lines.append(f"{short:70s} {calls:7d} {tot / 1e6:10.3f} {avg / 1e3:9.2f} "
                     f"{mn / 1e3:9.2f} {mx / 1e3:9.2f} {tot / total:6.1%}")
    return "\n".join(lines)


def counter_per_dispatch(path, counter, kernel_substr=None):
    """Mean of a counter over the dispatches whose kernel name contains
    kernel_substr (all dispatches if None); returns (mean, n)."""
    vals = {}
    for r in _rows(path):
        if r.get("Counter_Name") != counter:
            continue
        name = r.get("Kernel_Name", "")
        if kernel_substr is not None and kernel_substr not in name:
            continue
        key = (r.get("Dispatch_Id"), r.get("Agent_Id"))
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        return None, 0
    return sum(vals.values()) / len(vals), len(vals)


def _largest_dispatch(path, counter):
    """Counter of the largest dispatch (the calibration copy dominates)."""
    best = 0.0
    per = {}
    for r in _rows(path):
        if r.get("Counter_Name") != counter:
            continue
        key = (r.get("Dispatch_Id"), r.get("Agent_Id"))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    for v in per.values():
        best = max(best, v)
    return best


def traffic(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, cal_bytes, kernels):
    cf = _largest_dispatch(cal_fetch_csv, "FETCH_SIZE")
    cw = _largest_dispatch(cal_write_csv, "WRITE_SIZE")
    f_scale = cal_bytes / cf if cf else None
    w_scale = cal_bytes / cw if cw else None
    out = {"source_hash": gemm_source_hash(), "calibration": {
        "copy_bytes": cal_bytes, "fetch_reading": cf, "write_reading": cw,
        "fetch_bytes_per_unit": f_scale, "write_bytes_per_unit": w_scale}, "kernels": {}}
    for k in kernels:
        fv, nf = counter_per_dispatch(fetch_csv, "FETCH_SIZE", k)
        wv, nw = counter_per_dispatch(write_csv, "WRITE_SIZE", k)
        rec = {"dispatches": [nf, nw], "fetch_reading": fv, "write_reading": wv}
        if fv is not None and wv is not None and f_scale and w_scale:
            rec["fetch_bytes"] = fv * f_scale
            rec["write_bytes"] = wv * w_scale
            rec["hbm_bytes_per_launch"] = fv * f_scale + wv * w_scale
        out["kernels"][k] = rec
    return out


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--top", type=int, default=20)
    s.add_argument("--match", default=None, help="regex on kernel names")
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--cal-fetch", "--cal-write", "--out"):
        t.add_argument(a, required=True)
    t.add_argument("--cal-bytes", type=int, required=True)
    t.add_argument("--kernel", action="append", required=True)
    a = p.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.csv, a.top, a.match))
    else:
        d = traffic(a.fetch, a.write, a.cal_fetch, a.cal_write, a.cal_bytes, a.kernel)
        with open(a.out, "w") as f:
            json.dump(d, f, indent=1)
        json.dump(d, sys.stdout, indent=1)
        print()


if __name__ == "__main__":
    main()
