"""Summaries of rocprofv3 output for the verify-round kernels.

Two jobs, both on CSV files that rocprofv3 writes with --output-format csv:

  stats    per-kernel dispatch count and duration from a --kernel-trace
           --stats run (the *_kernel_stats.csv file), as a short text table;
  traffic  HBM bytes per dispatch of selected kernels from two --pmc runs
           (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled by
           the factor that makes the same counter read the known size of a
           plain device-to-device copy (the calibration runs of
           ``bench.py --copy-calibration``).

  counters per-kernel means of SQ counters from one or more --pmc runs, with
           per-wave instruction counts and shares of wave and SIMD time.

Usage (after the rocprofv3 runs):
  python -m target_verification_amd.profiling stats  --csv K.csv [--top 20] [--match RE]
  python -m target_verification_amd.profiling traffic --fetch F.csv --write W.csv
      --cal-fetch CF.csv --cal-write CW.csv --cal-bytes B --kernel 'k_qgemm<2, 4, 1, 3>'
      [--kernel ...] --out profiles/gemm_traffic.json
  python -m target_verification_amd.profiling counters --csv A.csv [--csv B.csv ...]
      [--match RE]
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


def _short(name):
    return name.split("(")[0].replace("void ", "")


def counter_means(paths, match=None):
    """{kernel: {counter: mean per dispatch}} over the dispatches of every
    file (a counter read in several files is averaged over all of them)."""
    rx = re.compile(match) if match else None
    sums, disp = {}, {}
    for path in paths:
        per = {}
        for r in _rows(path):
            k = _short(r.get("Kernel_Name", ""))
            if rx and not rx.search(k):
                continue
            key = (k, r["Counter_Name"], r.get("Dispatch_Id"), r.get("Agent_Id"))
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (k, c, _, _), v in per.items():
            sums.setdefault(k, {}).setdefault(c, 0.0)
            sums[k][c] += v
            disp.setdefault(k, {}).setdefault(c, 0)
            disp[k][c] += 1
    return {k: {c: sums[k][c] / disp[k][c] for c in sums[k]} for k in sums}, disp


def counters_table(paths, match=None):
    """Per kernel: dispatches, waves, instructions per wave, and the shares
    SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES (VALU issue in a wave's lifetime),
    SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (ready but not issued),
    SQ_WAIT_ANY / SQ_WAVE_CYCLES (stalled on a dependency or a wait count),
    SQ_ACTIVE_INST_VALU / SQ_BUSY_CU_CYCLES (VALU busy share of the SIMDs of
    busy CUs: ACTIVE_INST_VALU counts 4-cycle units, BUSY_CU_CYCLES cycles of
    a CU with 4 SIMDs) and SQ_VALU_MFMA_BUSY_CYCLES / (4 SQ_BUSY_CU_CYCLES)
    (matrix-core busy share).  Means over dispatches; counters from different
    passes are combined by kernel."""
    means, disp = counter_means(paths, match)

    def g(d, c):
        return d.get(c)

    def ratio(a, b, f=1.0):
        return None if a is None or not b else f * a / b

    cols = ("dispatches", "waves", "VALU/wave", "MFMA/wave", "VMEM rd/wave", "LDS/wave",
            "SALU/wave", "VALU issue", "ready, not issued", "waiting", "VALU busy (SIMD)",
            "MFMA busy (SIMD)")
    lines = ["| kernel | " + " | ".join(cols) + " |", "|---" * (len(cols) + 1) + "|"]
    order = sorted(means, key=lambda k: -(g(means[k], "SQ_WAVES") or 0) *
                   (max(disp[k].values()) if disp[k] else 0))
    for k in order:
        d = means[k]
        w = g(d, "SQ_WAVES")
        vals = [max(disp[k].values()), w,
                ratio(g(d, "SQ_INSTS_VALU"), w), ratio(g(d, "SQ_INSTS_MFMA"), w),
                ratio(g(d, "SQ_INSTS_VMEM_RD"), w), ratio(g(d, "SQ_INSTS_LDS"), w),
                ratio(g(d, "SQ_INSTS_SALU"), w),
                ratio(g(d, "SQ_ACTIVE_INST_VALU"), g(d, "SQ_WAVE_CYCLES")),
                ratio(g(d, "SQ_WAIT_INST_ANY"), g(d, "SQ_WAVE_CYCLES")),
                ratio(g(d, "SQ_WAIT_ANY"), g(d, "SQ_WAVE_CYCLES")),
                ratio(g(d, "SQ_ACTIVE_INST_VALU"), g(d, "SQ_BUSY_CU_CYCLES")),
                ratio(g(d, "SQ_VALU_MFMA_BUSY_CYCLES"), g(d, "SQ_BUSY_CU_CYCLES"), 0.25)]
        cells = []
        for i, v in enumerate(vals):
            if v is None:
                cells.append("-")
            elif i >= 7:
                cells.append(f"{v:.0%}")
            elif i <= 1:
                cells.append(f"{v:.0f}")
            else:
                cells.append(f"{v:.0f}")
        lines.append(f"| {k} | " + " | ".join(cells) + " |")
    return "\n".join(lines)


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
    c = sub.add_parser("counters")
    c.add_argument("--csv", action="append", required=True)
    c.add_argument("--match", default=None, help="regex on kernel names")
    a = p.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.csv, a.top, a.match))
    elif a.cmd == "counters":
        print(counters_table(a.csv, a.match))
    else:
        d = traffic(a.fetch, a.write, a.cal_fetch, a.cal_write, a.cal_bytes, a.kernel)
        with open(a.out, "w") as f:
            json.dump(d, f, indent=1)
        json.dump(d, sys.stdout, indent=1)
        print()


if __name__ == "__main__":
    main()
