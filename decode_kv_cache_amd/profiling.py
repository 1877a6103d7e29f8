"""Summaries of rocprofv3 CSV output for the files under profiles/.

  python -m decode_kv_cache_amd.profiling trace <dir> <out.txt> --command "..." [--bench-json FILE]
      per-kernel call count and durations from <dir>/*_kernel_stats.csv and
      *_kernel_trace.csv (rocprofv3 --kernel-trace --stats -f csv), and the
      roofline object of the bench.py line printed by the same run
  python -m decode_kv_cache_amd.profiling pmc <fetch_dir> <write_dir> <out.txt> \\
          --workload NAME --kernel K (--push-bytes B | --total-bytes B) \\
          --command-fetch "..." --command-write "..."
      HBM traffic per dispatch of kernel K from a FETCH_SIZE pass and a
      WRITE_SIZE pass of ``bench.py --counters``, each scaled by what the same
      counter reads for the plain copy kernel of known size run first, against
      the algorithmic bytes per dispatch (given, or the bytes of every
      dispatch of K together divided by their number).

The pmc summary carries the digest of the kernel sources it was taken with;
bench.py reports its traffic only while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
PUSH_KERNEL = "kvx::copy_kernel<0, "   # any launch shape of the push mode
HEADS_KERNEL = ("kvx::heads_kernel", "kvx::heads_many_kernel")
MANY_KERNEL = ("kvx::copy_many_kernel<", "kvx::scale_many_kernel<")   # batched launches and their scale launches
RUN_KERNEL = "kvx::run_kernel<0>"       # push of a run-table plan
KERNELS = {"push": PUSH_KERNEL, "heads": HEADS_KERNEL, "many": MANY_KERNEL, "runs": RUN_KERNEL}
CALIB_KERNEL = "copy_kernel(unsigned int __vector(4)*"   # kvxb_copy in libkvx_bench.so
CALIB_BYTES = 1 << 30


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace runs collapsed, so
    that edits to comments or layout (which do not change the compiled
    kernels) keep a counter summary valid.  String literals in these files
    hold no comment markers."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("kvx_kernels.hip", "kvx_internal.h"):
        with open(os.path.join(PKG, "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _one(pattern: str) -> str:
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _short(name: str) -> str:
    return name if len(name) <= 90 else name[:87] + "..."


def back_to_back(intervals):
    """Launches of one kind in start order: the gaps between one launch's end
    and the next one's start on its queue, and the union of their intervals
    against the sum of their durations (equal when no two overlap)."""
    iv = sorted(intervals)
    gaps = [b[0] - a[1] for a, b in zip(iv, iv[1:])]
    union, cur_s, cur_e = 0, None, None
    for s_, e_ in iv:
        if cur_e is None or s_ > cur_e:
            if cur_e is not None:
                union += cur_e - cur_s
            cur_s, cur_e = s_, e_
        else:
            cur_e = max(cur_e, e_)
    if cur_e is not None:
        union += cur_e - cur_s
    total = sum(e_ - s_ for s_, e_ in iv)
    return gaps, union, total


def bench_roofline(path: str) -> list:
    """The roofline object of the last bench.py JSON line in `path`."""
    import json
    line = None
    for ln in open(path):
        ln = ln.strip()
        if ln.startswith("{") and '"roofline"' in ln:
            line = ln
    if line is None:
        return ["", "bench.py line: none found"]
    r = json.loads(line)
    rf = r["roofline"]
    return ["", f"bench.py line of the same run: value {r['value']} {r['unit']}, workload {r['config']['workload']}",
            f"roofline kernel: {rf.get('kernel')}",
            f"roofline avg_launch_us (dispatch timestamps inside bench.py): {rf.get('avg_launch_us')}",
            f"roofline algorithmic_bytes_per_launch: {rf.get('algorithmic_bytes_per_launch')}",
            f"roofline achieved: {rf['achieved']} GB/s, frac {rf['frac']}"]


def trace_summary(d: str, command: str, bench_json: str = None) -> str:
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_stats.csv")))))
    trace = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_trace.csv")))))
    per = defaultdict(list)
    by_grid = defaultdict(list)
    for r in trace:
        s_, e_ = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        per[r["Kernel_Name"]].append(e_ - s_)
        if "kvx::" in r["Kernel_Name"]:
            key = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), r.get("Queue_Id", ""))
            by_grid[key].append((s_, e_))
    out = ["# rocprofv3 --kernel-trace --stats summary", f"command: {command}",
           f"kernel_source_sha256_16: {kernel_source_digest()}", "",
           "| kernel | calls | avg us | median us | min us | max us | share |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        durs = per.get(name, [])
        med = statistics.median(durs) / 1e3 if durs else float("nan")
        out.append(f"| {_short(name)} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {med:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    out += ["", "libkvx launches by kernel and grid (grid x = work-items along x; one queue each):", "",
            "| kernel | grid x | grid y | queue | calls | avg us | median us | median gap to the next us | "
            "union / sum of durations |", "|---|---|---|---|---|---|---|---|---|"]
    for (name, gx, gy, qid), iv in sorted(by_grid.items(), key=lambda kv: -len(kv[1])):
        if len(iv) < 2:
            continue
        durs = [e_ - s_ for s_, e_ in iv]
        gaps, union, total = back_to_back(iv)
        out.append(f"| {_short(name)} | {gx} | {gy} | {qid} | {len(iv)} | {statistics.mean(durs) / 1e3:.2f} | "
                   f"{statistics.median(durs) / 1e3:.2f} | {statistics.median(gaps) / 1e3:.2f} | "
                   f"{union / total:.4f} |")
    if bench_json:
        out += bench_roofline(bench_json)
    return "\n".join(out) + "\n"


def counters(d: str):
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
    per = defaultdict(list)
    for r in rows:
        per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def _avg_for(per, key):
    keys = key if isinstance(key, tuple) else (key,)
    vals = [v for k, vs in per.items() if any(x in k for x in keys) for v in vs]
    if not vals:
        raise KeyError(key)
    return sum(vals) / len(vals), len(vals)


def pmc_summary(fetch_dir: str, write_dir: str, workload: str, push_bytes, cmd_f: str, cmd_w: str,
                kernel: str = "push", total_bytes=None) -> str:
    f, w = counters(fetch_dir), counters(write_dir)
    cf, ncf = _avg_for(f, CALIB_KERNEL)
    cw, ncw = _avg_for(w, CALIB_KERNEL)
    pf, npf = _avg_for(f, KERNELS[kernel])
    pw, npw = _avg_for(w, KERNELS[kernel])
    if npf != npw:
        raise ValueError(f"{kernel}: {npf} dispatches in the FETCH_SIZE pass, {npw} in the WRITE_SIZE pass")
    if push_bytes is None:
        push_bytes = round(total_bytes / npf)
    ff = CALIB_BYTES / (cf * 1024)
    fw = CALIB_BYTES / (cw * 1024)
    rd = pf * 1024 * ff
    wr = pw * 1024 * fw
    lines = [
        f"# {kernel} kernel HBM traffic, workload {workload}: rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE",
        f"command_fetch: {cmd_f}",
        f"command_write: {cmd_w}",
        f"kernel_source_sha256_16: {kernel_source_digest()}",
        f"calib_kernel: kvxb_copy, {CALIB_BYTES} B read and {CALIB_BYTES} B written per dispatch",
        f"calib_fetch_kib_per_dispatch: {cf:.1f}  (dispatches: {ncf})",
        f"calib_write_kib_per_dispatch: {cw:.1f}  (dispatches: {ncw})",
        f"fetch_factor: {ff:.5f}",
        f"write_factor: {fw:.5f}",
        f"kernel_fetch_kib_per_dispatch: {pf:.1f}  (dispatches: {npf})",
        f"kernel_write_kib_per_dispatch: {pw:.1f}  (dispatches: {npw})",
        f"calibrated_read_bytes_per_launch: {rd:.0f}",
        f"calibrated_write_bytes_per_launch: {wr:.0f}",
        f"calibrated_hbm_bytes_per_launch: {rd + wr:.0f}",
        f"algorithmic_bytes_per_launch: {push_bytes}",
        f"traffic_over_algorithmic: {(rd + wr) / push_bytes:.4f}",
    ]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("out")
    t.add_argument("--command", required=True)
    t.add_argument("--bench-json", default=None, help="stdout of the profiled bench.py run")
    p = sub.add_parser("pmc")
    p.add_argument("fetch_dir")
    p.add_argument("write_dir")
    p.add_argument("out")
    p.add_argument("--workload", required=True)
    b = p.add_mutually_exclusive_group(required=True)
    b.add_argument("--push-bytes", type=int, help="algorithmic bytes per dispatch")
    b.add_argument("--total-bytes", type=int, help="algorithmic bytes of every dispatch of the kernel together")
    p.add_argument("--command-fetch", required=True)
    p.add_argument("--command-write", required=True)
    p.add_argument("--kernel", choices=sorted(KERNELS), default="push")
    a = ap.parse_args()
    if a.what == "trace":
        text = trace_summary(a.dir, a.command, a.bench_json)
    else:
        text = pmc_summary(a.fetch_dir, a.write_dir, a.workload, a.push_bytes, a.command_fetch, a.command_write,
                           a.kernel, a.total_bytes)
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    main()
