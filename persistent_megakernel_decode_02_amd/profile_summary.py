"""Turn rocprofv3 output into the short summaries kept under profiles/.

Two summaries per kernel and workload, each naming the commands that made it:

* ``kernel-trace``: the per-kernel statistics of ``rocprofv3 --kernel-trace
  --stats`` (calls, average / min / max duration), beside the mean kernel time
  the same process measured with HIP events (bench.py's ``kernel_ms_mean``);
* ``traffic``: HBM bytes per launch from two counter passes (``FETCH_SIZE``,
  then ``WRITE_SIZE``), each scaled by what the same counter reports for a
  plain device copy of known size (bench.py ``--calib-copy``), against the
  launch's algorithmic bytes.  A JSON twin records the result with the hash
  of the kernel sources, so bench.py reports it only while the kernel is the
  one that was measured.

Usage (after the rocprofv3 runs; paths are rocprofv3 output directories and
bench.py's JSON output lines):

  python -m persistent_megakernel_decode_02_amd.profile_summary kernel-trace \
      --kernel K --workload W --stats DIR --bench OUT.json [--plain-bench OUT2.json] \
      --command "..." [--command "..."] --out profiles/K_W_kernel_trace.md
  python -m persistent_megakernel_decode_02_amd.profile_summary traffic \
      --kernel K --workload W --fetch DIR --write DIR --calib-fetch DIR --calib-write DIR \
      --calib-bytes N --bench OUT.json --command "..." ... --out profiles/K_W_traffic.md
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
from typing import Dict, List

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
KERNEL_SRCS = ["mkd_device.h", "mkd_internal.h", "mkd_kernel_dense.hip", "mkd_kernel_moe.hip",
               "mkd_kernel_batch.hip", "mkd_launch.hip"]


def kernel_digest() -> str:
    """sha256[:16] over the device sources (the same digest bench.py checks)."""
    h = hashlib.sha256()
    for name in KERNEL_SRCS:
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def _one(pattern: str) -> str:
    found = sorted(glob.glob(pattern, recursive=True))
    if not found:
        raise SystemExit(f"no file matches {pattern}")
    return found[0]


def _bench(path: str) -> dict:
    """The last JSON line bench.py printed."""
    last = None
    for line in open(path):
        line = line.strip()
        if line.startswith("{"):
            last = json.loads(line)
    if last is None:
        raise SystemExit(f"no bench.py JSON line in {path}")
    return last


def kernel_stats(dirname: str) -> List[dict]:
    """Rows of rocprofv3's kernel statistics (durations in ns)."""
    rows = []
    with open(_one(os.path.join(dirname, "**", "*kernel_stats.csv"))) as f:
        for r in csv.DictReader(f):
            rows.append({"name": r["Name"], "calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
                         "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"])})
    return rows


def counter_values(dirname: str, counter: str, kernel_prefix: str) -> List[float]:
    """Per-dispatch values of one counter for the kernels whose name starts
    with kernel_prefix (a kernel's value is summed over its rows: rocprofv3
    may report one row per dimension instance)."""
    per: Dict[int, float] = {}
    with open(_one(os.path.join(dirname, "**", "*counter_collection.csv"))) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or not r["Kernel_Name"].startswith(kernel_prefix):
                continue
            d = int(r["Dispatch_Id"])
            per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def _fmt_ms(ns: float) -> str:
    return f"{ns / 1e6:.3f}" if ns >= 1e5 else f"{ns / 1e6:.4f}"


def write_kernel_trace(a) -> None:
    rows = kernel_stats(a.stats)
    b = _bench(a.bench)
    lines = [f"# {a.kernel}, {a.workload}: rocprofv3 kernel trace", ""]
    lines.append("Commands (repo root, one MI355X; the profiled run dispatches the same grid without the "
                 "cooperative flag: after a cooperative dispatch, rocprofv3 7.2 crashes at process exit "
                 "before it writes any output):")
    lines.append("")
    lines.append("```")
    lines += a.command
    lines.append("```")
    lines.append("")
    lines.append("| Kernel | Calls | Average ms | Min ms | Max ms |")
    lines.append("|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -r["avg_ns"] * r["calls"]):
        if r["name"].startswith("mkd_"):
            lines.append(f"| {r['name']} | {r['calls']} | {_fmt_ms(r['avg_ns'])} | {_fmt_ms(r['min_ns'])} | "
                         f"{_fmt_ms(r['max_ns'])} |")
    lines.append("")
    rf = b["roofline"]
    cfg = b["config"]
    lines.append(f"Same process, HIP events around each launch (bench.py `kernel_ms_mean`, timed steps only): "
                 f"{rf['kernel_ms_mean']:.3f} ms.")
    if a.plain_bench:
        p = _bench(a.plain_bench)
        pr = p["roofline"]
        lines.append(f"Cooperative launch, no profiler: {pr['kernel_ms_mean']:.3f} ms, "
                     f"{p['us_per_token']:.1f} us/token, {pr['achieved']:.0f} GB/s algorithmic = "
                     f"{100 * pr['frac']:.1f}% of 8 TB/s.")
    lines.append(f"Decode tokens per launch: {cfg['decode_tokens_per_step']}; n_wg {cfg['n_wg']}, "
                 f"n_chunks {cfg['n_chunks']}; algorithmic bytes per launch {rf['algorithmic_bytes_per_launch']:.4e}.")
    lines.append(f"Kernel source sha256[:16]: {kernel_digest()}.")
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    open(a.out, "w").write("\n".join(lines) + "\n")
    print(f"wrote {a.out}")


def write_traffic(a) -> None:
    b = _bench(a.bench)
    n_alg = float(b["roofline"]["algorithmic_bytes_per_launch"])
    fetch = counter_values(a.fetch, "FETCH_SIZE", a.kernel)
    write = counter_values(a.write, "WRITE_SIZE", a.kernel)
    cf = counter_values(a.calib_fetch, "FETCH_SIZE", a.calib_kernel)
    cw = counter_values(a.calib_write, "WRITE_SIZE", a.calib_kernel)
    if not (fetch and write and cf and cw):
        raise SystemExit("missing counter values")
    # the copy kernel's dispatches of the full size are the calibration ones
    cf_big = max(cf)
    cw_big = max(cw)
    f_scale = a.calib_bytes / (cf_big * 1024)
    w_scale = a.calib_bytes / (cw_big * 1024)
    fetch_b = sum(fetch) / len(fetch) * 1024 * f_scale
    write_b = sum(write) / len(write) * 1024 * w_scale
    total = fetch_b + write_b
    digest = kernel_digest()
    lines = [f"# {a.kernel}, {a.workload}: HBM traffic counters", ""]
    lines.append("Each counter in a pass of its own (repo root, one MI355X):")
    lines.append("")
    lines.append("```")
    lines += a.command
    lines.append("```")
    lines.append("")
    lines.append(f"| Counter | {a.kernel} (KiB per dispatch) | {a.calib_bytes / 2**30:g} GiB copy (KiB per dispatch) | "
                 f"scale to bytes | bytes per launch |")
    lines.append("|---|---|---|---|---|")
    lines.append(f"| FETCH_SIZE | {', '.join(f'{v:.0f}' for v in fetch)} | {cf_big:.0f} | x{f_scale:.4f} x1024 | "
                 f"{fetch_b:.4e} |")
    lines.append(f"| WRITE_SIZE | {', '.join(f'{v:.0f}' for v in write)} | {cw_big:.0f} | x{w_scale:.4f} x1024 | "
                 f"{write_b:.4e} |")
    lines.append("")
    lines.append(f"Scale: the copy reads and writes exactly {a.calib_bytes:,} B; FETCH_SIZE reports {cf_big:.0f} KiB "
                 f"of it and WRITE_SIZE {cw_big:.0f} KiB, so the factors are {f_scale:.4f} and {w_scale:.4f}.")
    lines.append(f"HBM bytes per launch (fetch + write): {total:.4e}. Algorithmic bytes per launch "
                 f"(weights + K/V read + K/V append): {n_alg:.4e}; measured / algorithmic = {total / n_alg:.4f} "
                 f"(fetch alone {fetch_b / n_alg:.4f}).")
    lines.append(f"Kernel source sha256[:16]: {digest}.")
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    open(a.out, "w").write("\n".join(lines) + "\n")
    js = os.path.splitext(a.out)[0] + ".json"
    json.dump({"kernel": a.kernel, "workload": a.workload, "kernel_sha256_16": digest,
               "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
               "hbm_bytes_per_launch": total, "algorithmic_bytes_per_launch": n_alg,
               "fetch_scale": f_scale, "write_scale": w_scale,
               "source": os.path.relpath(a.out, os.path.dirname(HERE))}, open(js, "w"), indent=1)
    print(f"wrote {a.out} and {js}")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernel-trace")
    k.add_argument("--kernel", required=True)
    k.add_argument("--workload", required=True)
    k.add_argument("--stats", required=True, help="rocprofv3 output directory of the --kernel-trace --stats run")
    k.add_argument("--bench", required=True, help="bench.py output of the profiled run")
    k.add_argument("--plain-bench", default=None, help="bench.py output of the same workload without the profiler")
    k.add_argument("--command", action="append", default=[])
    k.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--calib-fetch", required=True)
    t.add_argument("--calib-write", required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--calib-kernel", default="", help="name prefix of the copy kernel (default: any)")
    t.add_argument("--bench", required=True)
    t.add_argument("--command", action="append", default=[])
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.what == "kernel-trace":
        write_kernel_trace(a)
    else:
        write_traffic(a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
