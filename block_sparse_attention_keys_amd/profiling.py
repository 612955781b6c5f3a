"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m block_sparse_attention_keys_amd.profiling trace \
        --dir OUT_DIR --cmd "the profiled command" --title T --out profiles/x.txt
    python -m block_sparse_attention_keys_amd.profiling counters \
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes N \
        --kernel REGEX --algo-bytes B --cmd "..." --title T --out profiles/y.txt

`counters` scales each HBM counter (FETCH_SIZE, WRITE_SIZE: KiB per
dispatch) by what the same counter reads for a plain device copy of a known
number of bytes, and records the sha256 of the kernel source it was taken
on: bench.py reports the traffic figure only while that source is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics
from typing import Dict, List

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")


def kernel_source_sha256() -> str:
    """sha256 over every source file of the library (kernels, shared device
    helpers, launch configuration), in name order."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_sha256(run_dir: str) -> str:
    """The library sources' sha256 recorded next to a measurement
    (``source_sha256.txt`` in the run directory or its parent, written by
    ``python -m block_sparse_attention_keys_amd.profiling sha > FILE`` on the
    GPU machine before profiling); the current sources' when none was recorded."""
    for d in (run_dir, os.path.dirname(os.path.normpath(run_dir))):
        f = os.path.join(d, "source_sha256.txt")
        if os.path.exists(f):
            return open(f).read().strip()
    return kernel_source_sha256()


def _one(pattern: str) -> str:
    files = sorted(glob.glob(pattern, recursive=True))
    if not files:
        raise FileNotFoundError(pattern)
    return files[0]


def _short(name: str) -> str:
    name = re.sub(r"^void ", "", name)
    name = name.replace("qsa::(anonymous namespace)::", "")
    return re.sub(r"\(.*$", "", name)


def trace_rows(d: str) -> List[dict]:
    path = _one(os.path.join(d, "**", "*kernel_trace.csv"))
    with open(path) as f:
        return list(csv.DictReader(f))


def trace_summary(d: str) -> List[dict]:
    per: Dict[str, List[float]] = {}
    for r in trace_rows(d):
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        per.setdefault(_short(r["Kernel_Name"]), []).append(dur)
    out = []
    for k, v in per.items():
        out.append({"kernel": k, "calls": len(v), "avg_us": statistics.mean(v),
                    "min_us": min(v), "max_us": max(v), "total_ms": sum(v) / 1000.0})
    out.sort(key=lambda x: -x["total_ms"])
    return out


def counter_values(d: str, counter: str, kernel_regex: str) -> List[float]:
    path = _one(os.path.join(d, "**", "*counter_collection.csv"))
    vals = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and re.search(kernel_regex, r["Kernel_Name"]):
                vals.append(float(r["Counter_Value"]))
    return vals


def counter_per_launch(d: str, counter: str, kernel_regex: str) -> Dict[str, float]:
    """Mean counter value per dispatch of each matching kernel; a launch of the
    measured entry point is one dispatch of each, so their sum is per launch."""
    path = _one(os.path.join(d, "**", "*counter_collection.csv"))
    per: Dict[str, List[float]] = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and re.search(kernel_regex, r["Kernel_Name"]):
                per.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: statistics.mean(v) for k, v in per.items()}


def cmd_trace(a) -> None:
    rows = trace_summary(a.dir)
    lines = [f"# {a.title}", "", f"command: {a.cmd}",
             f"kernel_source_sha256: {measured_sha256(a.dir)}", "",
             "| kernel | calls | avg us | min us | max us | total ms |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        if a.only and not re.search(a.only, r["kernel"]):
            continue
        lines.append(f"| {r['kernel']} | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} | {r['total_ms']:.3f} |")
    if a.note:
        lines += ["", a.note]
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


def cmd_counters(a) -> None:
    fetch = counter_per_launch(a.fetch, "FETCH_SIZE", a.kernel)
    write = counter_per_launch(a.write, "WRITE_SIZE", a.kernel)
    cf = counter_values(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cw = counter_values(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    if not (fetch and write and cf and cw):
        raise SystemExit("missing counter rows")
    # bytes per counted KiB, from the plain copy (reads and writes copy_bytes each)
    f_factor = a.copy_bytes / (statistics.median(cf) * 1024.0)
    w_factor = a.copy_bytes / (statistics.median(cw) * 1024.0)
    fk, wk = sum(fetch.values()), sum(write.values())
    traffic = fk * 1024.0 * f_factor + wk * 1024.0 * w_factor
    lines = [f"# {a.title}", "", f"command (fetch): {a.cmd_fetch}", f"command (write): {a.cmd_write}",
             f"command (copy calibration): {a.cmd_copy}",
             f"kernel: {a.kernel}", f"kernel_source_sha256: {measured_sha256(a.fetch)}",
             "fetch_kib_per_dispatch_by_kernel: " +
             ", ".join(f"{k} {v:.1f}" for k, v in fetch.items()),
             "write_kib_per_dispatch_by_kernel: " +
             ", ".join(f"{k} {v:.1f}" for k, v in write.items()),
             f"fetch_kib_per_launch: {fk:.1f}", f"write_kib_per_launch: {wk:.1f}",
             f"copy_bytes: {a.copy_bytes}",
             f"copy_fetch_kib: {statistics.median(cf):.1f}",
             f"copy_write_kib: {statistics.median(cw):.1f}",
             f"fetch_factor_bytes_per_kib: {f_factor * 1024.0:.1f}",
             f"write_factor_bytes_per_kib: {w_factor * 1024.0:.1f}",
             f"traffic_bytes_per_launch: {traffic:.0f}",
             f"algorithmic_bytes_per_launch: {a.algo_bytes}",
             f"traffic_over_algorithmic: {traffic / a.algo_bytes:.3f}"]
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


def read_summary(path: str) -> Dict[str, str]:
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        m = re.match(r"^([a-z_0-9]+): (.*)$", line.strip())
        if m:
            out[m.group(1)] = m.group(2)
    return out


def cmd_pmc(a) -> None:
    """Mean per dispatch of every counter in one or more --pmc runs (one
    --dir and one --cmd per run, in the same order), for the kernels
    matching --kernel."""
    if len(a.dir) != len(a.cmd):
        raise SystemExit("give one --cmd per --dir")
    shas = {measured_sha256(d) for d in a.dir}
    if len(shas) != 1:
        raise SystemExit(f"the runs were measured on different sources: {sorted(shas)}")
    per: Dict[tuple, List[float]] = {}
    for d in a.dir:
        with open(_one(os.path.join(d, "**", "*counter_collection.csv"))) as f:
            for r in csv.DictReader(f):
                if re.search(a.kernel, r["Kernel_Name"]):
                    per.setdefault((_short(r["Kernel_Name"]), r["Counter_Name"]), []).append(
                        float(r["Counter_Value"]))
    lines = [f"# {a.title}", ""] + [f"command: {c}" for c in a.cmd] + [
             f"kernel_source_sha256: {shas.pop()}", "",
             "| kernel | counter | dispatches | mean per dispatch |", "|---|---|---|---|"]
    for (k, c), v in sorted(per.items()):
        lines.append(f"| {k} | {c} | {len(v)} | {statistics.mean(v):.6g} |")
    if a.note:
        lines += ["", a.note]
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--dir", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--only", default="")
    t.add_argument("--note", default="")
    sub.add_parser("sha")
    q = sub.add_parser("pmc")
    for k in ("dir", "cmd"):
        q.add_argument("--" + k, required=True, action="append")
    for k in ("title", "out", "kernel"):
        q.add_argument("--" + k, required=True)
    q.add_argument("--note", default="")
    c = sub.add_parser("counters")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        c.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--copy-kernel", default="copyBuffer|copy")
    c.add_argument("--kernel", required=True)
    c.add_argument("--algo-bytes", type=int, required=True)
    c.add_argument("--cmd-fetch", required=True)
    c.add_argument("--cmd-write", required=True)
    c.add_argument("--cmd-copy", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.what == "sha":
        print(kernel_source_sha256())
        return
    {"trace": cmd_trace, "counters": cmd_counters, "pmc": cmd_pmc}[a.what](a)


if __name__ == "__main__":
    main()
