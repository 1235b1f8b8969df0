"""Summaries of rocprofv3 runs for the profiles/ folder, and the HBM
traffic figure the benchmark reports.

    python -m block_diffusion_lm_amd.profiling summarize \\
        --workload c4 --trace T.db [--fetch F.db --write W.db] \\
        --command "..." --out profiles/

reads the SQLite databases rocprofv3 writes (default output format) and
writes two short text files:

* ``kernels_<workload>.txt`` -- per-kernel calls and average duration from
  a ``--kernel-trace --stats`` run;
* ``traffic_<kernel>_<workload>.txt`` -- HBM bytes per launch of the
  dominant (longest) kernel from two ``--pmc`` runs (FETCH_SIZE, then
  WRITE_SIZE, KiB per dispatch).  Each counter is scaled by what it reads
  for the device copy of known size that the same run performs
  (``bench.py --copy-calibration-mib``).  The file records a hash of that
  kernel's sources (the shared headers and its own file); ``bench.py``
  reports the figure only while they still hash the same.
"""
from __future__ import annotations

import argparse
import hashlib
import os
import sqlite3
from typing import Dict, Optional

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# bench.py's names of the kernels it times, and the symbols they map to
KERNELS = {
    "fwd": "fwd_kernel",
    "bwd_dq": "bwd_dq_kernel",
    "bwd_dkdv": "bwd_dkdv",
}
COPY_SYMBOL = "copyBuffer"


# the source file that holds each timed kernel
KERNEL_SOURCES = {"fwd": "attn_fwd.hip", "bwd_dq": "attn_bwd.hip", "bwd_dkdv": "attn_bwd.hip",
                  "fwd_fp8": "attn_fwd_fp8.hip"}


def source_hash(kernel: Optional[str] = None) -> str:
    """sha256 over kernel sources (file names and contents): the shared
    headers plus the file holding ``kernel``, or every source when None."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".h", ".hip", ".cpp")):
            continue
        if kernel is not None and not name.endswith(".h") and name != KERNEL_SOURCES[kernel]:
            continue
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _short(name: str) -> str:
    for key, sym in KERNELS.items():
        if sym in name:
            return key
    return name.split("(")[0]


def kernel_stats(db: str) -> Dict[str, dict]:
    """Calls, total and average duration (ns) per kernel from the dispatch table."""
    con = sqlite3.connect(db)
    out = {}
    for name, calls, total, avg in con.execute(
            "select name, count(*), sum(duration), avg(duration) from kernels group by name"):
        out[name] = {"calls": int(calls), "total_ns": float(total), "avg_ns": float(avg)}
    return out


def counter(db: str, counter_name: str) -> Dict[str, float]:
    """Average value per dispatch of one counter, by kernel name."""
    con = sqlite3.connect(db)
    out = {}
    for name, val in con.execute(
            "select kernel_name, avg(value) from counters_collection where counter_name = ? "
            "group by kernel_name", (counter_name,)):
        out[name] = float(val)
    return out


def _find(d: Dict[str, float], needle: str) -> Optional[float]:
    for k, v in d.items():
        if needle in k:
            return v
    return None


def read_traffic(path: str) -> Optional[dict]:
    """Parse a traffic_<kernel>_<workload>.txt file (key: value lines)."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    return vals


def summarize(workload: str, trace: str, fetch: Optional[str], write: Optional[str], command: str,
              out_dir: str, copy_mib: int = 1024, fetch_command: str = "", write_command: str = "") -> None:
    stats = kernel_stats(trace)
    ours = {n: s for n, s in stats.items() if "bd::" in n}
    lines = [f"# rocprofv3 kernel trace, workload {workload}", f"# command: {command}",
             f"# kernel sources sha256 (all files): {source_hash()}", "",
             f"{'kernel':58s} {'calls':>6s} {'avg_us':>10s} {'total_ms':>10s}"]
    for name, s in sorted(ours.items(), key=lambda kv: -kv[1]["avg_ns"]):
        lines.append(f"{name.replace('void ', '')[:58]:58s} {s['calls']:6d} {s['avg_ns'] / 1e3:10.1f} "
                     f"{s['total_ns'] / 1e6:10.2f}")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"kernels_{workload}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if not (fetch and write):
        return
    dom_name = max(ours, key=lambda n: ours[n]["avg_ns"])
    dom = _short(dom_name)
    fk = counter(fetch, "FETCH_SIZE")
    wk = counter(write, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    f_copy = _find(fk, COPY_SYMBOL)
    w_copy = _find(wk, COPY_SYMBOL)
    f_k = _find(fk, KERNELS.get(dom, dom))
    w_k = _find(wk, KERNELS.get(dom, dom))
    f_scale = copy_kib / f_copy
    w_scale = copy_kib / w_copy
    bytes_per_launch = (f_k * f_scale + w_k * w_scale) * 1024.0
    txt = [
        f"# HBM traffic per launch of the dominant kernel ({dom}) on workload {workload}",
        f"# FETCH_SIZE command: {fetch_command}",
        f"# WRITE_SIZE command: {write_command}",
        f"# the copy of {copy_mib} MiB (read + write) calibrates each counter",
        f"kernel: {dom}",
        f"kernel_symbol: {dom_name}",
        f"workload: {workload}",
        f"source_sha256: {source_hash(dom)}",
        f"fetch_kib_per_dispatch: {f_k:.1f}",
        f"write_kib_per_dispatch: {w_k:.1f}",
        f"copy_fetch_kib: {f_copy:.1f}",
        f"copy_write_kib: {w_copy:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"bytes_per_launch: {bytes_per_launch:.0f}",
    ]
    with open(os.path.join(out_dir, f"traffic_{dom}_{workload}.txt"), "w") as f:
        f.write("\n".join(txt) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--workload", required=True)
    s.add_argument("--trace", required=True)
    s.add_argument("--fetch")
    s.add_argument("--write")
    s.add_argument("--command", default="", help="the kernel-trace command")
    s.add_argument("--fetch-command", default="")
    s.add_argument("--write-command", default="")
    s.add_argument("--copy-mib", type=int, default=1024)
    s.add_argument("--out", default="profiles")
    sub.add_parser("hash")
    a = ap.parse_args()
    if a.cmd == "hash":
        print(source_hash())
    else:
        summarize(a.workload, a.trace, a.fetch, a.write, a.command, a.out, a.copy_mib,
                  a.fetch_command, a.write_command)


if __name__ == "__main__":
    main()
