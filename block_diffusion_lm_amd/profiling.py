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


def read_counters(path: str) -> Optional[dict]:
    """Parse a counters_<workload>.txt file: {"source_sha256": ..., kernel:
    {name: value}} (None when missing)."""
    if not os.path.exists(path):
        return None
    out: dict = {}
    cur = None
    with open(path) as f:
        for line in f:
            if line.startswith("# kernel sources sha256 (all files):"):
                out["source_sha256"] = line.split(":", 1)[1].strip()
            elif line.startswith("["):
                cur = out.setdefault(line[1:line.index("]")], {})
            elif cur is not None and line.startswith("  ") and line.strip():
                name, val = line.split()
                cur[name] = float(val)
    return out


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


# The counter passes behind counters_<workload>.txt (each within one
# pass's hardware limits: at most 8 SQ, 4 TCC and 2 GRBM counters).
COUNTER_PASSES = [
    ["GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
     "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_LDS_BANK_CONFLICT"],
    ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VALU_TRANS_F32",
     "SQ_WAIT_INST_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES"],
    ["FETCH_SIZE"],
    ["WRITE_SIZE"],
    ["GRBM_GUI_ACTIVE", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_MISC",
     "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU_FMA_F32", "SQ_INSTS_VALU_MUL_F32", "SQ_INSTS_VALU_ADD_F32"],
]
NUM_CU = 256      # MI355X compute units
SIMD_PER_CU = 4
NUM_XCD = 8       # GRBM_GUI_ACTIVE reads the sum over the 8 XCDs (it is 8x the
                  # kernel's duration times the clock)


def counters_summary(workload: str, trace: str, pmc_dbs, commands, copy_mib: int, out_dir: str) -> str:
    """Per kernel: the average per dispatch of every counter of
    COUNTER_PASSES, and what follows from them (see the file's notes)."""
    stats = {_short(n): s for n, s in kernel_stats(trace).items() if "bd::" in n}
    vals: Dict[str, Dict[str, float]] = {}
    copy = {}
    for db in pmc_dbs:
        con = sqlite3.connect(db)
        for name, cname, val in con.execute(
                "select kernel_name, counter_name, avg(value) from counters_collection "
                "group by kernel_name, counter_name"):
            if COPY_SYMBOL in name:
                copy[cname] = float(val)
            if "bd::" in name:
                vals.setdefault(_short(name), {})[cname] = float(val)
    copy_kib = copy_mib * 1024.0
    fscale = copy_kib / copy["FETCH_SIZE"] if copy.get("FETCH_SIZE") else None
    wscale = copy_kib / copy["WRITE_SIZE"] if copy.get("WRITE_SIZE") else None
    lines = [f"# rocprofv3 counters per dispatch, workload {workload}",
             f"# kernel sources sha256 (all files): {source_hash()}",
             "# commands (one counter pass each; the kernel durations from the trace):"]
    lines += [f"#   {c}" for c in commands]
    lines += ["# derived:",
              "#   clock_mhz = GRBM_GUI_ACTIVE / 8 XCDs / duration",
              "#   mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs * 256 CU * 4 SIMD):",
              "#     the share of the matrix cores' cycles spent on MFMAs (32 cycles per 32x32x16 bf16)",
              "#   valu_busy = SQ_ACTIVE_INST_VALU / (GRBM_GUI_ACTIVE / 8 XCDs * 256 CU): the share of",
              "#     the vector units' issue cycles in use (quad-cycles per CU, rocprofv3's VALUBusy)",
              "#   mfma_tflops = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 flop / duration",
              "#   valu_per_mfma, lds_per_mfma, salu_per_mfma = instruction counts / SQ_INSTS_MFMA",
              "#   hbm_gbs = (FETCH_SIZE * fetch_scale + WRITE_SIZE * write_scale) KiB / duration,",
              f"#   scales from a {copy_mib} MiB device copy in the same runs "
              f"(fetch {fscale if fscale else float('nan'):.3f}, write {wscale if wscale else float('nan'):.3f})",
              ""]
    for k in sorted(vals, key=lambda k: -stats.get(k, {"avg_ns": 0})["avg_ns"]):
        v = vals[k]
        dur = stats.get(k, {}).get("avg_ns")
        lines.append(f"[{k}] {dur / 1e3:.1f} us per dispatch" if dur else f"[{k}]")
        for cname in [c for p in COUNTER_PASSES for c in p]:
            if cname in v:
                lines.append(f"  {cname:32s} {v[cname]:.6g}")
        mf = v.get("SQ_INSTS_MFMA")
        if v.get("GRBM_GUI_ACTIVE") and dur:
            lines.append(f"  {'clock_mhz':32s} {v['GRBM_GUI_ACTIVE'] / NUM_XCD / (dur * 1e-9) / 1e6:.0f}")
        if v.get("SQ_VALU_MFMA_BUSY_CYCLES") and v.get("GRBM_GUI_ACTIVE"):
            cyc = v["GRBM_GUI_ACTIVE"] / NUM_XCD * NUM_CU * SIMD_PER_CU
            lines.append(f"  {'mfma_busy':32s} {v['SQ_VALU_MFMA_BUSY_CYCLES'] / cyc:.4f}")
        if v.get("SQ_ACTIVE_INST_VALU") and v.get("GRBM_GUI_ACTIVE"):
            lines.append(f"  {'valu_busy':32s} {v['SQ_ACTIVE_INST_VALU'] / (v['GRBM_GUI_ACTIVE'] / NUM_XCD * NUM_CU):.4f}")
        if v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16") and dur:
            lines.append(f"  {'mfma_tflops':32s} {v['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / (dur * 1e-9) / 1e12:.1f}")
        if mf:
            for cname, label in (("SQ_INSTS_VALU", "valu_per_mfma"), ("SQ_INSTS_LDS", "lds_per_mfma"),
                                 ("SQ_INSTS_SALU", "salu_per_mfma")):
                if cname in v:
                    lines.append(f"  {label:32s} {v[cname] / mf:.3f}")
        if fscale and wscale and "FETCH_SIZE" in v and "WRITE_SIZE" in v and dur:
            b = (v["FETCH_SIZE"] * fscale + v["WRITE_SIZE"] * wscale) * 1024.0
            lines.append(f"  {'hbm_bytes':32s} {b:.4g}")
            lines.append(f"  {'hbm_gbs':32s} {b / (dur * 1e-9) / 1e9:.1f}")
        lines.append("")
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, f"counters_{workload}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


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
    c = sub.add_parser("counters")
    c.add_argument("--workload", required=True)
    c.add_argument("--trace", required=True)
    c.add_argument("--pmc", nargs="+", required=True, help="one database per counter pass")
    c.add_argument("--commands", nargs="+", default=[])
    c.add_argument("--copy-mib", type=int, default=1024)
    c.add_argument("--out", default="profiles")
    c2 = sub.add_parser("passes", help="print the counter passes, one per line")
    sub.add_parser("hash")
    a = ap.parse_args()
    if a.cmd == "hash":
        print(source_hash())
    elif a.cmd == "passes":
        for p in COUNTER_PASSES:
            print(" ".join(p))
    elif a.cmd == "counters":
        print(counters_summary(a.workload, a.trace, a.pmc, a.commands, a.copy_mib, a.out))
    else:
        summarize(a.workload, a.trace, a.fetch, a.write, a.command, a.out, a.copy_mib,
                  a.fetch_command, a.write_command)


if __name__ == "__main__":
    main()
