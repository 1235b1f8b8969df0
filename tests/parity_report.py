"""Collects the errors the GPU parity checks measure, per problem, so that a
run can write them out (the environment variable BDATTN_PARITY_REPORT names
a JSON file; tests/conftest.py writes it at the end of the session).

Each record holds the problem's tag, the workload it belongs to (or None)
and the measured quantities: forward max-abs error, how many elements
exceed 1e-2, the output-rounding floor max |bf16(O_ref) - O_ref|, the LSE
error, and each gradient's max-abs error relative to max |g_ref|.
"""
from __future__ import annotations

import json
import os
from typing import Dict, List

RECORDS: List[Dict] = []


def record(kind: str, what: str, config, **values) -> None:
    rec = {"kind": kind, "what": what, "config": config}
    rec.update(values)
    RECORDS.append(rec)


def summarize(records=None) -> Dict[str, Dict]:
    """Per workload: the worst forward error, the elements above 1e-2 (and
    above the per-element bound), the worst output-rounding floor, the worst
    LSE error and the worst relative gradient errors."""
    out: Dict[str, Dict] = {}
    for r in records if records is not None else RECORDS:
        if r["config"] is None:
            continue
        s = out.setdefault(r["config"], {"fwd_max": 0.0, "above_1e-2": 0, "beyond_bound": 0, "floor_max": 0.0,
                                          "lse_max": 0.0, "elements": 0, "dq_rel": 0.0, "dk_rel": 0.0,
                                          "dv_rel": 0.0, "checks": 0})
        if r["kind"] == "fwd":
            s["fwd_max"] = max(s["fwd_max"], r["fwd_max"])
            s["above_1e-2"] += r["above_1e-2"]
            s["beyond_bound"] += r["beyond_bound"]
            s["floor_max"] = max(s["floor_max"], r["floor_max"])
            s["lse_max"] = max(s["lse_max"], r["lse_max"])
            s["elements"] += r["elements"]
            s["checks"] += 1
        else:
            key = r["name"] + "_rel"
            s[key] = max(s[key], r["rel"])
    return out


def write(path: str) -> None:
    d = os.path.dirname(path)
    if d:
        os.makedirs(d, exist_ok=True)
    with open(path, "w") as f:
        json.dump({"summary": summarize(), "records": RECORDS}, f, indent=1)
