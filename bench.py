#!/usr/bin/env python3
"""Benchmark of block-diffusion attention (forward + backward) on one MI355X.

One step is the whole hot path on one batch: the forward kernel, then the
two backward kernels (dQ, which also computes each row's delta and base-2
log-sum-exp, then dK/dV), all through the C ABI of libbdattn.so on torch's
current stream, with inputs resident in HBM.

Throughput counts visible (query, key) pairs only (Fast Diffusion
Attention, "The right yardstick"): 4 * pairs * headdim * heads * batch flops
for the forward pass and 2.5 times that for the backward pass.  The
yardstick is the library's own causal kernel on the same bytes viewed as 2B
sequences of n tokens, timed in interleaved rounds with the diffusion kernel
in one process and reported as medians (the pages' protocol for clocks that
follow power draw).

Prints one JSON line.  Default workload: the long-sequence problem
(B=2, n=8192, H=32, D=128, block size 32).  The grouped-query workloads
(g1..g3: query heads sharing key/value heads) also report the backward
time of the same kernels run ungrouped, on key/value heads repeated to H
(without the reduction of dK / dV over the group that this would still
need): the saving of the grouped backward (Fast Diffusion Attention,
"Ampere and Ada").
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import statistics
import sys
import time

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def visible_pairs(n: int, b: int) -> int:
    """n^2 + sum of squared block sizes ("The right yardstick": n^2 + n*b)."""
    full, rest = divmod(n, b)
    return n * n + full * b * b + rest * rest


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--rounds", type=int, default=5, help="interleaved diffusion/causal rounds")
    ap.add_argument("--round-ms", type=float, default=300.0, help="target duration of each phase of a round")
    ap.add_argument("--no-causal", action="store_true", help="skip the causal yardstick rounds")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time of the oracle's timed sample")
    ap.add_argument("--profiles", default=os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles"),
                    help="folder holding traffic_<kernel>_<workload>.txt (HBM bytes per launch)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def cpu_baseline(w, q, k, v, do, target_s=10.0, chunk=2048):
    """Time the float64 oracle (as it stands) on a bounded sample of the same
    workload: whole (sample, head) pairs, processed in chunks of query rows
    (forward and backward of each chunk against all 2n keys), until about
    target_s seconds of CPU work have been done."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = 1
    n, scale = w.n, 1.0 / math.sqrt(w.D)
    G = w.H // w.kv_heads
    pairs, chunks, heads = 0, 0, 0
    t_fwd = t_bwd = 0.0
    t_start = time.perf_counter()
    done = False
    for bi in range(w.B):
        for hi in range(w.H):
            qh, dh = oracle.to_f64(q[bi, :, hi]), oracle.to_f64(do[bi, :, hi])
            kh, vh = oracle.to_f64(k[bi, :, hi // G]), oracle.to_f64(v[bi, :, hi // G])
            for r0 in range(0, 2 * n, chunk):
                rows = np.arange(r0, min(r0 + chunk, 2 * n))
                M = oracle.block_diffusion_mask(n, w.b, rows)
                pairs += int(M.sum())
                t0 = time.perf_counter()
                oracle.masked_attention_forward(qh[rows], kh, vh, M, scale)
                t1 = time.perf_counter()
                oracle.masked_attention_backward(qh[rows], kh, vh, dh[rows], M, scale)
                t2 = time.perf_counter()
                t_fwd += t1 - t0
                t_bwd += t2 - t1
                chunks += 1
                if time.perf_counter() - t_start >= target_s and r0 + chunk >= 2 * n:
                    done = True
                    break
            heads += 1
            if done:
                break
        if done:
            break
    flops = 3.5 * 4 * pairs * w.D
    return {
        "value": flops / (t_fwd + t_bwd) / 1e12,
        "unit": "TFLOPS",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"float64 oracle forward + backward of {heads} whole (sample, head) pair(s) of {w.name} "
                   f"({chunks} chunks of {chunk} query rows against all {2 * n} keys; {pairs} visible pairs); "
                   f"{t_fwd:.1f} s forward + {t_bwd:.1f} s backward; BLAS threads {cores}; "
                   f"host {platform.processor() or platform.machine()}"),
    }


class ClockSampler:
    """Polls the GPU's graphics clock (amdsmi, SYS clock, MHz) from a
    background thread while kernels run: the rates above are only comparable
    at known clocks.  Reports None where amdsmi is unavailable."""

    def __init__(self, period_s: float = 0.005):
        import threading
        self.samples = []
        self.period = period_s
        self.handle = None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if handles:
                self.amdsmi = amdsmi
                self.handle = handles[0]
                self.read()
        except Exception:
            self.handle = None

    def read(self):
        info = self.amdsmi.amdsmi_get_clock_info(self.handle, self.amdsmi.AmdSmiClkType.SYS)
        return float(info["clk"])

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self.read())
            except Exception:
                return
            self._stop.wait(self.period)

    def start(self):
        import threading
        if self.handle is None:
            return
        self._stop.clear()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join(timeout=1.0)
            self._thread = None

    def summary(self):
        if not self.samples:
            return None
        return {"median_mhz": statistics.median(self.samples), "min_mhz": min(self.samples),
                "max_mhz": max(self.samples), "samples": len(self.samples), "source": "amdsmi SYS clock"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(the attention of every (sample, head) is independent; see the design notes "
              "for how it would shard).", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_diffusion_lm_amd as bd
    from workloads import GQA_WORKLOADS, WORKLOADS, make_workload_inputs

    all_workloads = {**WORKLOADS, **GQA_WORKLOADS}
    if args.workload not in all_workloads:
        print(f"unknown workload {args.workload!r}; known: {', '.join(all_workloads)}", file=sys.stderr)
        sys.exit(2)
    w = all_workloads[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, n, H, Hkv, D, b = w.B, w.n, w.H, w.kv_heads, w.D, w.b
    T = 2 * n
    scale = 1.0 / math.sqrt(D)

    q_c, k_c, v_c, do_c = make_workload_inputs(w)
    q, k, v, do = (x.to(dev) for x in (q_c, k_c, v_c, do_c))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dq = torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws_bytes = bd.diffusion_attn_bwd_gqa_workspace_size(B, n, H, Hkv, D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    # causal yardstick: the same bytes as 2B sequences of n tokens
    cq, cdo = (x.view(2 * B, n, H, D) for x in (q, do))
    ck, cv = (x.view(2 * B, n, Hkv, D) for x in (k, v))
    cout = torch.empty_like(cq)
    clse = torch.empty((2 * B, H, n), dtype=torch.float32, device=dev)
    cdq = torch.empty_like(cq)
    cdk, cdv = torch.empty_like(ck), torch.empty_like(cv)
    cws = torch.empty(bd.causal_attn_bwd_gqa_workspace_size(2 * B, n, H, Hkv, D), dtype=torch.uint8,
                      device=dev)

    MD, MC = bd.MODE_DIFFUSION, bd.MODE_CAUSAL

    def fwd_diffusion():
        if Hkv == H:
            bd.diffusion_attn_fwd(q, k, v, out, lse, B, n, H, D, b, scale)
        else:
            bd.diffusion_attn_fwd_gqa(q, k, v, out, lse, B, n, H, Hkv, D, b, scale)

    def fwd_causal():
        if Hkv == H:
            bd.causal_attn_fwd(cq, ck, cv, cout, clse, 2 * B, n, H, D, scale)
        else:
            bd.causal_attn_fwd_gqa(cq, ck, cv, cout, clse, 2 * B, n, H, Hkv, D, scale)

    def diffusion_step(ev=None):
        if ev is not None:
            ev[0].record()
        fwd_diffusion()
        if ev is not None:
            ev[1].record()
        for stage in range(2):
            bd.bdattn_bwd_stage(MD, stage, q, k, v, out, do, lse, dq, dk, dv, B, n, H, Hkv, D, b, scale,
                                ws, ws_bytes)
            if ev is not None:
                ev[2 + stage].record()

    def causal_step(ev=None):
        if ev is not None:
            ev[0].record()
        fwd_causal()
        if ev is not None:
            ev[1].record()
        for stage in range(2):
            bd.bdattn_bwd_stage(MC, stage, cq, ck, cv, cout, cdo, clse, cdq, cdk, cdv, 2 * B, n, H, Hkv,
                                D, 1, scale, cws)
            if ev is not None:
                ev[2 + stage].record()

    def new_events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    # ---- warm-up, then exactly K timed steps --------------------------------
    for _ in range(args.warmup):
        diffusion_step()
    torch.cuda.synchronize()
    evs = [new_events() for _ in range(args.steps)]
    clock = ClockSampler()
    torch.cuda.synchronize()
    clock.start()
    t0 = time.perf_counter()
    for i in range(args.steps):
        diffusion_step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock.stop()
    ms_per_step = wall * 1e3 / args.steps

    def split(ev_list):
        per = {"fwd": [], "bwd_dq": [], "bwd_dkdv": []}
        for ev in ev_list:
            per["fwd"].append(ev[0].elapsed_time(ev[1]))
            per["bwd_dq"].append(ev[1].elapsed_time(ev[2]))
            per["bwd_dkdv"].append(ev[2].elapsed_time(ev[3]))
        return per

    kern = split(evs)
    kern_avg = {key: sum(vals) / len(vals) for key, vals in kern.items()}

    P = visible_pairs(n, b)
    assert P == bd.bdattn_visible_pairs(MD, n, b)
    F_fwd = 4.0 * P * D * H * B
    F_bwd = 2.5 * F_fwd
    value = (F_fwd + F_bwd) / (ms_per_step * 1e-3) / 1e12
    t_fwd = kern_avg["fwd"]
    t_bwd = kern_avg["bwd_dq"] + kern_avg["bwd_dkdv"]

    # ---- the dominant kernel against its roofline ---------------------------
    per_kernel_flops = {"fwd": 2 * 2.0 * P * D * H * B,        # S = QK^T, O = PV
                        "bwd_dkdv": 4 * 2.0 * P * D * H * B,   # S, dP, dV, dK
                        "bwd_dq": 3 * 2.0 * P * D * H * B}     # S, dP, dQ
    dom = max(per_kernel_flops, key=lambda kname: kern_avg[kname])
    achieved = per_kernel_flops[dom] / (kern_avg[dom] * 1e-3) / 1e12
    # HBM bytes per launch from the rocprofv3 counter runs, valid only while
    # the kernel sources are the ones the counters were taken on
    from block_diffusion_lm_amd import profiling
    traffic = None
    tr = profiling.read_traffic(os.path.join(args.profiles, f"traffic_{dom}_{w.name}.txt"))
    if tr and tr.get("source_sha256") == profiling.source_hash():
        traffic = float(tr["bytes_per_launch"])
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic, "kernel": dom,
                "algorithmic_flops_per_launch": per_kernel_flops[dom],
                "avg_launch_ms": kern_avg[dom]}

    # ---- interleaved rounds against the causal yardstick --------------------
    ratio = None
    medians = None
    if not args.no_causal:
        for _ in range(2):
            causal_step()
        torch.cuda.synchronize()
        reps = max(1, int(math.ceil(args.round_ms / max(ms_per_step, 1e-3))))
        rounds = {"diff": [], "causal": []}
        clock.start()
        for _ in range(args.rounds):
            for name, fn in (("diff", diffusion_step), ("causal", causal_step)):
                ev_list = [new_events() for _ in range(reps)]
                for i in range(reps):
                    fn(ev_list[i])
                torch.cuda.synchronize()
                per = split(ev_list)
                f = sum(per["fwd"]) / reps
                bwd = sum(per["bwd_dq"][i] + per["bwd_dkdv"][i] for i in range(reps)) / reps
                rounds[name].append((f, bwd))
        clock.stop()
        med = {name: (statistics.median(x[0] for x in r), statistics.median(x[1] for x in r),
                      statistics.median(x[0] + x[1] for x in r)) for name, r in rounds.items()}
        Pc = n * (n + 1) // 2
        Fc_fwd = 4.0 * Pc * D * H * (2 * B)
        tf = lambda F, ms: F / (ms * 1e-3) / 1e12
        medians = {
            "diffusion_tflops": {"fwd": tf(F_fwd, med["diff"][0]), "bwd": tf(F_bwd, med["diff"][1]),
                                 "step": tf(F_fwd + F_bwd, med["diff"][2])},
            "causal_tflops": {"fwd": tf(Fc_fwd, med["causal"][0]), "bwd": tf(2.5 * Fc_fwd, med["causal"][1]),
                              "step": tf(3.5 * Fc_fwd, med["causal"][2])},
            "reps_per_phase": reps, "rounds": args.rounds,
        }
        ratio = {kname: medians["diffusion_tflops"][kname] / medians["causal_tflops"][kname]
                 for kname in ("fwd", "bwd", "step")}

    # ---- grouped-query workloads: the backward run ungrouped ----------------
    ungrouped = None
    if Hkv != H:
        G = H // Hkv
        ek, ev_ = (x.repeat_interleave(G, dim=2).contiguous() for x in (k, v))
        edk, edv = torch.empty_like(q), torch.empty_like(q)
        times = {"grouped": [], "ungrouped": []}
        for _ in range(3):
            for name, kk, vv, gk, gv, hk in (("grouped", k, v, dk, dv, Hkv), ("ungrouped", ek, ev_, edk, edv, H)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 5
                e0.record()
                for _ in range(reps):
                    for stage in range(2):
                        bd.bdattn_bwd_stage(MD, stage, q, kk, vv, out, do, lse, dq, gk, gv, B, n, H, hk, D, b,
                                            scale, ws, ws_bytes)
                e1.record()
                torch.cuda.synchronize()
                times[name].append(e0.elapsed_time(e1) / reps)
        med = {name: statistics.median(x) for name, x in times.items()}
        ungrouped = {"bwd_ms_grouped": med["grouped"], "bwd_ms_ungrouped": med["ungrouped"],
                     "speedup": med["ungrouped"] / med["grouped"],
                     "note": "ungrouped = the same kernels on key/value heads repeated to H, "
                             "without the dK/dV reduction over the group"}
        del ek, ev_, edk, edv

    if args.copy_calibration_mib > 0:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, q_c, k_c, v_c, do_c, args.cpu_seconds)

    line = {
        "metric": "fwd+bwd TFLOPS (visible pairs only) and ratio vs own causal kernel on 2B×n",
        "value": value,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.describe(), "global_batch": B, "seq_len": T, "block_size": b,
                   "heads": H, "kv_heads": Hkv, "headdim": D, "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fwd_tflops": F_fwd / (t_fwd * 1e-3) / 1e12,
        "bwd_tflops": F_bwd / (t_bwd * 1e-3) / 1e12,
        "frac_of_peak": value / PEAK_BF16_TFLOPS,
        "ratio_vs_causal": ratio,
        "interleaved_medians": medians,
        "kernel_avg_ms": kern_avg,
        "device": torch.cuda.get_device_name(dev),
        "sclk": clock.summary(),
    }
    if ungrouped is not None:
        line["grouped_backward"] = ungrouped
    print(json.dumps(line))


if __name__ == "__main__":
    main()
