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
"Ampere and Ada").  The packed workloads (v1, v2: samples of random
lengths) count the visible pairs of every sample, and their yardstick is
the causal kernel on the same packed bytes, each half of each sample one
sequence.
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
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_SCLK_MHZ = 2400.0      # the engine clock the MFMA peaks are quoted at


def at_clock(roofline, sclk):
    """Add the peak scaled to the median graphics clock sampled during the
    run, and the fraction of it: the chip is power-capped under this load and
    runs well below the clock the published peak assumes."""
    if sclk and sclk.get("median_mhz"):
        peak = roofline["peak"] * sclk["median_mhz"] / PEAK_SCLK_MHZ
        roofline["peak_at_median_sclk"] = peak
        roofline["frac_at_median_sclk"] = roofline["achieved"] / peak
    return roofline


def visible_pairs(n: int, b: int) -> int:
    """n^2 + sum of squared block sizes ("The right yardstick": n^2 + n*b)."""
    full, rest = divmod(n, b)
    return n * n + full * b * b + rest * rest


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 35 steps of the default workload take about 330 ms: the warm-up and the
    # timed region each last at least 300 ms, so that a power-capped clock has
    # settled before timing (Fast Diffusion Attention, "Measuring on
    # power-capped GPUs")
    ap.add_argument("--steps", type=int, default=35)
    ap.add_argument("--warmup", type=int, default=35)
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
    ap.add_argument("--softcap", type=float, default=0.0,
                    help="cap the scores to softcap * tanh(s / softcap) (batched workloads; 0: off)")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 (E4M3) forward pass instead (batched workloads)")
    return ap.parse_args()


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _oracle_chunk(task):
    """One unit of the CPU baseline, run in a worker process with one BLAS
    thread: the oracle's forward and backward of query rows [r0, r1) of one
    (sample, head) against all 2n keys.  q, k, v, dout arrive as the bf16
    bit patterns (uint16)."""
    import numpy as np
    import torch
    import oracle
    from threadpoolctl import threadpool_limits
    qb, kb, vb, db, n, b, r0, r1 = task
    with threadpool_limits(1):
        qh, kh, vh, dh = (oracle.to_f64(torch.from_numpy(x).view(torch.bfloat16)) for x in (qb, kb, vb, db))
        scale = 1.0 / math.sqrt(qh.shape[1])
        rows = np.arange(r0, r1)
        M = oracle.block_diffusion_mask(n, b, rows)
        t0 = time.perf_counter()
        oracle.masked_attention_forward(qh[rows], kh, vh, M, scale)
        t1 = time.perf_counter()
        oracle.masked_attention_backward(qh[rows], kh, vh, dh[rows], M, scale)
        t2 = time.perf_counter()
    return int(M.sum()), t1 - t0, t2 - t1


def cpu_baseline(heads, name, target_s=10.0, chunk=2048):
    """Time the float64 oracle (as it stands) on a bounded sample of the same
    workload, on every host core: a pool of len(os.sched_getaffinity(0))
    worker processes, one BLAS thread each, takes chunks of query rows of
    whole (sample, head) problems (forward and backward of each chunk
    against all keys of its sample) in the order ``heads`` yields them (q,
    k, v, dout of one head as bf16 CPU tensors, the half length n and the
    block size b), until about target_s seconds of wall time have passed.
    The rate is the chunks' visible-pair flops (3.5 x 4 x pairs x D) over
    the wall time of the pool.  Runs before anything touches the GPU: the
    workers are started fresh ("spawn"), never from a process holding GPU
    state."""
    import concurrent.futures
    import multiprocessing

    cores = len(os.sched_getaffinity(0))

    def tasks():
        for qh, kh, vh, dh, n, b in heads:
            bits = tuple(x.contiguous().view(__import__("torch").int16).numpy().view("uint16")
                         for x in (qh, kh, vh, dh))
            for r0 in range(0, 2 * n, chunk):
                yield bits + (n, b, r0, min(r0 + chunk, 2 * n)), qh.shape[1]

    it = tasks()
    pairs = flops = chunks = 0
    t_fwd = t_bwd = 0.0
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(cores, mp_context=ctx) as ex:
        ex.submit(int, 0).result()  # workers up before the clock starts
        t_start = time.perf_counter()
        running = {}
        for _ in range(cores):
            nxt = next(it, None)
            if nxt is not None:
                running[ex.submit(_oracle_chunk, nxt[0])] = nxt[1]
        while running:
            done, _ = concurrent.futures.wait(running, return_when=concurrent.futures.FIRST_COMPLETED)
            for fut in done:
                D = running.pop(fut)
                p, tf, tb = fut.result()
                pairs += p
                flops += 3.5 * 4 * p * D
                t_fwd += tf
                t_bwd += tb
                chunks += 1
                if time.perf_counter() - t_start < target_s:
                    nxt = next(it, None)
                    if nxt is not None:
                        running[ex.submit(_oracle_chunk, nxt[0])] = nxt[1]
        wall = time.perf_counter() - t_start
    return {
        "value": flops / wall / 1e12,
        "unit": "TFLOPS",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"float64 oracle forward + backward of {chunks} chunks of up to {chunk} query rows of {name} "
                   f"(each against all keys of its sample; {pairs} visible pairs), whole (sample, head) "
                   f"problems in order; {cores} worker processes, one BLAS thread each, {wall:.1f} s wall "
                   f"({t_fwd:.1f} s forward + {t_bwd:.1f} s backward of worker time); CPU {_cpu_model()}"),
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


class Problem:
    """The timed work of one workload: a diffusion step and the causal
    yardstick step on the same bytes, with their visible-pair counts."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def new_events(torch):
    return [torch.cuda.Event(enable_timing=True) for _ in range(4)]


def mark(ev, i):
    """Record event i of a step: 0 before the forward, 1 after it, 2 after dQ, 3 after dK/dV."""
    if ev is not None:
        ev[i].record()


def cpu_inputs(w):
    """The workload's seeded CPU tensors (q, k, v, dout[, cu_seqlens])."""
    from workloads import VARLEN_WORKLOADS, make_varlen_workload_inputs, make_workload_inputs
    if w.name in VARLEN_WORKLOADS:
        return make_varlen_workload_inputs(w)
    return make_workload_inputs(w)


def cpu_heads(w, cpu):
    """(q, k, v, dout, n, b) of each (sample, head) of the CPU inputs; packed
    samples longest first."""
    from workloads import VARLEN_WORKLOADS
    G = w.H // w.kv_heads
    if w.name in VARLEN_WORKLOADS:
        ns, cu = w.half_lengths, cpu[4]
        for bi in sorted(range(w.B), key=lambda i: -ns[i]):
            s0, s1 = cu[bi], cu[bi + 1]
            for hi in range(w.H):
                yield (cpu[0][s0:s1, hi], cpu[1][s0:s1, hi // G], cpu[2][s0:s1, hi // G], cpu[3][s0:s1, hi],
                       ns[bi], w.b)
        return
    for bi in range(w.B):
        for hi in range(w.H):
            yield cpu[0][bi, :, hi], cpu[1][bi, :, hi // G], cpu[2][bi, :, hi // G], cpu[3][bi, :, hi], w.n, w.b


def setup_batched(w, dev, torch, bd, cpu, softcap=0.0):
    """(B, 2n, H, D) tensors; the yardstick views them as (2B, n, H, D).
    softcap > 0 runs both through the general entry points with that cap."""
    B, n, H, Hkv, D, b = w.B, w.n, w.H, w.kv_heads, w.D, w.b
    scale = 1.0 / math.sqrt(D)
    q, k, v, do = (x.to(dev) for x in cpu)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, 2 * n), dtype=torch.float32, device=dev)
    dq = torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws_bytes = bd.diffusion_attn_bwd_gqa_workspace_size(B, n, H, Hkv, D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    cq, cdo = (x.view(2 * B, n, H, D) for x in (q, do))
    ck, cv = (x.view(2 * B, n, Hkv, D) for x in (k, v))
    cout = torch.empty_like(cq)
    clse = torch.empty((2 * B, H, n), dtype=torch.float32, device=dev)
    cdq = torch.empty_like(cq)
    cdk, cdv = torch.empty_like(ck), torch.empty_like(cv)
    cws = torch.empty(bd.causal_attn_bwd_gqa_workspace_size(2 * B, n, H, Hkv, D), dtype=torch.uint8,
                      device=dev)
    MD, MC = bd.MODE_DIFFUSION, bd.MODE_CAUSAL

    def diffusion_step(ev=None):
        mark(ev, 0)
        if softcap:
            bd.bdattn_fwd(MD, q, k, v, out, lse, None, B, n, 0, H, Hkv, D, b, scale, softcap)
        elif Hkv == H:
            bd.diffusion_attn_fwd(q, k, v, out, lse, B, n, H, D, b, scale)
        else:
            bd.diffusion_attn_fwd_gqa(q, k, v, out, lse, B, n, H, Hkv, D, b, scale)
        mark(ev, 1)
        for stage in range(2):
            bd.bdattn_bwd_stage(MD, stage, q, k, v, out, do, lse, dq, dk, dv, None, B, n, 0, H, Hkv, D, b,
                                scale, softcap, ws, ws_bytes)
            mark(ev, 2 + stage)

    def causal_step(ev=None):
        mark(ev, 0)
        if softcap:
            bd.bdattn_fwd(MC, cq, ck, cv, cout, clse, None, 2 * B, n, 0, H, Hkv, D, 1, scale, softcap)
        elif Hkv == H:
            bd.causal_attn_fwd(cq, ck, cv, cout, clse, 2 * B, n, H, D, scale)
        else:
            bd.causal_attn_fwd_gqa(cq, ck, cv, cout, clse, 2 * B, n, H, Hkv, D, scale)
        mark(ev, 1)
        for stage in range(2):
            bd.bdattn_bwd_stage(MC, stage, cq, ck, cv, cout, cdo, clse, cdq, cdk, cdv, None, 2 * B, n, 0,
                                H, Hkv, D, 1, scale, softcap, cws)
            mark(ev, 2 + stage)

    def ungrouped():
        """Backward of the same kernels on key/value heads repeated to H."""
        if Hkv == H:
            return None
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
                        bd.bdattn_bwd_stage(MD, stage, q, kk, vv, out, do, lse, dq, gk, gv, None, B, n, 0, H,
                                            hk, D, b, scale, 0.0, ws, ws_bytes)
                e1.record()
                torch.cuda.synchronize()
                times[name].append(e0.elapsed_time(e1) / reps)
        med = {name: statistics.median(x) for name, x in times.items()}
        return {"bwd_ms_grouped": med["grouped"], "bwd_ms_ungrouped": med["ungrouped"],
                "speedup": med["ungrouped"] / med["grouped"],
                "note": "ungrouped = the same kernels on key/value heads repeated to H, "
                        "without the dK/dV reduction over the group"}

    P = visible_pairs(n, b)
    assert P == bd.bdattn_visible_pairs(MD, n, b)
    return Problem(diffusion_step=diffusion_step, causal_step=causal_step, ungrouped=ungrouped,
                   pair_heads=P * H * B, causal_pair_heads=n * (n + 1) // 2 * H * 2 * B,
                   config={"workload": w.describe(), "global_batch": B, "seq_len": 2 * n, "block_size": b,
                           "heads": H, "kv_heads": Hkv, "headdim": D, "softcap": softcap,
                           "parallelism": "single-gpu"})


def setup_varlen(w, dev, torch, bd, cpu):
    """Packed samples of random lengths; the yardstick packs the same bytes
    as 2B causal sequences (each half of each sample)."""
    from workloads import cu_seqlens
    ns = w.half_lengths
    B, H, Hkv, D, b = w.B, w.H, w.kv_heads, w.D, w.b
    max_n = max(ns)
    scale = 1.0 / math.sqrt(D)
    q, k, v, do = (x.to(dev) for x in cpu[:4])
    cu = cpu[4]
    total = cu[-1]
    cu_t = torch.tensor(cu, dtype=torch.int32, device=dev)
    ccu_t = torch.tensor(cu_seqlens([x for nb in ns for x in (nb, nb)], causal=True), dtype=torch.int32,
                         device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device=dev)
    dq = torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws_bytes = bd.diffusion_attn_varlen_bwd_workspace_size(B, max_n, total, H, Hkv, D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    cout = torch.empty_like(q)
    clse = torch.empty((H, total), dtype=torch.float32, device=dev)
    cdq = torch.empty_like(q)
    cdk, cdv = torch.empty_like(k), torch.empty_like(v)
    cws_bytes = bd.causal_attn_varlen_bwd_workspace_size(2 * B, max_n, total, H, Hkv, D)
    cws = torch.empty(cws_bytes, dtype=torch.uint8, device=dev)
    MD, MC = bd.MODE_DIFFUSION, bd.MODE_CAUSAL

    def diffusion_step(ev=None):
        mark(ev, 0)
        bd.diffusion_attn_varlen_fwd(q, k, v, out, lse, cu_t, B, max_n, total, H, Hkv, D, b, scale)
        mark(ev, 1)
        for stage in range(2):
            bd.bdattn_bwd_stage(MD, stage, q, k, v, out, do, lse, dq, dk, dv, cu_t, B, max_n, total, H, Hkv,
                                D, b, scale, 0.0, ws, ws_bytes)
            mark(ev, 2 + stage)

    def causal_step(ev=None):
        mark(ev, 0)
        bd.causal_attn_varlen_fwd(q, k, v, cout, clse, ccu_t, 2 * B, max_n, total, H, Hkv, D, scale)
        mark(ev, 1)
        for stage in range(2):
            bd.bdattn_bwd_stage(MC, stage, q, k, v, cout, do, clse, cdq, cdk, cdv, ccu_t, 2 * B, max_n, total,
                                H, Hkv, D, 1, scale, 0.0, cws, cws_bytes)
            mark(ev, 2 + stage)

    P = sum(visible_pairs(nb, b) for nb in ns if nb > 0)
    return Problem(diffusion_step=diffusion_step, causal_step=causal_step, ungrouped=lambda: None,
                   pair_heads=P * H,
                   causal_pair_heads=sum(nb * (nb + 1) for nb in ns) * H,
                   config={"workload": w.describe(), "global_batch": B, "seq_len": 2 * max_n,
                           "total_tokens": total, "block_size": b, "heads": H, "kv_heads": Hkv,
                           "headdim": D, "parallelism": "single-gpu"})


def bench_fp8(args, w, dev, torch, bd):
    """The FP8 forward on a batched workload: its rate, its FP8 causal
    yardstick (interleaved rounds, medians) and the bf16 forward on the
    same shapes."""
    from workloads import make_fp8_inputs, make_workload_inputs
    B, n, H, Hkv, D, b = w.B, w.n, w.H, w.kv_heads, w.D, w.b
    scale = 1.0 / math.sqrt(D)
    q8, k8, v8, qd, kd, vd = (x.to(dev) for x in make_fp8_inputs(B, n, H, D, w.seed, H_kv=w.H_kv))
    out = torch.empty((B, 2 * n, H, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, 2 * n), dtype=torch.float32, device=dev)
    cq, ck, cv = q8.view(2 * B, n, H, D), k8.view(2 * B, n, Hkv, D), v8.view(2 * B, n, Hkv, D)
    cqd, ckd, cvd = (x.repeat_interleave(2, dim=0).contiguous() for x in (qd, kd, vd))
    cout = torch.empty((2 * B, n, H, D), dtype=torch.bfloat16, device=dev)
    clse = torch.empty((2 * B, H, n), dtype=torch.float32, device=dev)
    q, k, v, _ = (x.to(dev) if x is not None else None for x in make_workload_inputs(w, with_dout=False))

    def fp8_fwd():
        bd.diffusion_attn_fwd_fp8(q8, k8, v8, qd, kd, vd, out, lse, B, n, H, Hkv, D, b, scale)

    def fp8_causal():
        bd.causal_attn_fwd_fp8(cq, ck, cv, cqd, ckd, cvd, cout, clse, 2 * B, n, H, Hkv, D, scale)

    def bf16_fwd():
        if Hkv == H:
            bd.diffusion_attn_fwd(q, k, v, out, lse, B, n, H, D, b, scale)
        else:
            bd.diffusion_attn_fwd_gqa(q, k, v, out, lse, B, n, H, Hkv, D, b, scale)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for fn in (fp8_fwd, fp8_causal, bf16_fwd):
        for _ in range(args.warmup):
            fn()
    torch.cuda.synchronize()
    clock = ClockSampler()
    clock.start()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fp8_fwd()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_event = timed(fp8_fwd, args.steps)
    reps = max(1, int(math.ceil(args.round_ms / max(ms, 1e-3))))
    rounds = {"fp8": [], "fp8_causal": [], "bf16": []}
    for _ in range(args.rounds):
        for name, fn in (("fp8", fp8_fwd), ("fp8_causal", fp8_causal), ("bf16", bf16_fwd)):
            rounds[name].append(timed(fn, reps))
    clock.stop()
    med = {name: statistics.median(x) for name, x in rounds.items()}
    P = visible_pairs(n, b)
    F = 4.0 * P * D * H * B
    Fc = 4.0 * (n * (n + 1) // 2) * D * H * 2 * B
    tf = lambda F_, ms_: F_ / (ms_ * 1e-3) / 1e12
    achieved = tf(F, ms_event)
    return {
        "metric": "FP8 forward TFLOPS (visible pairs only)",
        "value": tf(F, ms),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.describe(), "global_batch": B, "seq_len": 2 * n, "block_size": b,
                   "heads": H, "kv_heads": Hkv, "headdim": D, "parallelism": "single-gpu"},
        "roofline": at_clock({"bound": "mfma", "achieved": achieved, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                              "frac": achieved / PEAK_FP8_TFLOPS, "traffic": None, "kernel": "fwd_fp8",
                              "algorithmic_flops_per_launch": F, "avg_launch_ms": ms_event}, clock.summary()),
        "interleaved_medians_ms": med,
        "ratio_vs_causal": tf(F, med["fp8"]) / tf(Fc, med["fp8_causal"]),
        "speedup_vs_bf16_forward": med["bf16"] / med["fp8"],
        "device": torch.cuda.get_device_name(dev),
        "sclk": clock.summary(),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: there is no multi-GPU path (the attention "
              "of every (sample, head) is independent, so batch or head shards would need no "
              "communication inside attention).", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_diffusion_lm_amd as bd
    from workloads import GQA_WORKLOADS, HEAD_DIM_WORKLOADS, VARLEN_WORKLOADS, WORKLOADS

    batched = {**WORKLOADS, **GQA_WORKLOADS, **HEAD_DIM_WORKLOADS}
    if args.workload in batched:
        w, setup = batched[args.workload], setup_batched
    elif args.workload in VARLEN_WORKLOADS:
        w, setup = VARLEN_WORKLOADS[args.workload], setup_varlen
    else:
        known = ", ".join(list(batched) + list(VARLEN_WORKLOADS))
        print(f"unknown workload {args.workload!r}; known: {known}", file=sys.stderr)
        sys.exit(2)
    # The CPU baseline runs first: its worker processes start before anything
    # in this process touches the GPU.
    cpu = None
    inputs = None
    if not args.fp8:
        inputs = cpu_inputs(w)
        if not args.no_cpu_baseline:
            cpu = cpu_baseline(cpu_heads(w, inputs), w.name, args.cpu_seconds)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.fp8:
        if setup is not setup_batched:
            print("--fp8 takes a batched workload", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(bench_fp8(args, w, dev, torch, bd)))
        return
    if args.softcap and setup is not setup_batched:
        print("--softcap takes a batched workload", file=sys.stderr)
        sys.exit(2)
    prob = setup_batched(w, dev, torch, bd, inputs, args.softcap) if args.softcap else setup(w, dev, torch, bd, inputs)
    D = w.D

    # ---- warm-up, then exactly K timed steps --------------------------------
    for _ in range(args.warmup):
        prob.diffusion_step()
    torch.cuda.synchronize()
    evs = [new_events(torch) for _ in range(args.steps)]
    clock = ClockSampler()
    torch.cuda.synchronize()
    clock.start()
    t0 = time.perf_counter()
    for i in range(args.steps):
        prob.diffusion_step(evs[i])
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

    PH = prob.pair_heads          # visible (query, key) pairs summed over samples and heads
    F_fwd = 4.0 * PH * D
    F_bwd = 2.5 * F_fwd
    value = (F_fwd + F_bwd) / (ms_per_step * 1e-3) / 1e12
    t_fwd = kern_avg["fwd"]
    t_bwd = kern_avg["bwd_dq"] + kern_avg["bwd_dkdv"]

    # ---- the dominant kernel against its roofline ---------------------------
    per_kernel_flops = {"fwd": 2 * 2.0 * PH * D,        # S = QK^T, O = PV
                        "bwd_dkdv": 4 * 2.0 * PH * D,   # S, dP, dV, dK
                        "bwd_dq": 3 * 2.0 * PH * D}     # S, dP, dQ
    dom = max(per_kernel_flops, key=lambda kname: kern_avg[kname])
    achieved = per_kernel_flops[dom] / (kern_avg[dom] * 1e-3) / 1e12
    # HBM bytes per launch from the rocprofv3 counter runs, valid only while
    # the kernel sources are the ones the counters were taken on
    from block_diffusion_lm_amd import profiling
    traffic = None
    tr = profiling.read_traffic(os.path.join(args.profiles, f"traffic_{dom}_{w.name}.txt"))
    if tr and tr.get("source_sha256") == profiling.source_hash(dom):
        traffic = float(tr["bytes_per_launch"])
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic, "kernel": dom,
                "algorithmic_flops_per_launch": per_kernel_flops[dom],
                "avg_launch_ms": kern_avg[dom]}
    # MFMA- and vector-busy shares and clock of each kernel from the committed counter
    # runs, while the kernel sources are the ones they were taken on
    ctr = profiling.read_counters(os.path.join(args.profiles, f"counters_{w.name}.txt"))
    if ctr and ctr.get("source_sha256") == profiling.source_hash():
        roofline["mfma_busy"] = {k: v.get("mfma_busy") for k, v in ctr.items() if isinstance(v, dict)}
        roofline["valu_busy"] = {k: v.get("valu_busy") for k, v in ctr.items() if isinstance(v, dict)}
        roofline["counter_clock_mhz"] = {k: v.get("clock_mhz") for k, v in ctr.items() if isinstance(v, dict)}

    # ---- interleaved rounds against the causal yardstick --------------------
    ratio = None
    medians = None
    if not args.no_causal:
        for _ in range(2):
            prob.causal_step()
        torch.cuda.synchronize()
        reps = max(1, int(math.ceil(args.round_ms / max(ms_per_step, 1e-3))))
        rounds = {"diff": [], "causal": []}
        clock.start()
        for _ in range(args.rounds):
            for name, fn in (("diff", prob.diffusion_step), ("causal", prob.causal_step)):
                ev_list = [new_events(torch) for _ in range(reps)]
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
        Fc_fwd = 4.0 * prob.causal_pair_heads * D
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

    ungrouped = prob.ungrouped()

    if args.copy_calibration_mib > 0:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

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
        "config": prob.config,
        "roofline": at_clock(roofline, clock.summary()),
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
