"""GPU parity: the HIP path (called through the C ABI) against the float64
oracle, on identical seeded bf16 inputs.

Tolerances (the stated targets for bf16 inputs with fp32 accumulation):
  * forward output: every element within max(1e-2, halfulp_bf16(O_ref) +
    1e-3).  For |O_ref| < 4 that is the flat 1e-2; above, rounding the
    exact output to bf16 alone can cost half an ulp (2^-6 for |O| in
    [4, 8)), more than 1e-2, so such an element may be off by that floor
    plus 1e-3 of float32 accumulation.  Every check records the largest
    error, the count of elements above 1e-2 and the floor
    max |bf16(O_ref) - O_ref| (tests/parity_report.py);
  * log-sum-exp: max |LSE - LSE_ref| <= 1e-3;
  * dq, dk, dv: max |g - g_ref| <= 2e-2 * max |g_ref|; when the exact
    gradient is identically zero (a half of one token: every row sees only
    itself, P = 1, dS = 0) the relative bound is 0, and an absolute 1e-5
    (far below one bf16 ulp of any nonzero gradient here) is used instead.
Scales other than +-1/sqrt(D) (the only ones the workloads use) are held
to check_fwd_rounding's bound instead (see there).
Small problems are compared in full.  The full-size workloads run exactly
as the benchmark launches them (every sample and head on the GPU); the
oracle then checks whole heads (all rows of O and LSE), sampled rows and
key columns of every (sample, head), and, for the largest problem, sampled
rows of dQ and sampled key columns of dK / dV of two whole heads.
"""
import functools
import math
import os

import numpy as np
import pytest
import torch

import oracle
import parity_report
import block_diffusion_lm_amd as bd
from workloads import (GQA_WORKLOADS, HEAD_DIM_WORKLOADS, VARLEN_WORKLOADS, WORKLOADS,
                       make_causal_view, make_fp8_inputs, make_fp8_integer_score_inputs, make_inputs,
                       make_varlen_inputs, make_varlen_workload_inputs, make_workload_inputs)

pytestmark = pytest.mark.gpu

FWD_TOL, LSE_TOL, GRAD_REL = 1e-2, 1e-3, 2e-2
ZERO_GRAD_ABS = 1e-5


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_diffusion(q, k, v, do, b, scale, bwd=True):
    """One forward (and backward) through the C ABI; returns CPU tensors."""
    dev = _dev()
    B, T, H, D = q.shape
    n = T // 2
    q, k, v = (x.to(dev) for x in (q, k, v))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    bd.diffusion_attn_fwd(q, k, v, out, lse, B, n, H, D, b, scale)
    res = {"out": out, "lse": lse}
    if bwd:
        do = do.to(dev)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        ws = torch.empty(bd.diffusion_attn_bwd_workspace_size(B, n, H, D), dtype=torch.uint8, device=dev)
        bd.diffusion_attn_bwd(q, k, v, out, do, lse, dq, dk, dv, B, n, H, D, b, scale, ws)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {key: t.cpu() for key, t in res.items()}


def run_grouped(q, k, v, do, b, scale, causal=False):
    """Forward and backward through the grouped-query entry points (k and v
    carry H_kv heads); returns CPU tensors."""
    dev = _dev()
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    q, k, v, do = (x.to(dev) for x in (q, k, v, do))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if causal:
        bd.causal_attn_fwd_gqa(q, k, v, out, lse, B, T, H, Hkv, D, scale)
        ws = torch.empty(bd.causal_attn_bwd_gqa_workspace_size(B, T, H, Hkv, D), dtype=torch.uint8, device=dev)
        bd.causal_attn_bwd_gqa(q, k, v, out, do, lse, dq, dk, dv, B, T, H, Hkv, D, scale, ws)
    else:
        n = T // 2
        bd.diffusion_attn_fwd_gqa(q, k, v, out, lse, B, n, H, Hkv, D, b, scale)
        ws = torch.empty(bd.diffusion_attn_bwd_gqa_workspace_size(B, n, H, Hkv, D), dtype=torch.uint8,
                         device=dev)
        bd.diffusion_attn_bwd_gqa(q, k, v, out, do, lse, dq, dk, dv, B, n, H, Hkv, D, b, scale, ws)
    torch.cuda.synchronize()
    res = {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    return {key: t.cpu() for key, t in res.items()}


def run_causal(q, k, v, do, scale, bwd=True):
    dev = _dev()
    B, S, H, D = q.shape
    q, k, v = (x.to(dev) for x in (q, k, v))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    bd.causal_attn_fwd(q, k, v, out, lse, B, S, H, D, scale)
    res = {"out": out, "lse": lse}
    if bwd:
        do = do.to(dev)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        ws = torch.empty(bd.causal_attn_bwd_workspace_size(B, S, H, D), dtype=torch.uint8, device=dev)
        bd.causal_attn_bwd(q, k, v, out, do, lse, dq, dk, dv, B, S, H, D, scale, ws)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {key: t.cpu() for key, t in res.items()}


def _halfulp_bf16(x):
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def _bf16_floor(o_ref):
    """max |bf16(O_ref) - O_ref|: what rounding the exact output to bf16
    costs at least (round to nearest even)."""
    r = torch.from_numpy(np.ascontiguousarray(o_ref, dtype=np.float32)).to(torch.bfloat16).double().numpy()
    return float(np.abs(r - o_ref).max()) if o_ref.size else 0.0


def check_fwd(o, lse, o_ref, lse_ref, what, config=None):
    """Every element within max(1e-2, halfulp_bf16(O_ref) + 1e-3); LSE within
    1e-3.  config names the workload the check belongs to, for the report."""
    o = oracle.to_f64(o)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    err = np.abs(o - o_ref)
    bound = np.maximum(FWD_TOL, _halfulp_bf16(o_ref) + 1e-3)
    lerr = float(np.abs(oracle.to_f64(lse) - lse_ref).max())
    beyond = int((err > bound).sum())
    parity_report.record("fwd", what, config, fwd_max=float(err.max()), **{"above_1e-2": int((err > FWD_TOL).sum())},
                         beyond_bound=beyond, floor_max=_bf16_floor(o_ref), lse_max=lerr, elements=int(err.size))
    if beyond:
        worst = np.argmax(err - bound)
        raise AssertionError(f"{what}: {beyond} forward element(s) beyond max(1e-2, halfulp + 1e-3); worst "
                             f"error {err.flat[worst]:.4g} at |O_ref| {abs(o_ref.flat[worst]):.4g} "
                             f"(bound {bound.flat[worst]:.4g})")
    assert lerr <= LSE_TOL, f"{what}: LSE max-abs error {lerr:.3g} > {LSE_TOL}"
    print(f"[{what}] fwd max err {err.max():.3g} (above 1e-2: {int((err > FWD_TOL).sum())}), lse err {lerr:.3g}")


def check_grad(g, g_ref, name, what, config=None):
    g = oracle.to_f64(g)
    scale = np.abs(g_ref).max()
    err = np.abs(g - g_ref).max()
    bound = GRAD_REL * scale if scale > 0 else ZERO_GRAD_ABS
    parity_report.record("grad", what, config, name=name, rel=float(err / scale) if scale > 0 else 0.0,
                         max_abs=float(err))
    assert err <= bound, f"{what}: {name} max-abs error {err:.3g} > {bound:.3g} (max |ref| {scale:.3g})"
    print(f"[{what}] {name} err {err:.3g} (max |ref| {scale:.3g}, rel {err / max(scale, 1e-300):.3g})")


def full_oracle(q, k, v, do, b, scale, heads=None):
    f = lambda x: oracle.to_f64(x)
    O, L = oracle.batched(oracle.diffusion_forward, f(q), f(k), f(v), b=b, scale=scale, heads=heads)
    G = oracle.batched(oracle.diffusion_backward, f(q), f(k), f(v), f(do), b=b, scale=scale, heads=heads)
    return O, L, G


def compare_full(res, q, k, v, do, b, scale, what, heads=None, config=None):
    O, L, (dQ, dK, dV) = full_oracle(q, k, v, do, b, scale, heads)
    if heads is None:
        sel = lambda x: x
        selL = lambda x: x
    else:
        idx = heads
        sel = lambda x: np.stack([np.asarray(x)[bi, :, hi] for bi, hi in idx])
        selL = lambda x: np.stack([np.asarray(x)[bi, hi] for bi, hi in idx])
    check_fwd(sel(oracle.to_f64(res["out"])), selL(oracle.to_f64(res["lse"])), sel(O), selL(L), what, config)
    for name, ref in (("dq", dQ), ("dk", dK), ("dv", dV)):
        check_grad(sel(oracle.to_f64(res[name])), sel(ref), name, what, config)


# ---------------------------------------------------------------------------
# Small problems, compared in full: the tiny workload and the edge cases
# ---------------------------------------------------------------------------

def test_smallest_workload():
    w = WORKLOADS["c1"]
    q, k, v, do = make_workload_inputs(w)
    scale = 1 / math.sqrt(w.D)
    res = run_diffusion(q, k, v, do, w.b, scale)
    compare_full(res, q, k, v, do, w.b, scale, "c1", config="c1")


# every head dimension of the bf16 kernels
HEAD_DIMS = [64, 96, 128, 192, 256]

EDGE = [(n, b) for n in (1, 7, 100, 129, 300) for b in (1, 3, 16, 64, 127, 200, n, n + 5)]


@pytest.mark.parametrize("D", HEAD_DIMS)
@pytest.mark.parametrize("n,b", EDGE)
def test_edge_shapes(n, b, D):
    """Ragged halves (n not a multiple of any tile), blocks of 1 token, blocks
    longer than a half, misaligned blocks."""
    q, k, v, do = make_inputs(2, n, 3, D, seed=7000 + 31 * n + b + D)
    scale = 1 / math.sqrt(D)
    res = run_diffusion(q, k, v, do, b, scale)
    compare_full(res, q, k, v, do, b, scale, f"n{n} b{b} D{D}")


@pytest.mark.parametrize("D", HEAD_DIMS)
@pytest.mark.parametrize("S", [1, 7, 129, 300])
def test_causal_small(S, D):
    q, k, v, do = make_inputs(3, S, 2, D, seed=8000 + S + D)
    q, k, v, do = (x[:, :S].contiguous() for x in (q, k, v, do))
    scale = 1 / math.sqrt(D)
    res = run_causal(q, k, v, do, scale)
    f = oracle.to_f64
    O, L = oracle.batched(oracle.causal_forward, f(q), f(k), f(v), scale=scale)
    dQ, dK, dV = oracle.batched(oracle.causal_backward, f(q), f(k), f(v), f(do), scale=scale)
    check_fwd(res["out"], res["lse"], O, L, f"causal S{S} D{D}")
    for name, ref in (("dq", dQ), ("dk", dK), ("dv", dV)):
        check_grad(res[name], ref, name, f"causal S{S} D{D}")


def test_scale_other_than_default():
    """A scale 2.4 times 1/sqrt(D): the forward is held to check_fwd_rounding's
    bound (the tolerance 1e-2 is stated for the workloads' 1/sqrt(D))."""
    q, k, v, do = make_inputs(1, 70, 2, 64, seed=9001)
    res = run_diffusion(q, k, v, do, 5, 0.3)
    f = oracle.to_f64
    O, L = oracle.batched(oracle.diffusion_forward, f(q), f(k), f(v), b=5, scale=0.3)
    PV, _ = oracle.batched(oracle.diffusion_forward, f(q), f(k), np.abs(f(v)), b=5, scale=0.3)
    G = oracle.batched(oracle.diffusion_backward, f(q), f(k), f(v), f(do), b=5, scale=0.3)
    check_fwd_rounding(res["out"], res["lse"], O, L, PV, "scale 0.3")
    for name, ref in zip(("dq", "dk", "dv"), G):
        check_grad(res[name], ref, name, "scale 0.3")


@pytest.mark.parametrize("D", HEAD_DIMS)
@pytest.mark.parametrize("mag", ["default", "0.2"])
def test_negative_scale(D, mag):
    """The forward folds the sign into Q; the backward uses the signed
    factor.  At -1/sqrt(D) the forward is held to the stated tolerance
    (check_fwd); |scale| = 0.2 is 1.6 to 3.2 times 1/sqrt(D), a scale the
    stated tolerance does not cover, so there the forward is held to
    check_fwd_rounding's bound."""
    scale = -1 / math.sqrt(D) if mag == "default" else -0.2
    q, k, v, do = make_inputs(1, 150, 2, D, seed=9002)
    f = oracle.to_f64
    res = run_diffusion(q, k, v, do, 16, scale)
    O, L = oracle.batched(oracle.diffusion_forward, f(q), f(k), f(v), b=16, scale=scale)
    PV, _ = oracle.batched(oracle.diffusion_forward, f(q), f(k), np.abs(f(v)), b=16, scale=scale)
    G = oracle.batched(oracle.diffusion_backward, f(q), f(k), f(v), f(do), b=16, scale=scale)
    check = check_fwd if mag == "default" else (lambda o, l, O_, L_, w: check_fwd_rounding(o, l, O_, L_, PV, w))
    check(res["out"], res["lse"], O, L, f"scale {scale:.3g} D{D}")
    for name, ref in zip(("dq", "dk", "dv"), G):
        check_grad(res[name], ref, name, f"scale {scale:.3g} D{D}")
    cq, ck, cv, cdo = (make_causal_view(x) for x in (q, k, v, do))
    res = run_causal(cq, ck, cv, cdo, scale)
    O, L = oracle.batched(oracle.causal_forward, f(cq), f(ck), f(cv), scale=scale)
    PV, _ = oracle.batched(oracle.causal_forward, f(cq), f(ck), np.abs(f(cv)), scale=scale)
    dQ, dK, dV = oracle.batched(oracle.causal_backward, f(cq), f(ck), f(cv), f(cdo), scale=scale)
    check(res["out"], res["lse"], O, L, f"causal scale {scale:.3g} D{D}")
    for name, ref in (("dq", dQ), ("dk", dK), ("dv", dV)):
        check_grad(res[name], ref, name, f"causal scale {scale:.3g} D{D}")


# ---------------------------------------------------------------------------
# Determinism and the block-size-1 / causal identity
# ---------------------------------------------------------------------------

def test_bitwise_reproducible():
    w = WORKLOADS["c2"]
    q, k, v, do = make_workload_inputs(w)
    scale = 1 / math.sqrt(w.D)
    a = run_diffusion(q, k, v, do, w.b, scale)
    b = run_diffusion(q, k, v, do, w.b, scale)
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_block_size_one_clean_half_equals_causal_bitwise(D):
    """With block size 1 the clean half is causal attention on the clean
    tokens (Fast Diffusion Attention, "Accuracy"); both entry points run the
    same tile engine with the same key-tile order, so the clean half of the
    diffusion result equals the causal kernel's bit for bit."""
    B, n, H = 2, 300, 3
    q, k, v, do = make_inputs(B, n, H, D, seed=9100 + D)
    scale = 1 / math.sqrt(D)
    d = run_diffusion(q, k, v, do, 1, scale)
    c = run_causal(*(x[:, n:].contiguous() for x in (q, k, v, do)), scale)
    assert torch.equal(d["out"][:, n:], c["out"])
    assert torch.equal(d["lse"][:, :, n:], c["lse"])
    assert torch.equal(d["dq"][:, n:], c["dq"])


def test_autograd_wrapper_matches_entry_points():
    dev = _dev()
    q, k, v, do = make_inputs(2, 96, 2, 64, seed=9200)
    ref = run_diffusion(q, k, v, do, 4, 0.125)
    tq, tk, tv = (x.to(dev).requires_grad_() for x in (q, k, v))
    out, lse = bd.diffusion_attn_func(tq, tk, tv, 4, softmax_scale=0.125, return_lse=True)
    out.backward(do.to(dev))
    assert torch.equal(out.detach().cpu(), ref["out"])
    assert torch.equal(lse.cpu(), ref["lse"])
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert torch.equal(t.grad.cpu(), ref[name]), name


def test_backward_stages_in_order_on_two_streams():
    # stage 0 (dQ, which also writes the row statistics) on one stream, stage
    # 1 (dK/dV, which reads them) on another, ordered by an event: the same
    # bits as the one-call backward
    dev = _dev()
    w = WORKLOADS["c2"]
    q, k, v, do = make_workload_inputs(w)
    scale = 1 / math.sqrt(w.D)
    ref = run_diffusion(q, k, v, do, w.b, scale)
    B, T, H, D = q.shape
    n = T // 2
    q, k, v, do = (x.to(dev) for x in (q, k, v, do))
    out, lse = ref["out"].to(dev), ref["lse"].to(dev)
    dq, dk, dv = (torch.zeros_like(q) for _ in range(3))
    ws = torch.empty(bd.diffusion_attn_bwd_workspace_size(B, n, H, D), dtype=torch.uint8, device=dev)
    MD = bd.MODE_DIFFUSION
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    done0 = torch.cuda.Event()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        bd.bdattn_bwd_stage(MD, 0, q, k, v, out, do, lse, dq, dk, dv, None, B, n, 0, H, H, D, w.b, scale, 0.0, ws,
                            stream=s1)
        done0.record(s1)
    s2.wait_event(done0)
    with torch.cuda.stream(s2):
        bd.bdattn_bwd_stage(MD, 1, q, k, v, out, do, lse, dq, dk, dv, None, B, n, 0, H, H, D, w.b, scale, 0.0, ws,
                            stream=s2)
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.equal(t.cpu(), ref[name]), name


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,heads", [("c2", [(0, 0), (1, 5), (2, 10), (3, 15)]),
                                        ("c3", [(0, 0), (7, 15)])])
def test_workload_whole_heads(name, heads):
    w = WORKLOADS[name]
    q, k, v, do = make_workload_inputs(w)
    scale = 1 / math.sqrt(w.D)
    res = run_diffusion(q, k, v, do, w.b, scale)
    compare_full(res, q, k, v, do, w.b, scale, name, heads=heads, config=name)


C5 = sorted(n for n in WORKLOADS if n.startswith("c5"))


@pytest.mark.parametrize("name", C5)
def test_block_size_sweep(name):
    w = WORKLOADS[name]
    q, k, v, do = make_workload_inputs(w)
    scale = 1 / math.sqrt(w.D)
    res = run_diffusion(q, k, v, do, w.b, scale)
    compare_full(res, q, k, v, do, w.b, scale, name, heads=[(3, 7)], config=name)


@pytest.mark.parametrize("name", sorted(HEAD_DIM_WORKLOADS))
def test_head_dim_workload(name):
    """Head dimensions 96, 192 and 256 at full size: every output of two
    heads."""
    w = HEAD_DIM_WORKLOADS[name]
    q, k, v, do = make_workload_inputs(w)
    scale = 1 / math.sqrt(w.D)
    res = run_diffusion(q, k, v, do, w.b, scale)
    compare_full(res, q, k, v, do, w.b, scale, name, heads=[(0, 0), (w.B - 1, w.H - 1)], config=name)


def _sample_positions(n, b, rng, count):
    s = {0, 1, n - 1, n - 2, min(b, n - 1), max(0, n - b)}
    for t in (64, 128, 256):
        for m in range(t, n, t * 7):
            s.update({m - 1, m})
    s.update(rng.integers(0, n, size=count).tolist())
    return sorted(x for x in s if 0 <= x < n)


def test_largest_workload_sampled():
    """The long-sequence workload: all rows of O and LSE of two heads, dQ on
    sampled rows and dK / dV on sampled key columns of those heads."""
    w = WORKLOADS["c4"]
    q, k, v, do = make_workload_inputs(w)
    scale = 1 / math.sqrt(w.D)
    res = run_diffusion(q, k, v, do, w.b, scale)
    rng = np.random.default_rng(4)
    n = w.n
    for bi, hi in ((0, 0), (1, 31)):
        f = lambda x: oracle.to_f64(x[bi, :, hi])
        qh, kh, vh, dh = f(q), f(k), f(v), f(do)
        O = np.empty((2 * n, w.D))
        L = np.empty(2 * n)
        for r0 in range(0, 2 * n, 2048):
            rows = np.arange(r0, r0 + 2048)
            O[rows], L[rows] = oracle.diffusion_forward_rows(qh, kh, vh, w.b, scale, rows)
        tag = f"c4 head ({bi},{hi})"
        check_fwd(res["out"][bi, :, hi], res["lse"][bi, hi], O, L, tag, "c4")
        pos = _sample_positions(n, w.b, rng, 24)
        rows = np.array(pos + [n + p for p in pos])
        dq_ref = oracle.diffusion_grad_q_rows(qh, kh, vh, dh, w.b, scale, rows)
        check_grad(res["dq"][bi, rows, hi], dq_ref, "dq", tag, "c4")
        dk_ref, dv_ref = oracle.diffusion_grad_kv_cols(qh, kh, vh, dh, O, L, w.b, scale, rows)
        check_grad(res["dk"][bi, rows, hi], dk_ref, "dk", tag, "c4")
        check_grad(res["dv"][bi, rows, hi], dv_ref, "dv", tag, "c4")


# Every (sample, head) of the full-size workloads, on a fixed set of positions.
EVERY_HEAD = ["c2", "c3", "c4"] + C5 + ["h1", "h2", "h3", "g1", "g2", "g3"]


def head_positions(n, b, j, seed):
    """The positions (inside a half) checked for the j-th (sample, head) pair
    of a workload (j = sample * H + head):
      * the first two and last two positions, 0, 1, n - 2, n - 1;
      * both sides of the start of the second, third and last block
        (b - 1, b, 2b - 1, 2b, and the last block's start and the position
        before it);
      * both sides of every sixteenth multiple of 32 starting at the
        (j mod 16 + 1)-th: 32 positions is the height of a wave's query rows
        and of a key block, and multiples of it are the boundaries of every
        query and key tile (64 and 128 wide), so sixteen consecutive pairs
        cover every boundary of a half;
      * 32 positions drawn uniformly from a generator seeded with
        seed * 1000 + j.
    """
    s = {0, 1, n - 2, n - 1}
    for m in (b, 2 * b, (n - 1) // b * b):
        s.update({m - 1, m})
    for t in range(32 * (1 + j % 16), n, 32 * 16):
        s.update({t - 1, t})
    s.update(np.random.default_rng(seed * 1000 + j).integers(0, n, size=32).tolist())
    return sorted(x for x in s if 0 <= x < n)


def kv_columns(n, b, pos, window):
    """Key positions (of the whole sample) whose dK and dV are checked, and
    the query rows that see any of them: every noisy position of ``pos``
    (a noisy key is seen only by the noisy rows of its own block), and the
    clean positions of ``pos`` in the last ``window`` of the half (a clean
    key is seen by the clean rows from its block on and by the noisy rows of
    later blocks, so a key near the start of the half needs the statistics
    of almost every row)."""
    noisy = [p for p in pos]
    clean = [p for p in pos if p >= n - window]
    cols = np.array(noisy + [n + p for p in clean], dtype=np.int64)
    rows = set()
    for p in noisy:
        bs = p // b * b
        rows.update(range(bs, min(bs + b, n)))
    if clean:
        bs = min(clean) // b * b
        be = min(bs + b, n)
        rows.update(range(n + bs, 2 * n))  # clean rows of the same or later blocks
        rows.update(range(be, n))          # noisy rows of later blocks
    return cols, np.array(sorted(rows), dtype=np.int64)


@functools.lru_cache(maxsize=1)
def _workload_result(name):
    """Inputs and GPU outputs of a full-size workload, launched as the
    benchmark launches it (kept for the consecutive parts of one workload)."""
    w = {**WORKLOADS, **HEAD_DIM_WORKLOADS, **GQA_WORKLOADS}[name]
    q, k, v, do = make_workload_inputs(w)
    scale = 1 / math.sqrt(w.D)
    run = run_grouped if w.kv_heads != w.H else run_diffusion
    return w, (q, k, v, do), run(q, k, v, do, w.b, scale)


def _q_refs(qh, kh, vh, dh, n, b, scale, pos):
    """O, LSE and dQ of one query head at the rows of ``pos`` in both halves
    (see test_every_head_sampled)."""
    rows = np.array(pos + [n + p for p in pos], dtype=np.int64)
    O, L = oracle.diffusion_forward_rows(qh, kh, vh, b, scale, rows)
    dq_ref = oracle.diffusion_grad_q_rows(qh, kh, vh, dh, b, scale, rows)
    return rows, O, L, dq_ref


def _kv_refs(qhs, kh, vh, dhs, n, b, D, scale, cols, seen):
    """dK and dV of one key/value head at the key columns ``cols``: the sum
    over the query heads that read it (qhs, dhs), each needing O and LSE of
    the rows ``seen`` that see those columns."""
    dk_ref, dv_ref = 0.0, 0.0
    for qh, dh in zip(qhs, dhs):
        Of, Lf = np.zeros((2 * n, D)), np.zeros(2 * n)
        Of[seen], Lf[seen] = oracle.diffusion_forward_rows(qh, kh, vh, b, scale, seen)
        dk, dv = oracle.diffusion_grad_kv_cols(qh, kh, vh, dh, Of, Lf, b, scale, cols)
        dk_ref, dv_ref = dk_ref + dk, dv_ref + dv
    return dk_ref, dv_ref


def _full_row_stats(qh, kh, vh, b, scale, ex, chunk=2048):
    """O and LSE of every row of one head, in chunks of rows on the pool ex."""
    T = qh.shape[0]
    parts = list(ex.map(lambda r0: oracle.diffusion_forward_rows(qh, kh, vh, b, scale,
                                                                 np.arange(r0, min(r0 + chunk, T))),
                        range(0, T, chunk)))
    return np.concatenate([o for o, _ in parts]), np.concatenate([l for _, l in parts])


@pytest.mark.parametrize("name", EVERY_HEAD)
def test_every_head_sampled(name):
    """Every (sample, head) of the full-size workloads, as the benchmark
    launches them: O, LSE and dQ of every query head at the rows
    head_positions names (in both halves, j = sample * H + head), and dK / dV
    of every key/value head at the key columns kv_columns derives from
    head_positions for j = sample * H_kv + kv head (the clean columns within
    the last max(512, 2^21 / 2n) positions of the half, all of it at c2);
    with grouped heads the reference dK / dV sums over the query heads of the
    group.  The gradients are held to 2e-2 times the largest oracle value of
    their tensor that this test computes: every sampled row and column of
    every head, plus the first 64 clean key columns of key/value head (0, 0)
    (seen by nearly every row, they carry the largest dK and dV), a lower
    bound of the tensor's maximum.  The oracle runs on one thread per task
    (one BLAS thread each)."""
    import concurrent.futures
    from threadpoolctl import threadpool_limits
    w, (q, k, v, do), res = _workload_result(name)
    scale = 1 / math.sqrt(w.D)
    n, b, H, Hkv = w.n, w.b, w.H, w.kv_heads
    G = H // Hkv
    window = min(n, max(512, 2 ** 21 // (2 * n)))
    f = lambda x: oracle.to_f64(x)
    qpairs = [divmod(j, H) for j in range(w.B * H)]
    kvpairs = [divmod(j, Hkv) for j in range(w.B * Hkv)]
    kvcols = {bh: kv_columns(n, b, head_positions(n, b, bh[0] * Hkv + bh[1], w.seed), window) for bh in kvpairs}
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(1), concurrent.futures.ThreadPoolExecutor(workers) as ex:
        qrefs = list(ex.map(lambda bh: _q_refs(f(q[bh[0], :, bh[1]]), f(k[bh[0], :, bh[1] // G]),
                                               f(v[bh[0], :, bh[1] // G]), f(do[bh[0], :, bh[1]]), n, b, scale,
                                               head_positions(n, b, bh[0] * H + bh[1], w.seed)),
                            qpairs))
        kvrefs = list(ex.map(lambda bh: _kv_refs([f(q[bh[0], :, bh[1] * G + g]) for g in range(G)],
                                                 f(k[bh[0], :, bh[1]]), f(v[bh[0], :, bh[1]]),
                                                 [f(do[bh[0], :, bh[1] * G + g]) for g in range(G)],
                                                 n, b, w.D, scale, *kvcols[bh]),
                             kvpairs))
        k0, v0 = f(k[0, :, 0]), f(v[0, :, 0])
        early = n + np.arange(min(64, n))
        dk0, dv0 = 0.0, 0.0
        for g in range(G):
            q0, d0 = f(q[0, :, g]), f(do[0, :, g])
            O0, L0 = _full_row_stats(q0, k0, v0, b, scale, ex)
            dk, dv = oracle.diffusion_grad_kv_cols(q0, k0, v0, d0, O0, L0, b, scale, early)
            dk0, dv0 = dk0 + dk, dv0 + dv
    gmax = {"dq": max(np.abs(r[3]).max() for r in qrefs),
            "dk": max(max(np.abs(r[0]).max() for r in kvrefs), np.abs(dk0).max()),
            "dv": max(max(np.abs(r[1]).max() for r in kvrefs), np.abs(dv0).max())}
    checks = [(0, 0, "dk", early, dk0), (0, 0, "dv", early, dv0)]
    for (bi, hi), (rows, O, L, dq_ref) in zip(qpairs, qrefs):
        check_fwd(res["out"][bi, rows, hi], res["lse"][bi, hi, rows], O, L, f"{name} ({bi},{hi})", name)
        checks.append((bi, hi, "dq", rows, dq_ref))
    for (bi, hk), (dk_ref, dv_ref) in zip(kvpairs, kvrefs):
        cols = kvcols[(bi, hk)][0]
        checks += [(bi, hk, "dk", cols, dk_ref), (bi, hk, "dv", cols, dv_ref)]
    for bi, hi, gname, idx, ref in checks:
        check_grad_scaled(res[gname][bi, idx, hi], ref, gmax[gname], gname, f"{name} ({bi},{hi})", name)


def check_grad_scaled(g, g_ref, g_max, name, what, config=None):
    """max |g - g_ref| <= 2e-2 * g_max, g_max the largest |oracle value| of
    the whole tensor (or a lower bound of it)."""
    g = oracle.to_f64(g)
    err = np.abs(g - g_ref).max()
    bound = GRAD_REL * g_max
    parity_report.record("grad", what, config, name=name, rel=float(err / g_max), max_abs=float(err))
    assert err <= bound, f"{what}: {name} max-abs error {err:.3g} > {bound:.3g} (max |ref| of the tensor {g_max:.3g})"


def test_causal_yardstick_workload():
    """The equal-work causal problem of the medium workload: 16 sequences of
    2048 tokens (its two halves per sample), checked on two sequences."""
    w = WORKLOADS["c3"]
    q, k, v, do = (x.reshape(2 * w.B, w.n, w.H, w.D) for x in make_workload_inputs(w))
    scale = 1 / math.sqrt(w.D)
    res = run_causal(q, k, v, do, scale)
    f = oracle.to_f64
    for si, hi in ((0, 0), (15, 9)):
        O, L = oracle.causal_forward(f(q[si, :, hi]), f(k[si, :, hi]), f(v[si, :, hi]), scale)
        check_fwd(res["out"][si, :, hi], res["lse"][si, hi], O, L, f"causal c3 seq {si}")
        dQ, dK, dV = oracle.causal_backward(f(q[si, :, hi]), f(k[si, :, hi]), f(v[si, :, hi]),
                                            f(do[si, :, hi]), scale)
        for name, ref in (("dq", dQ), ("dk", dK), ("dv", dV)):
            check_grad(res[name][si, :, hi], ref, name, f"causal c3 seq {si}")


# ---------------------------------------------------------------------------
# Grouped-query attention (query heads sharing key/value heads)
# ---------------------------------------------------------------------------

def compare_grouped(res, q, k, v, do, b, scale, what, causal=False, groups=None, config=None):
    """Oracle check of a grouped result; ``groups`` lists (sample, key/value
    head) pairs to check (default: all), each with all the query heads that
    read it."""
    f = oracle.to_f64
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    one_fwd = (lambda qq, kk, vv, **kw: oracle.causal_forward(qq, kk, vv, kw["scale"])) if causal \
        else oracle.diffusion_forward
    one_bwd = (lambda qq, kk, vv, dd, **kw: oracle.causal_backward(qq, kk, vv, dd, kw["scale"])) if causal \
        else oracle.diffusion_backward
    todo = groups if groups is not None else [(bi, j) for bi in range(B) for j in range(Hkv)]
    for bi, j in todo:
        hs = slice(j * G, (j + 1) * G)
        sq, sdo = f(q[bi:bi + 1, :, hs]), f(do[bi:bi + 1, :, hs])
        sk, sv = f(k[bi:bi + 1, :, j:j + 1]), f(v[bi:bi + 1, :, j:j + 1])
        O, L = oracle.grouped_forward(one_fwd, sq, sk, sv, b=b, scale=scale)
        dQ, dK, dV = oracle.grouped_backward(one_bwd, sq, sk, sv, sdo, b=b, scale=scale)
        tag = f"{what} sample {bi} kv head {j}"
        check_fwd(res["out"][bi:bi + 1, :, hs], res["lse"][bi:bi + 1, hs], O, L, tag, config)
        check_grad(res["dq"][bi:bi + 1, :, hs], dQ, "dq", tag, config)
        check_grad(res["dk"][bi:bi + 1, :, j:j + 1], dK, "dk", tag, config)
        check_grad(res["dv"][bi:bi + 1, :, j:j + 1], dV, "dv", tag, config)


GQA_SMALL = [  # B, n, H, H_kv, D, b
    (2, 100, 4, 2, 64, 16), (1, 129, 6, 3, 128, 7), (2, 300, 4, 1, 64, 64),
    (1, 7, 8, 2, 128, 3), (1, 257, 8, 1, 128, 32), (2, 64, 3, 1, 64, 200),
    (1, 200, 4, 1, 256, 16), (2, 65, 6, 2, 256, 5),
    (2, 150, 8, 2, 96, 12), (1, 333, 6, 1, 192, 40),
]


@pytest.mark.parametrize("B,n,H,Hkv,D,b", GQA_SMALL)
def test_grouped_small(B, n, H, Hkv, D, b):
    q, k, v, do = make_inputs(B, n, H, D, seed=9300 + n + H + Hkv, H_kv=Hkv)
    scale = 1 / math.sqrt(D)
    res = run_grouped(q, k, v, do, b, scale)
    compare_grouped(res, q, k, v, do, b, scale, f"gqa n{n} H{H}/{Hkv} D{D} b{b}")


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_grouped_causal_small(D):
    q, k, v, do = make_inputs(2, 150, 6, D, seed=9400 + D, H_kv=2)
    q, k, v, do = (x[:, :150].contiguous() for x in (q, k, v, do))
    scale = 1 / math.sqrt(D)
    res = run_grouped(q, k, v, do, 1, scale, causal=True)
    compare_grouped(res, q, k, v, do, 1, scale, f"causal gqa D{D}", causal=True)


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_grouped_matches_repeated_heads(D):
    """Each query head reads its group's key/value head, so O, LSE and dQ
    equal (bit for bit) the plain entry points on key/value heads repeated
    to H; with H_kv = H the grouped entry points are the plain ones."""
    B, n, H, Hkv, b = 2, 200, 6, 2, 8
    q, k, v, do = make_inputs(B, n, H, D, seed=9500 + D, H_kv=Hkv)
    scale = 1 / math.sqrt(D)
    g = run_grouped(q, k, v, do, b, scale)
    rk, rv = (x.repeat_interleave(H // Hkv, dim=2).contiguous() for x in (k, v))
    m = run_diffusion(q, rk, rv, do, b, scale)
    for key in ("out", "lse", "dq"):
        assert torch.equal(g[key], m[key]), key
    same = run_grouped(q, rk, rv, do, b, scale)
    for key in m:
        assert torch.equal(same[key], m[key]), key


@pytest.mark.parametrize("name", sorted(n for n in GQA_WORKLOADS if n != "g2"))
def test_grouped_workload_heads(name):
    w = GQA_WORKLOADS[name]
    q, k, v, do = make_workload_inputs(w)
    scale = 1 / math.sqrt(w.D)
    res = run_grouped(q, k, v, do, w.b, scale)
    # first and last key/value head; a multi-query problem has one group of
    # all H query heads per sample, checked on the last sample
    groups = [(0, 0), (w.B - 1, w.kv_heads - 1)] if w.kv_heads > 1 else [(w.B - 1, 0)]
    compare_grouped(res, q, k, v, do, w.b, scale, name, groups=groups, config=name)


def test_grouped_long_workload_sampled():
    """The long-sequence grouped problem: for one key/value head, all rows of
    O and LSE of its query heads, sampled dQ rows of each, and dK / dV on
    sampled key columns (summed over the group by the oracle)."""
    w = GQA_WORKLOADS["g2"]
    q, k, v, do = make_workload_inputs(w)
    scale = 1 / math.sqrt(w.D)
    res = run_grouped(q, k, v, do, w.b, scale)
    rng = np.random.default_rng(5)
    n, G = w.n, w.H // w.kv_heads
    bi, j = 1, w.kv_heads - 1
    f = lambda x: oracle.to_f64(x)
    kh, vh = f(k[bi, :, j]), f(v[bi, :, j])
    pos = _sample_positions(n, w.b, rng, 16)
    rows = np.array(pos + [n + p for p in pos])
    qs, dos, outs, lses = [], [], [], []
    for h in range(j * G, (j + 1) * G):
        qh, dh = f(q[bi, :, h]), f(do[bi, :, h])
        O = np.empty((2 * n, w.D))
        L = np.empty(2 * n)
        for r0 in range(0, 2 * n, 2048):
            rr = np.arange(r0, r0 + 2048)
            O[rr], L[rr] = oracle.diffusion_forward_rows(qh, kh, vh, w.b, scale, rr)
        tag = f"g2 sample {bi} head {h}"
        check_fwd(res["out"][bi, :, h], res["lse"][bi, h], O, L, tag, "g2")
        dq_ref = oracle.diffusion_grad_q_rows(qh, kh, vh, dh, w.b, scale, rows)
        check_grad(res["dq"][bi, rows, h], dq_ref, "dq", tag, "g2")
        qs.append(qh)
        dos.append(dh)
        outs.append(O)
        lses.append(L)
    dk_ref, dv_ref = oracle.grouped_grad_kv_cols(qs, kh, vh, dos, outs, lses, w.b, scale, rows)
    check_grad(res["dk"][bi, rows, j], dk_ref, "dk", f"g2 kv head {j}", "g2")
    check_grad(res["dv"][bi, rows, j], dv_ref, "dv", f"g2 kv head {j}", "g2")


def test_grouped_autograd_wrapper():
    dev = _dev()
    q, k, v, do = make_inputs(2, 96, 4, 64, seed=9600, H_kv=2)
    ref = run_grouped(q, k, v, do, 4, 0.125)
    tq, tk, tv = (x.to(dev).requires_grad_() for x in (q, k, v))
    out, lse = bd.diffusion_attn_func(tq, tk, tv, 4, softmax_scale=0.125, return_lse=True)
    out.backward(do.to(dev))
    assert torch.equal(out.detach().cpu(), ref["out"])
    assert torch.equal(lse.cpu(), ref["lse"])
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert torch.equal(t.grad.cpu(), ref[name]), name


# ---------------------------------------------------------------------------
# Packed batches of samples of different lengths
# ---------------------------------------------------------------------------

def run_varlen(q, k, v, do, cu, max_n, b, scale, causal=False):
    """Forward and backward through the varlen entry points; CPU results."""
    dev = _dev()
    total, H, D = q.shape
    Hkv = k.shape[1]
    B = len(cu) - 1
    q, k, v, do = (x.to(dev) for x in (q, k, v, do))
    cu_t = torch.tensor(cu, dtype=torch.int32, device=dev)
    # poisoned outputs: rows outside every sample must come back untouched
    out = torch.full_like(q, 7.0)
    lse = torch.full((H, total), 7.0, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(v, 7.0)
    if causal:
        bd.causal_attn_varlen_fwd(q, k, v, out, lse, cu_t, B, max_n, total, H, Hkv, D, scale)
        wsb = bd.causal_attn_varlen_bwd_workspace_size(B, max_n, total, H, Hkv, D)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        bd.causal_attn_varlen_bwd(q, k, v, out, do, lse, dq, dk, dv, cu_t, B, max_n, total, H, Hkv, D,
                                  scale, ws, wsb)
    else:
        bd.diffusion_attn_varlen_fwd(q, k, v, out, lse, cu_t, B, max_n, total, H, Hkv, D, b, scale)
        wsb = bd.diffusion_attn_varlen_bwd_workspace_size(B, max_n, total, H, Hkv, D)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        bd.diffusion_attn_varlen_bwd(q, k, v, out, do, lse, dq, dk, dv, cu_t, B, max_n, total, H, Hkv,
                                     D, b, scale, ws, wsb)
    torch.cuda.synchronize()
    res = {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    return {key: t.cpu() for key, t in res.items()}


VARLEN_SMALL = [  # half lengths, H, H_kv, D, b
    ([100, 0, 7, 129, 1, 300], 3, 3, 64, 16),
    ([64, 250, 0, 0, 33], 4, 2, 128, 5),
    ([1, 2, 3, 200], 6, 1, 64, 200),
    ([128, 384, 127, 129], 2, 2, 128, 32),
    ([100, 0, 65, 257], 2, 1, 256, 16),
    ([33, 0, 190, 64], 4, 2, 96, 8),
    ([129, 5, 0, 260], 2, 2, 192, 48),
]


@pytest.mark.parametrize("ns,H,Hkv,D,b", VARLEN_SMALL)
def test_varlen_small(ns, H, Hkv, D, b):
    """Mixed lengths, empty samples, ragged tiles: against the oracle on every
    sample; rows outside samples (none here) and no sample's rows are left
    with the poison value."""
    q, k, v, do, cu = make_varlen_inputs(ns, H, D, seed=9700 + sum(ns) + D, H_kv=Hkv)
    scale = 1 / math.sqrt(D)
    res = run_varlen(q, k, v, do, cu, max(ns), b, scale)
    f = oracle.to_f64
    O, L = oracle.varlen_forward(oracle.diffusion_forward, f(q), f(k), f(v), cu, b=b, scale=scale)
    G = oracle.varlen_backward(oracle.diffusion_backward, f(q), f(k), f(v), f(do), cu, b=b, scale=scale)
    tag = f"varlen {ns} H{H}/{Hkv} D{D} b{b}"
    check_fwd(res["out"], res["lse"], O, L, tag)
    for name, ref in zip(("dq", "dk", "dv"), G):
        check_grad(res[name], ref, name, tag)


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_varlen_equals_batched_per_sample_bitwise(D):
    """Each packed sample is computed exactly as the batched entry points
    compute it alone (Fast Diffusion Attention, "Accuracy": the varlen
    kernels agree with the batched ones), bit for bit; rows after the last
    sample keep the caller's contents."""
    ns, H, b = [300, 0, 129, 1, 64], 3, 16
    q, k, v, do, cu = make_varlen_inputs(ns, H, D, seed=9800 + D)
    pad = 5  # tokens after the last sample, in no sample
    q, k, v, do = (torch.cat([x, torch.ones(pad, *x.shape[1:], dtype=x.dtype)]) for x in (q, k, v, do))
    scale = 1 / math.sqrt(D)
    res = run_varlen(q, k, v, do, cu, max(ns), b, scale)
    for bi, nb in enumerate(ns):
        if nb == 0:
            continue
        s0, s1 = cu[bi], cu[bi + 1]
        one = run_diffusion(*(x[None, s0:s1] for x in (q, k, v, do)), b, scale)
        for key in ("out", "dq", "dk", "dv"):
            assert torch.equal(res[key][s0:s1], one[key][0]), (bi, key)
        assert torch.equal(res["lse"][:, s0:s1], one["lse"][0]), bi
    tail = slice(cu[-1], cu[-1] + pad)
    for key in ("out", "dq", "dk", "dv"):
        assert bool((res[key][tail] == 7.0).all()), key
    assert bool((res["lse"][:, tail] == 7.0).all())


@pytest.mark.parametrize("Hkv", [4, 2])
def test_varlen_causal_small(Hkv):
    ns, H, D = [150, 0, 77, 300], 4, 64
    q, k, v, do, cu = make_varlen_inputs(ns, H, D, seed=9900 + Hkv, H_kv=Hkv, causal=True)
    scale = 1 / math.sqrt(D)
    res = run_varlen(q, k, v, do, cu, max(ns), 1, scale, causal=True)
    f = oracle.to_f64
    fwd = lambda qq, kk, vv, scale: oracle.causal_forward(qq, kk, vv, scale)
    bwd = lambda qq, kk, vv, dd, scale: oracle.causal_backward(qq, kk, vv, dd, scale)
    O, L = oracle.varlen_forward(fwd, f(q), f(k), f(v), cu, scale=scale)
    G = oracle.varlen_backward(bwd, f(q), f(k), f(v), f(do), cu, scale=scale)
    check_fwd(res["out"], res["lse"], O, L, f"causal varlen H{H}/{Hkv}")
    for name, ref in zip(("dq", "dk", "dv"), G):
        check_grad(res[name], ref, name, f"causal varlen H{H}/{Hkv}")


def test_varlen_skips_inconsistent_offsets():
    """A sample whose offsets are inconsistent (here: an odd token count, and
    one running past the packed total) is skipped by the kernels' own
    checks; the consistent samples are still exact and nothing else is
    written."""
    H, D, b = 2, 64, 8
    ns = [40, 30, 50]
    q, k, v, do, cu = make_varlen_inputs(ns, H, D, seed=9950)
    total = cu[-1]
    scale = 1 / math.sqrt(D)
    assert cu == [0, 80, 140, 240]
    # sample 1 has an odd token count (59); sample 2 then covers tokens
    # 139..239, a consistent 2 x 50
    bad = [0, 80, 139, 239]
    res = run_varlen(q, k, v, do, bad, 50, b, scale)
    good = run_varlen(q, k, v, do, cu, 50, b, scale)
    for key in ("out", "dq", "dk", "dv"):
        assert torch.equal(res[key][:80], good[key][:80]), key
        assert bool((res[key][80:139] == 7.0).all()), key
        assert bool(torch.isfinite(res[key][139:239].float()).all()), key
        assert bool((res[key][239:] == 7.0).all()), key
    past = [0, 80, total + 64]                         # sample 1 ends past the tensors
    res = run_varlen(q[:total], k[:total], v[:total], do[:total], past, 50, b, scale)
    assert torch.equal(res["out"][:40 * 2], good["out"][:80])


@pytest.mark.parametrize("name", sorted(VARLEN_WORKLOADS))
def test_varlen_workloads(name):
    """The packed workloads as the benchmark launches them: the longest and
    the shortest sample of each, and one in between, checked on two heads."""
    w = VARLEN_WORKLOADS[name]
    q, k, v, do, cu = make_varlen_workload_inputs(w)
    ns = w.half_lengths
    scale = 1 / math.sqrt(w.D)
    res = run_varlen(q, k, v, do, cu, max(ns), w.b, scale)
    f = oracle.to_f64
    G = w.H // w.kv_heads
    order = sorted(range(len(ns)), key=lambda i: ns[i])
    for bi in (order[-1], order[0], order[len(ns) // 2]):
        s0, s1 = cu[bi], cu[bi + 1]
        j = w.kv_heads - 1
        hs = slice(j * G, (j + 1) * G)
        sq, sdo = f(q[None, s0:s1, hs]), f(do[None, s0:s1, hs])
        sk, sv = f(k[None, s0:s1, j:j + 1]), f(v[None, s0:s1, j:j + 1])
        O, L = oracle.grouped_forward(oracle.diffusion_forward, sq, sk, sv, b=w.b, scale=scale)
        dQ, dK, dV = oracle.grouped_backward(oracle.diffusion_backward, sq, sk, sv, sdo, b=w.b, scale=scale)
        tag = f"{name} sample {bi} (n={ns[bi]}) kv head {j}"
        check_fwd(res["out"][None, s0:s1, hs], res["lse"][hs, s0:s1][None], O, L, tag, name)
        check_grad(res["dq"][None, s0:s1, hs], dQ, "dq", tag, name)
        check_grad(res["dk"][None, s0:s1, j:j + 1], dK, "dk", tag, name)
        check_grad(res["dv"][None, s0:s1, j:j + 1], dV, "dv", tag, name)


@pytest.mark.parametrize("name", sorted(VARLEN_WORKLOADS))
def test_varlen_every_head_sampled(name):
    """Every (sample, head) of the packed workloads, as the benchmark
    launches them, on the positions test_every_head_sampled uses (per sample,
    with its own half length): O, LSE and dQ of every query head, dK and dV
    of every key/value head (summed over its group).  Gradients are held to
    2e-2 times the largest oracle value computed (the first 64 clean key
    columns of the longest sample's first key/value head included)."""
    import concurrent.futures
    from threadpoolctl import threadpool_limits
    w = VARLEN_WORKLOADS[name]
    q, k, v, do, cu = make_varlen_workload_inputs(w)
    ns = w.half_lengths
    scale = 1 / math.sqrt(w.D)
    res = run_varlen(q, k, v, do, cu, max(ns), w.b, scale)
    f = oracle.to_f64
    H, Hkv, b = w.H, w.kv_heads, w.b
    G = H // Hkv
    samples = [bi for bi in range(len(ns)) if ns[bi] > 0]
    win = lambda n: min(n, max(512, 2 ** 21 // (2 * n)))
    qtasks = [(bi, hh) for bi in samples for hh in range(H)]
    kvtasks = [(bi, hk) for bi in samples for hk in range(Hkv)]
    kvcols = {(bi, hk): kv_columns(ns[bi], b, head_positions(ns[bi], b, bi * Hkv + hk, w.seed), win(ns[bi]))
              for bi, hk in kvtasks}
    sl = lambda x, bi, h: f(x[cu[bi]:cu[bi + 1], h])
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(1), concurrent.futures.ThreadPoolExecutor(workers) as ex:
        qrefs = list(ex.map(lambda t: _q_refs(sl(q, t[0], t[1]), sl(k, t[0], t[1] // G), sl(v, t[0], t[1] // G),
                                              sl(do, t[0], t[1]), ns[t[0]], b, scale,
                                              head_positions(ns[t[0]], b, t[0] * H + t[1], w.seed)),
                            qtasks))
        kvrefs = list(ex.map(lambda t: _kv_refs([sl(q, t[0], t[1] * G + g) for g in range(G)],
                                                sl(k, t[0], t[1]), sl(v, t[0], t[1]),
                                                [sl(do, t[0], t[1] * G + g) for g in range(G)],
                                                ns[t[0]], b, w.D, scale, *kvcols[t]),
                             kvtasks))
        bl = max(samples, key=lambda i: ns[i])
        nl = ns[bl]
        early = nl + np.arange(min(64, nl))
        k0, v0 = sl(k, bl, 0), sl(v, bl, 0)
        dk0, dv0 = 0.0, 0.0
        for g in range(G):
            q0, d0 = sl(q, bl, g), sl(do, bl, g)
            O0, L0 = _full_row_stats(q0, k0, v0, b, scale, ex)
            dk, dv = oracle.diffusion_grad_kv_cols(q0, k0, v0, d0, O0, L0, b, scale, early)
            dk0, dv0 = dk0 + dk, dv0 + dv
    gmax = {"dq": max(np.abs(r[3]).max() for r in qrefs),
            "dk": max(max(np.abs(r[0]).max() for r in kvrefs), np.abs(dk0).max()),
            "dv": max(max(np.abs(r[1]).max() for r in kvrefs), np.abs(dv0).max())}
    checks = [(bl, 0, "dk", early, dk0), (bl, 0, "dv", early, dv0)]
    for (bi, hh), (rows, O, L, dq_ref) in zip(qtasks, qrefs):
        tok = cu[bi] + rows
        check_fwd(res["out"][tok, hh], res["lse"][hh, tok], O, L, f"{name} sample {bi} head {hh}", name)
        checks.append((bi, hh, "dq", rows, dq_ref))
    for (bi, hk), (dk_ref, dv_ref) in zip(kvtasks, kvrefs):
        cols = kvcols[(bi, hk)][0]
        checks += [(bi, hk, "dk", cols, dk_ref), (bi, hk, "dv", cols, dv_ref)]
    for bi, h, gname, idx, ref in checks:
        check_grad_scaled(res[gname][cu[bi] + idx, h], ref, gmax[gname], gname, f"{name} sample {bi} head {h}", name)


def test_varlen_autograd_wrapper():
    dev = _dev()
    ns, H, Hkv, D = [70, 0, 33, 128], 4, 2, 64
    q, k, v, do, cu = make_varlen_inputs(ns, H, D, seed=9990, H_kv=Hkv)
    ref = run_varlen(q, k, v, do, cu, max(ns), 4, 0.125)
    tq, tk, tv = (x.to(dev).requires_grad_() for x in (q, k, v))
    cu_t = torch.tensor(cu, dtype=torch.int32, device=dev)
    out, lse = bd.diffusion_attn_varlen_func(tq, tk, tv, cu_t, max(ns), 4, softmax_scale=0.125,
                                             return_lse=True)
    out.backward(do.to(dev))
    assert torch.equal(out.detach().cpu(), ref["out"])
    assert torch.equal(lse.cpu(), ref["lse"])
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert torch.equal(t.grad.cpu(), ref[name]), name


def test_largest_accepted_sample():
    """The largest accepted sample: 2n tokens x 256 heads x D = 128 of bf16
    just under 2 GiB (one more token per half is rejected), so every 32-bit
    buffer offset is at its limit.  Checked on the last head: rows at the
    ends of both halves for O, LSE and dQ, and key columns there for dK/dV."""
    B, n, H, D, b = 1, 16383, 256, 128, 64
    assert 2 * n * H * D * 2 < 2 ** 31 <= 2 * (n + 1) * H * D * 2
    dev = _dev()
    q, k, v, do = make_inputs(B, n, H, D, seed=9995)
    scale = 1 / math.sqrt(D)
    res = run_diffusion(q, k, v, do, b, scale)
    hi = H - 1
    f = lambda x: oracle.to_f64(x[0, :, hi])
    qh, kh, vh, dh = f(q), f(k), f(v), f(do)
    rows = np.array([0, 1, n - 2, n - 1, n, n + 1, 2 * n - 2, 2 * n - 1])
    O, L = oracle.diffusion_forward_rows(qh, kh, vh, b, scale, rows)
    check_fwd(res["out"][0, rows, hi], res["lse"][0, hi, rows], O, L, "largest sample")
    check_grad(res["dq"][0, rows, hi], oracle.diffusion_grad_q_rows(qh, kh, vh, dh, b, scale, rows),
               "dq", "largest sample")
    # The last two keys of each half lie in its last block (63 keys) and are
    # seen only by the rows of that block (no noisy row sees a clean key of
    # the last block), so only
    # those rows' statistics are needed; the others get probability 0 for
    # these keys and are left at zero.
    cols = np.array([n - 2, n - 1, 2 * n - 2, 2 * n - 1])
    last = (n - 1) // b * b
    seen = np.r_[last:n, n + last:2 * n]
    Of = np.zeros((2 * n, D))
    Lf = np.zeros(2 * n)
    Of[seen], Lf[seen] = oracle.diffusion_forward_rows(qh, kh, vh, b, scale, seen)
    dk_ref, dv_ref = oracle.diffusion_grad_kv_cols(qh, kh, vh, dh, Of, Lf, b, scale, cols)
    check_grad(res["dk"][0, cols, hi], dk_ref, "dk", "largest sample")
    check_grad(res["dv"][0, cols, hi], dv_ref, "dv", "largest sample")


# ---------------------------------------------------------------------------
# FP8 (E4M3) forward
# ---------------------------------------------------------------------------

def run_fp8(q8, k8, v8, qd, kd, vd, b, scale, causal=False):
    dev = _dev()
    B, T, H, D = q8.shape
    Hkv = k8.shape[2]
    q8, k8, v8, qd, kd, vd = (x.to(dev) for x in (q8, k8, v8, qd, kd, vd))
    out = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    if causal:
        bd.causal_attn_fwd_fp8(q8, k8, v8, qd, kd, vd, out, lse, B, T, H, Hkv, D, scale)
    else:
        bd.diffusion_attn_fwd_fp8(q8, k8, v8, qd, kd, vd, out, lse, B, T // 2, H, Hkv, D, b, scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _fp8_head(q8, k8, v8, qd, kd, vd, bi, h):
    """Dequantized float64 q, k, v of (sample bi, query head h)."""
    G = q8.shape[2] // k8.shape[2]
    u8 = lambda t, hh: t[bi, :, hh].view(torch.uint8).numpy()
    return (oracle.dequantize_e4m3(u8(q8, h), float(qd[bi, h])),
            oracle.dequantize_e4m3(u8(k8, h // G), float(kd[bi, h // G])),
            oracle.dequantize_e4m3(u8(v8, h // G), float(vd[bi, h // G])))


def check_fp8_head(out, lse, q, k, v, b, scale, rows, what, exact_p=False, causal=False):
    """O and LSE of one head against exact attention on the dequantized
    values.  exact_p: every probability is exact in E4M3 (integer scores),
    so the bf16 tolerances apply; otherwise O may also move by the bound of
    the E4M3 rounding of P."""
    if causal:
        O, L = oracle.causal_forward(q, k, v, scale)
        O, L = O[rows], L[rows]
    else:
        O, L = oracle.diffusion_forward_rows(q, k, v, b, scale, rows)
    o = oracle.to_f64(out)
    if exact_p:
        check_fwd(out, lse, O, L, what)
        return
    mask = oracle.causal_mask(q.shape[0], rows) if causal else None
    bound = oracle.fp8_output_bound(q, k, v, b, scale, rows, mask=mask)
    err = np.abs(o - O)
    tol = bound + _halfulp_bf16(O) + 1e-3
    assert np.all(err <= tol), f"{what}: error {err.max():.3g} beyond the E4M3 bound (max {bound.max():.3g})"
    lerr = np.abs(oracle.to_f64(lse) - L).max()
    assert lerr <= LSE_TOL, f"{what}: LSE error {lerr:.3g}"
    print(f"[{what}] fp8 max err {err.max():.3g} (bound up to {bound.max():.3g}), lse err {lerr:.3g}")


FP8_SHAPES = [  # B, n, H, H_kv, D, b
    (1, 128, 2, 2, 64, 4), (2, 129, 3, 3, 128, 16), (1, 300, 4, 2, 128, 7),
    (2, 64, 4, 1, 64, 200), (1, 7, 2, 2, 128, 3), (1, 257, 2, 1, 64, 1),
]


@pytest.mark.parametrize("B,n,H,Hkv,D,b", FP8_SHAPES)
def test_fp8_integer_scores_exact(B, n, H, Hkv, D, b):
    """Scores that are small integers make every probability a power of two,
    exact in E4M3: the FP8 forward must then meet the bf16 tolerances."""
    q8, k8, v8, qd, kd, vd = make_fp8_integer_score_inputs(B, n, H, D, seed=9960 + n + D, H_kv=Hkv)
    scale = math.log(2.0)
    out, lse = run_fp8(q8, k8, v8, qd, kd, vd, b, scale)
    rows = np.arange(2 * n)
    for bi in range(B):
        for h in range(H):
            q, k, v = _fp8_head(q8, k8, v8, qd, kd, vd, bi, h)
            check_fp8_head(out[bi, :, h], lse[bi, h], q, k, v, b, scale, rows,
                           f"fp8 exact n{n} D{D} ({bi},{h})", exact_p=True)


@pytest.mark.parametrize("B,n,H,Hkv,D,b", FP8_SHAPES)
def test_fp8_random_within_bound(B, n, H, Hkv, D, b):
    q8, k8, v8, qd, kd, vd = make_fp8_inputs(B, n, H, D, seed=9970 + n + D, H_kv=Hkv)
    scale = 1 / math.sqrt(D)
    out, lse = run_fp8(q8, k8, v8, qd, kd, vd, b, scale)
    rows = np.arange(2 * n)
    for bi in range(B):
        for h in range(H):
            q, k, v = _fp8_head(q8, k8, v8, qd, kd, vd, bi, h)
            check_fp8_head(out[bi, :, h], lse[bi, h], q, k, v, b, scale, rows, f"fp8 n{n} D{D} ({bi},{h})")


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_negative_scale_and_causal(D):
    q8, k8, v8, qd, kd, vd = make_fp8_inputs(1, 150, 2, D, seed=9980 + D)
    out, lse = run_fp8(q8, k8, v8, qd, kd, vd, 16, -0.2)
    for h in range(2):
        q, k, v = _fp8_head(q8, k8, v8, qd, kd, vd, 0, h)
        check_fp8_head(out[0, :, h], lse[0, h], q, k, v, 16, -0.2, np.arange(300), f"fp8 scale -0.2 D{D}")
    S = 150
    cq, ck, cv = (x[:, :S].contiguous() for x in (q8, k8, v8))
    out, lse = run_fp8(cq, ck, cv, qd, kd, vd, 1, 1 / math.sqrt(D), causal=True)
    for h in range(2):
        q, k, v = _fp8_head(cq, ck, cv, qd, kd, vd, 0, h)
        check_fp8_head(out[0, :, h], lse[0, h], q, k, v, 1, 1 / math.sqrt(D), np.arange(S),
                       f"fp8 causal D{D}", causal=True)


def test_fp8_long_sequence_sampled():
    """The long-sequence shape (B=2, n=8192, H=32, D=128, b=32) in FP8: all
    rows of two heads."""
    B, n, H, D, b = 2, 8192, 32, 128, 32
    q8, k8, v8, qd, kd, vd = make_fp8_inputs(B, n, H, D, seed=9990)
    scale = 1 / math.sqrt(D)
    out, lse = run_fp8(q8, k8, v8, qd, kd, vd, b, scale)
    for bi, h in ((0, 0), (1, 31)):
        q, k, v = _fp8_head(q8, k8, v8, qd, kd, vd, bi, h)
        for r0 in range(0, 2 * n, 4096):
            rows = np.arange(r0, r0 + 4096)
            check_fp8_head(out[bi, rows, h], lse[bi, h, rows], q, k, v, b, scale, rows,
                           f"fp8 long ({bi},{h}) rows {r0}..")


# ---------------------------------------------------------------------------
# Softcapping (scores s -> cap * tanh(s / cap)) through the general entry points
# ---------------------------------------------------------------------------

def run_general(mode, q, k, v, do, b, scale, softcap, cu=None, max_n=None):
    """Forward and backward through bdattn_fwd / bdattn_bwd; batched tensors
    (B, T, heads, D) when cu is None, packed (total, heads, D) otherwise."""
    dev = _dev()
    q, k, v, do = (x.to(dev) for x in (q, k, v, do))
    Hkv = k.shape[-2]
    if cu is None:
        B, T, H, D = q.shape
        n = T // 2 if mode == bd.MODE_DIFFUSION else T
        total, cu_t = 0, None
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    else:
        total, H, D = q.shape
        B, n = len(cu) - 1, max_n
        cu_t = torch.tensor(cu, dtype=torch.int32, device=dev)
        lse = torch.empty((H, total), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bd.bdattn_fwd(mode, q, k, v, out, lse, cu_t, B, n, total, H, Hkv, D, b, scale, softcap)
    wsb = bd.bdattn_bwd_workspace_size(mode, cu is not None, B, n, total, H, Hkv, D)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    bd.bdattn_bwd(mode, q, k, v, out, do, lse, dq, dk, dv, cu_t, B, n, total, H, Hkv, D, b, scale, softcap,
                  ws, wsb)
    torch.cuda.synchronize()
    res = {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    return {key: t.cpu() for key, t in res.items()}


SOFTCAP_SHAPES = [  # B, n, H, H_kv, D, b, cap
    (2, 100, 2, 2, 64, 16, 5.0), (1, 129, 4, 2, 128, 7, 1.0), (2, 300, 4, 1, 64, 64, 2.5),
    (1, 64, 2, 2, 128, 200, 0.5), (1, 257, 8, 2, 128, 32, 20.0),
    (1, 130, 4, 2, 256, 9, 3.0),
    (1, 140, 4, 4, 96, 6, 4.0), (2, 97, 2, 1, 192, 33, 2.0),
]


@pytest.mark.parametrize("B,n,H,Hkv,D,b,cap", SOFTCAP_SHAPES)
def test_softcap_small(B, n, H, Hkv, D, b, cap):
    """Grouped or not, split groups or not, caps from strong (0.5) to mild
    (20): against the oracle with the same cap.  Inputs are scaled up so
    that the cap bites."""
    q, k, v, do = make_inputs(B, n, H, D, seed=10100 + n + D, H_kv=Hkv)
    q = (q.float() * 3).to(torch.bfloat16)
    scale = 1 / math.sqrt(D)
    res = run_general(bd.MODE_DIFFUSION, q, k, v, do, b, scale, cap)
    f = oracle.to_f64
    O, L = oracle.grouped_forward(oracle.diffusion_forward, f(q), f(k), f(v), b=b, scale=scale, softcap=cap)
    G = oracle.grouped_backward(oracle.diffusion_backward, f(q), f(k), f(v), f(do), b=b, scale=scale,
                                softcap=cap)
    tag = f"softcap {cap} n{n} H{H}/{Hkv} D{D} b{b}"
    check_fwd(res["out"], res["lse"], O, L, tag)
    for name, ref in zip(("dq", "dk", "dv"), G):
        check_grad(res[name], ref, name, tag)


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_softcap_causal_and_varlen(D):
    cap, scale = 2.0, -0.3  # a negative scale too: the cap keeps its sign
    q, k, v, do = make_inputs(2, 150, 2, D, seed=10200 + D)
    q = (q.float() * 3).to(torch.bfloat16)
    cq, ck, cv, cdo = (make_causal_view(x) for x in (q, k, v, do))
    res = run_general(bd.MODE_CAUSAL, cq, ck, cv, cdo, 1, scale, cap)
    f = oracle.to_f64
    O, L = oracle.batched(oracle.causal_forward, f(cq), f(ck), f(cv), scale=scale, softcap=cap)
    G = oracle.batched(oracle.causal_backward, f(cq), f(ck), f(cv), f(cdo), scale=scale, softcap=cap)
    check_fwd(res["out"], res["lse"], O, L, f"softcap causal D{D}")
    for name, ref in zip(("dq", "dk", "dv"), G):
        check_grad(res[name], ref, name, f"softcap causal D{D}")
    ns = [70, 0, 129, 33]
    pq, pk, pv, pdo, cu = make_varlen_inputs(ns, 4, D, seed=10300 + D, H_kv=2)
    pq = (pq.float() * 3).to(torch.bfloat16)
    res = run_general(bd.MODE_DIFFUSION, pq, pk, pv, pdo, 8, scale, cap, cu=cu, max_n=max(ns))
    O, L = oracle.varlen_forward(oracle.diffusion_forward, f(pq), f(pk), f(pv), cu, b=8, scale=scale,
                                 softcap=cap)
    G = oracle.varlen_backward(oracle.diffusion_backward, f(pq), f(pk), f(pv), f(pdo), cu, b=8,
                               scale=scale, softcap=cap)
    check_fwd(res["out"], res["lse"], O, L, f"softcap varlen D{D}")
    for name, ref in zip(("dq", "dk", "dv"), G):
        check_grad(res[name], ref, name, f"softcap varlen D{D}")


def test_general_entry_points_without_softcap_are_the_specific_ones():
    q, k, v, do = make_inputs(2, 200, 4, 128, seed=10400, H_kv=2)
    g = run_general(bd.MODE_DIFFUSION, q, k, v, do, 8, 0.1, 0.0)
    s_ = run_grouped(q, k, v, do, 8, 0.1)
    for key in g:
        assert torch.equal(g[key], s_[key]), key


def test_softcap_workload_heads():
    """The short-sequence workload with a cap of 2 (c2: B=4, n=1024, H=16,
    D=64, b=4), whole heads.  Its scaled scores reach about +-4, so the cap
    bites (tanh(2) = 0.96) while the inputs keep the workload's N(0, 1)
    draws, the regime the forward tolerance is stated for."""
    w = WORKLOADS["c2"]
    q, k, v, do = make_workload_inputs(w)
    scale = 1 / math.sqrt(w.D)
    cap = 2.0
    res = run_general(bd.MODE_DIFFUSION, q, k, v, do, w.b, scale, cap)
    f = oracle.to_f64
    for bi, hi in ((0, 0), (3, 15)):
        sl = lambda x: f(x[bi:bi + 1, :, hi:hi + 1])
        O, L = oracle.batched(oracle.diffusion_forward, sl(q), sl(k), sl(v), b=w.b, scale=scale, softcap=cap)
        G = oracle.batched(oracle.diffusion_backward, sl(q), sl(k), sl(v), sl(do), b=w.b, scale=scale,
                           softcap=cap)
        pick = lambda t: t[bi:bi + 1, :, hi:hi + 1]
        check_fwd(pick(res["out"]), res["lse"][bi:bi + 1, hi:hi + 1], O, L, f"softcap c2 ({bi},{hi})")
        for name, ref in zip(("dq", "dk", "dv"), G):
            check_grad(pick(res[name]), ref, name, f"softcap c2 ({bi},{hi})")


def test_softcap_autograd():
    dev = _dev()
    q, k, v, do = make_inputs(1, 96, 2, 64, seed=10500)
    ref = run_general(bd.MODE_DIFFUSION, q, k, v, do, 4, 0.125, 3.0)
    tq, tk, tv = (x.to(dev).requires_grad_() for x in (q, k, v))
    out, lse = bd.diffusion_attn_func(tq, tk, tv, 4, softmax_scale=0.125, return_lse=True, softcap=3.0)
    out.backward(do.to(dev))
    assert torch.equal(out.detach().cpu(), ref["out"])
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert torch.equal(t.grad.cpu(), ref[name]), name


def test_split_groups_and_varlen_are_bitwise_reproducible():
    """The split-group partials are summed in a fixed order and nothing uses
    atomics: repeated calls give the same bits, also for packed batches."""
    w = GQA_WORKLOADS["g3"]
    q, k, v, do = make_workload_inputs(w)
    scale = 1 / math.sqrt(w.D)
    a = run_grouped(q, k, v, do, w.b, scale)
    b = run_grouped(q, k, v, do, w.b, scale)
    for key in a:
        assert torch.equal(a[key], b[key]), key
    ns = [300, 0, 77, 1024]
    pq, pk, pv, pdo, cu = make_varlen_inputs(ns, 8, 64, seed=10600, H_kv=1)
    a = run_varlen(pq, pk, pv, pdo, cu, max(ns), 16, 0.125)
    b = run_varlen(pq, pk, pv, pdo, cu, max(ns), 16, 0.125)
    for key in a:
        assert torch.equal(a[key], b[key]), key


# ---------------------------------------------------------------------------
# Randomised combinations of every option, compared in full
# ---------------------------------------------------------------------------

def _random_case(i):
    """The i-th of a fixed list of small problems: mode, batched or packed
    layout, head grouping, head dimension, block size (tile-aligned or not,
    longer than a half), softcap and the sign and size of the scale, drawn
    from a generator seeded with i."""
    r = np.random.default_rng(20250 + i)
    mode = bd.MODE_CAUSAL if r.random() < 0.3 else bd.MODE_DIFFUSION
    packed = r.random() < 0.4
    D = int(r.choice(HEAD_DIMS))
    Hkv = int(r.integers(1, 4))
    H = Hkv * int(r.choice([1, 1, 2, 3, 4]))
    if packed:
        ns = [int(x) for x in r.integers(0, 260, size=int(r.integers(1, 5)))]
        if max(ns) == 0:
            ns[0] = 1  # at least one non-empty sample
        n = max(ns)
    else:
        ns = None
        n = int(r.integers(1, 300))
    b = int(r.choice([1, 2, 3, 4, 5, 8, 16, 31, 32, 33, 48, 64, 100, n + 3]))
    cap = float(r.choice([0.0, 0.0, 0.0, 1.5, 6.0]))
    scale = float(r.choice([1.0, 1.0, -1.0, 0.5, 2.0])) / math.sqrt(D)
    B = 1 if packed else int(r.integers(1, 4))
    return dict(mode=mode, packed=packed, D=D, H=H, Hkv=Hkv, ns=ns, n=n, b=b, cap=cap, scale=scale, B=B)


def check_fwd_rounding(o, lse, o_ref, lse_ref, pv_ref, what):
    """Forward check for scales other than the workloads' 1/sqrt(D): an
    element is held to 1e-2, or, where that is exceeded, to what rounding
    can cost it: half a bf16 ulp of the output plus the bf16 rounding of the
    probabilities fed to P.V, at most 2^-9 sum_j P_ij |v_j| (taken as 2^-8,
    with 1e-3 for the float32 accumulation).  pv_ref is the oracle's
    sum_j P_ij |v_j| (its forward on |v|).  LSE as in check_fwd."""
    o = oracle.to_f64(o)
    err = np.abs(o - o_ref)
    bound = np.maximum(FWD_TOL, _halfulp_bf16(o_ref) + 2.0 ** -8 * pv_ref + 1e-3)
    worst = np.argmax(err - bound)
    assert np.all(err <= bound), (f"{what}: forward error {err.flat[worst]:.3g} > bound {bound.flat[worst]:.3g} "
                                  f"(|O_ref| {abs(o_ref.flat[worst]):.3g}, P|V| {pv_ref.flat[worst]:.3g})")
    lerr = np.abs(oracle.to_f64(lse) - lse_ref).max()
    assert lerr <= LSE_TOL, f"{what}: LSE max-abs error {lerr:.3g} > {LSE_TOL}"
    print(f"[{what}] fwd max err {err.max():.3g} (elements past 1e-2: {int((err > FWD_TOL).sum())}), "
          f"lse err {lerr:.3g}")


@pytest.mark.parametrize("i", range(96))
def test_random_configurations(i):
    c = _random_case(i)
    f = oracle.to_f64
    causal = c["mode"] == bd.MODE_CAUSAL
    b = 1 if causal else c["b"]
    tag = (f"case {i}: {'causal' if causal else 'diffusion'} {'packed ' + str(c['ns']) if c['packed'] else 'B=' + str(c['B']) + ' n=' + str(c['n'])}"
           f" H{c['H']}/{c['Hkv']} D{c['D']} b{b} cap {c['cap']} scale {c['scale']:.3g}")
    print(tag, flush=True)
    kw = dict(scale=c["scale"], softcap=c["cap"])
    if not causal:
        kw["b"] = b
    fn_f = oracle.causal_forward if causal else oracle.diffusion_forward
    fn_b = oracle.causal_backward if causal else oracle.diffusion_backward
    if c["packed"]:
        q, k, v, do, cu = make_varlen_inputs(c["ns"], c["H"], c["D"], seed=30000 + i, H_kv=c["Hkv"], causal=causal)
        res = run_general(c["mode"], q, k, v, do, b, c["scale"], c["cap"], cu=cu, max_n=c["n"])
        O, L = oracle.varlen_forward(fn_f, f(q), f(k), f(v), cu, **kw)
        PV, _ = oracle.varlen_forward(fn_f, f(q), f(k), np.abs(f(v)), cu, **kw)
        G = oracle.varlen_backward(fn_b, f(q), f(k), f(v), f(do), cu, **kw)
    else:
        q, k, v, do = make_inputs(c["B"], c["n"], c["H"], c["D"], seed=30000 + i, H_kv=c["Hkv"])
        if causal:
            q, k, v, do = (make_causal_view(x) for x in (q, k, v, do))
        res = run_general(c["mode"], q, k, v, do, b, c["scale"], c["cap"])
        O, L = oracle.grouped_forward(fn_f, f(q), f(k), f(v), **kw)
        PV, _ = oracle.grouped_forward(fn_f, f(q), f(k), np.abs(f(v)), **kw)
        G = oracle.grouped_backward(fn_b, f(q), f(k), f(v), f(do), **kw)
    if abs(c["scale"] * math.sqrt(c["D"])) == 1.0:
        check_fwd(res["out"], res["lse"], O, L, tag)
    else:
        check_fwd_rounding(res["out"], res["lse"], O, L, PV, tag)
    for name, ref in zip(("dq", "dk", "dv"), G):
        check_grad(res[name], ref, name, tag)
