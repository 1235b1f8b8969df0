"""Accuracy statistics of the HIP path beyond the maximum error (Fast
Diffusion Attention, "Accuracy").

The pages hold their kernels to FlashAttention's methodology: against a
reference computed in higher precision from the same low-precision inputs,
the error of the output, the log-sum-exp and dQ / dK / dV must be at most
twice the error of a straightforward PyTorch implementation in the same
precision; over many random problems the relative bias and the relative
scale error of the output and of every gradient must average to zero within
4 standard errors, and be no larger than twice PyTorch's.

Readings (the pages define neither statistic nor the PyTorch program):
  * the higher-precision reference is the float64 oracle (the pages name
    float32; float64 is stricter);
  * the straightforward implementation is plain PyTorch on the CPU in
    bfloat16: S = (q k^T) * scale, the mask as -inf, softmax, P v, the
    log-sum-exp with torch.logsumexp, and the gradients by autograd, every
    intermediate a bfloat16 tensor;
  * for a tensor X with reference R (one problem, all its elements), the
    relative bias is sum(X - R) / sum|R| and the relative scale error is
    <X, R> / <R, R> - 1 (the least-squares factor between X and R, less 1);
  * "no larger than twice those of PyTorch" compares the root mean square
    of each statistic over the problems.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from test_gpu_parity import run_diffusion
from workloads import make_inputs

pytestmark = pytest.mark.gpu

NAMES = ("out", "lse", "dq", "dk", "dv")


def torch_bf16_reference(q, k, v, do, b, scale):
    """The straightforward bfloat16 PyTorch program on the CPU, for (B, 2n, H, D)
    bf16 tensors; returns float64 arrays in the oracle's layouts."""
    B, T, H, D = q.shape
    n = T // 2
    mask = torch.from_numpy(oracle.block_diffusion_mask(n, b))
    to_bh = lambda x: x.permute(0, 2, 1, 3).reshape(B * H, T, D).contiguous()
    tq, tk, tv = (to_bh(x).clone().requires_grad_() for x in (q, k, v))
    s = torch.matmul(tq, tk.transpose(1, 2).contiguous()) * scale
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    o = torch.matmul(torch.softmax(s, dim=-1), tv)
    o.backward(to_bh(do))
    back = lambda x: oracle.to_f64(x.detach().reshape(B, H, T, D).permute(0, 2, 1, 3))
    return {"out": back(o), "lse": oracle.to_f64(lse.detach().reshape(B, H, T)),
            "dq": back(tq.grad), "dk": back(tk.grad), "dv": back(tv.grad)}


def oracle_reference(q, k, v, do, b, scale):
    f = oracle.to_f64
    O, L = oracle.batched(oracle.diffusion_forward, f(q), f(k), f(v), b=b, scale=scale)
    dQ, dK, dV = oracle.batched(oracle.diffusion_backward, f(q), f(k), f(v), f(do), b=b, scale=scale)
    return {"out": O, "lse": L, "dq": dQ, "dk": dK, "dv": dV}


MAX_ERR_CASES = [  # B, n, H, D, b
    (1, 128, 2, 64, 4), (2, 300, 2, 128, 16), (1, 129, 3, 64, 3), (1, 256, 2, 128, 1),
    (2, 100, 2, 96, 7), (1, 200, 2, 192, 32), (1, 150, 2, 256, 200),
]


@pytest.mark.parametrize("B,n,H,D,b", MAX_ERR_CASES)
def test_error_at_most_twice_pytorch_bf16(B, n, H, D, b):
    q, k, v, do = make_inputs(B, n, H, D, seed=40000 + n + D + b)
    scale = 1 / math.sqrt(D)
    ours = {key: oracle.to_f64(t) for key, t in run_diffusion(q, k, v, do, b, scale).items()}
    ref = oracle_reference(q, k, v, do, b, scale)
    pt = torch_bf16_reference(q, k, v, do, b, scale)
    for key in NAMES:
        e_ours = np.abs(ours[key] - ref[key]).max()
        e_pt = np.abs(pt[key] - ref[key]).max()
        print(f"[n{n} D{D} b{b}] {key}: ours {e_ours:.3g}, PyTorch bf16 {e_pt:.3g}")
        assert e_ours <= 2 * e_pt, f"{key}: error {e_ours:.3g} > 2 x PyTorch bf16's {e_pt:.3g}"


def _stats(x, r):
    d = (x - r).ravel()
    r = r.ravel()
    return d.sum() / np.abs(r).sum(), np.dot(x.ravel(), r) / np.dot(r, r) - 1.0


def _problem(i):
    g = np.random.default_rng(41000 + i)
    n = int(g.integers(32, 300))
    D = int(g.choice([64, 128]))
    b = int(g.choice([1, 3, 4, 16, 32, 64, n + 1]))
    return 1, n, 2, D, b


STAT_PROBLEMS = 48


def test_no_systematic_error():
    """Over 48 seeded random problems (one sample, two heads, n from 32 to
    299, D 64 or 128, block sizes 1 to longer than the half): the relative
    bias and the relative scale error of O, dQ, dK and dV average to zero
    within 4 standard errors, and their root mean square over the problems
    is at most twice PyTorch bf16's."""
    stats = {key: {"ours": [], "pt": []} for key in ("out", "dq", "dk", "dv")}
    for i in range(STAT_PROBLEMS):
        B, n, H, D, b = _problem(i)
        q, k, v, do = make_inputs(B, n, H, D, seed=42000 + i)
        scale = 1 / math.sqrt(D)
        ours = {key: oracle.to_f64(t) for key, t in run_diffusion(q, k, v, do, b, scale).items()}
        ref = oracle_reference(q, k, v, do, b, scale)
        pt = torch_bf16_reference(q, k, v, do, b, scale)
        for key in stats:
            stats[key]["ours"].append(_stats(ours[key], ref[key]))
            stats[key]["pt"].append(_stats(pt[key], ref[key]))
    for key, st in stats.items():
        ours = np.array(st["ours"])
        pt = np.array(st["pt"])
        for c, label in ((0, "relative bias"), (1, "relative scale error")):
            x = ours[:, c]
            mean, se = x.mean(), x.std(ddof=1) / math.sqrt(len(x))
            rms, rms_pt = math.sqrt((x * x).mean()), math.sqrt((pt[:, c] ** 2).mean())
            print(f"{key} {label}: mean {mean:.3g} (standard error {se:.3g}), rms {rms:.3g}, "
                  f"PyTorch bf16 rms {rms_pt:.3g}")
            assert abs(mean) <= 4 * se, f"{key}: {label} averages {mean:.3g}, beyond 4 standard errors ({se:.3g})"
            assert rms <= 2 * rms_pt, f"{key}: {label} rms {rms:.3g} > 2 x PyTorch bf16's {rms_pt:.3g}"
