"""Seeded synthetic inputs for block-diffusion attention.

This module is shared by the CPU oracle, the tests and the benchmark.  It
holds shapes, seeds and random draws only -- none of the attention
arithmetic -- so that the oracle and the HIP path see identical bits
without sharing any code that computes the method.

Layout (Fast Diffusion Attention, "TL;DR" usage line): q, k, v and the
output gradient have shape (batch, 2n, heads, headdim); along dim 1 the
first n tokens are the noisy half and the last n the clean half.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws
float32 N(0, 1) values in the order q, k, v, dout; each is rounded to
bfloat16 (round-to-nearest-even, torch's ``.to``).  The pages benchmark on
FlashAttention's benchmark shapes, which they do not list; the synthetic
workloads below stand in for them.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Sequence, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One problem: B samples of 2n tokens, H query heads of width D reading
    H_kv key/value heads (0: H_kv = H), block size b."""

    name: str
    B: int
    n: int
    H: int
    D: int
    b: int
    seed: int
    H_kv: int = 0

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        return (self.B, 2 * self.n, self.H, self.D)

    def describe(self) -> str:
        kv = f" H_kv={self.kv_heads}" if self.kv_heads != self.H else ""
        return (f"{self.name}: B={self.B} n={self.n} (2n={2 * self.n}) H={self.H}{kv} "
                f"D={self.D} b={self.b} seed={self.seed}")


def _c5(D: int, b: int) -> Workload:
    return Workload(f"c5_d{D}_b{b}", B=4, n=4096, H=16, D=D, b=b, seed=1005 if D == 64 else 1006)


# The five workloads of the block-diffusion attention study: a tiny case, a
# short-sequence case, a medium case with the causal yardstick, the
# long-sequence case (the largest, on which throughput is quoted) and a
# block-size sweep with tile-misaligned and tile-sized blocks.
WORKLOADS: Dict[str, Workload] = {
    "c1": Workload("c1", B=1, n=128, H=2, D=64, b=4, seed=1001),
    "c2": Workload("c2", B=4, n=1024, H=16, D=64, b=4, seed=1002),
    "c3": Workload("c3", B=8, n=2048, H=16, D=128, b=16, seed=1003),
    "c4": Workload("c4", B=2, n=8192, H=32, D=128, b=32, seed=1004),
}
for _D in (64, 128):
    for _b in (1, 3, 48, 128, 256):
        _w = _c5(_D, _b)
        WORKLOADS[_w.name] = _w

# Head dimensions other than 64 and 128, on the block-size-sweep problem
# (n = 4096, b = 48): at D = 256 with half the heads (the same tokens, bytes
# and FLOPs as its D = 128 member); at D = 192 and D = 96 with its 16 heads.
HEAD_DIM_WORKLOADS: Dict[str, Workload] = {
    "h1": Workload("h1", B=4, n=4096, H=8, D=256, b=48, seed=1031),
    "h2": Workload("h2", B=4, n=4096, H=16, D=192, b=48, seed=1032),
    "h3": Workload("h3", B=4, n=4096, H=16, D=96, b=48, seed=1033),
}

# Grouped-query problems (query heads sharing key/value heads): the
# short-sequence regime in which the pages report the grouped backward's
# gain (512 to 1K tokens per half), the long-sequence problem with four
# query heads per key/value head, and multi-query attention (one key/value
# head).  Parity cases and side measurements; throughput is quoted on c4.
GQA_WORKLOADS: Dict[str, Workload] = {
    "g1": Workload("g1", B=8, n=1024, H=32, D=128, b=16, seed=1011, H_kv=8),
    "g2": Workload("g2", B=2, n=8192, H=32, D=128, b=32, seed=1012, H_kv=8),
    "g3": Workload("g3", B=4, n=2048, H=16, D=64, b=4, seed=1013, H_kv=1),
}



@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """B packed samples whose half lengths n_b are drawn uniformly from
    [n_min, n_max] (CPU torch.Generator seeded with len_seed, drawn before
    and apart from the tensors); H query heads, H_kv key/value heads
    (0: H), width D, block size b; tensors from ``seed``."""

    name: str
    B: int
    n_min: int
    n_max: int
    H: int
    D: int
    b: int
    seed: int
    len_seed: int
    H_kv: int = 0

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def half_lengths(self) -> List[int]:
        g = torch.Generator(device="cpu")
        g.manual_seed(int(self.len_seed))
        return torch.randint(self.n_min, self.n_max + 1, (self.B,), generator=g).tolist()

    def describe(self) -> str:
        kv = f" H_kv={self.kv_heads}" if self.kv_heads != self.H else ""
        ns = self.half_lengths
        return (f"{self.name}: varlen B={self.B} n_b in [{self.n_min}, {self.n_max}] "
                f"(total {2 * sum(ns)} tokens, max n {max(ns)}) H={self.H}{kv} D={self.D} "
                f"b={self.b} seed={self.seed}")


# Packed batches of samples of random lengths (the pages' SFT-style varlen
# workload): multi-head D=128, and grouped heads at D=64 with short samples.
VARLEN_WORKLOADS: Dict[str, VarlenWorkload] = {
    "v1": VarlenWorkload("v1", B=16, n_min=256, n_max=4096, H=16, D=128, b=32, seed=1021, len_seed=1022),
    "v2": VarlenWorkload("v2", B=24, n_min=64, n_max=2048, H=32, D=64, b=4, seed=1023, len_seed=1024,
                         H_kv=8),
}

LARGEST = "c4"


def make_inputs(B: int, n: int, H: int, D: int, seed: int, with_dout: bool = True,
                H_kv: int = 0):
    """Return bf16 CPU tensors (q, k, v, dout): q and dout of shape
    (B, 2n, H, D), k and v of shape (B, 2n, H_kv, D) (H_kv = 0: H).

    Draw order is fixed (q, k, v, dout) so that every consumer of a seed
    sees the same bits.  ``with_dout=False`` still draws nothing extra and
    returns dout as None.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    kv = H_kv or H
    shapes = [(B, 2 * n, H, D), (B, 2 * n, kv, D), (B, 2 * n, kv, D), (B, 2 * n, H, D)]
    out = []
    for shape in shapes[:4 if with_dout else 3]:
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        out.append(x.to(torch.bfloat16))
    if not with_dout:
        out.append(None)
    return tuple(out)


def make_workload_inputs(w: Workload, with_dout: bool = True):
    return make_inputs(w.B, w.n, w.H, w.D, w.seed, with_dout=with_dout, H_kv=w.H_kv)


def make_causal_view(x: torch.Tensor) -> torch.Tensor:
    """View (B, 2n, H, D) as (2B, n, H, D): each half becomes one sequence.

    This is a pure reshape (no arithmetic): the same bytes seen as 2B
    sequences of length n, the equal-work causal problem.
    """
    B, twon, H, D = x.shape
    return x.reshape(2 * B, twon // 2, H, D)


def cu_seqlens(half_lengths: Sequence[int], causal: bool = False) -> List[int]:
    """Cumulative token offsets of packed samples: sample b occupies tokens
    [cu[b], cu[b+1]), 2 n_b of them ([noisy | clean]), or n_b in the causal
    layout."""
    cu = [0]
    for nb in half_lengths:
        cu.append(cu[-1] + (nb if causal else 2 * nb))
    return cu


def make_varlen_inputs(half_lengths: Sequence[int], H: int, D: int, seed: int, H_kv: int = 0,
                       causal: bool = False):
    """Packed bf16 CPU tensors (q, k, v, dout) of shape (total, heads, D) --
    q and dout with H heads, k and v with H_kv (0: H) -- and the offsets
    ``cu``.  Same draw order and rounding as ``make_inputs``."""
    cu = cu_seqlens(half_lengths, causal)
    total = cu[-1]
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    kv = H_kv or H
    out = []
    for heads in (H, kv, kv, H):
        out.append(torch.randn((total, heads, D), generator=g, dtype=torch.float32).to(torch.bfloat16))
    return (*out, cu)


def make_varlen_workload_inputs(w: VarlenWorkload):
    return make_varlen_inputs(w.half_lengths, w.H, w.D, w.seed, H_kv=w.H_kv)


def make_fp8_inputs(B: int, n: int, H: int, D: int, seed: int, H_kv: int = 0):
    """FP8 (OCP E4M3) inputs of the FP8 forward pass and their descale factors.

    Draws float32 N(0, 1) q (H heads), k and v (H_kv heads, 0: H) in that
    order, then per (sample, head) descale exponents u in [-3, 1] for q, k,
    v; each tensor is divided by 2^u and cast to float8_e4m3fn (torch's
    round-to-nearest-even).  Returns (q8, k8, v8, q_descale [B][H],
    k_descale [B][H_kv], v_descale [B][H_kv]), all CPU tensors."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    kv = H_kv or H
    x = [torch.randn((B, 2 * n, h, D), generator=g, dtype=torch.float32) for h in (H, kv, kv)]
    ds = [torch.exp2(torch.randint(-3, 2, (B, h), generator=g).to(torch.float32)) for h in (H, kv, kv)]
    q8, k8, v8 = ((t / d[:, None, :, None]).to(torch.float8_e4m3fn) for t, d in zip(x, ds))
    return q8, k8, v8, ds[0], ds[1], ds[2]


def make_fp8_integer_score_inputs(B: int, n: int, H: int, D: int, seed: int, H_kv: int = 0):
    """FP8 inputs whose scores are small integers: every row of q and k has
    two entries of +-1 (descale 1), so q.k lies in [-2, 2]; v as in
    ``make_fp8_inputs``.  With scale = ln 2 the scaled base-2 scores are
    integers, so every unnormalised probability is a power of two (exact in
    E4M3).  Returns the same six tensors."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    kv = H_kv or H

    def sparse(h):
        t = torch.zeros((B, 2 * n, h, D), dtype=torch.float32)
        rows = B * 2 * n * h
        idx = torch.argsort(torch.rand((rows, D), generator=g), dim=1)[:, :2]  # two distinct columns
        sgn = torch.randint(0, 2, (rows, 2), generator=g).to(torch.float32) * 2 - 1
        t.view(-1, D).scatter_(1, idx, sgn)
        return t.to(torch.float8_e4m3fn)

    q8, k8 = sparse(H), sparse(kv)
    v = torch.randn((B, 2 * n, kv, D), generator=g, dtype=torch.float32)
    vd = torch.exp2(torch.randint(-3, 2, (B, kv), generator=g).to(torch.float32))
    v8 = (v / vd[:, None, :, None]).to(torch.float8_e4m3fn)
    return q8, k8, v8, torch.ones(B, H), torch.ones(B, kv), vd
