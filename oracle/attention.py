"""Dense float64 reference for attention under the block-diffusion mask.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain, slow and
meant to be checked by eye against the pages.

Sources (cited by page title and section):

* Mask -- "Fast Diffusion Attention", section "Block diffusion in one
  picture": on the concatenation [noisy | clean] of a sample, a noisy
  block attends to itself in both directions and to every clean block
  before it; a clean block attends to itself and the clean blocks before
  it; every other (query, key) pair is masked.  The "right yardstick"
  section fixes "before" as strictly earlier: noisy row-block i sees the
  i - 1 earlier clean blocks plus its own noisy block.
* Softmax attention and its numerically stable form -- "FlashAttention:
  Exact Attention Without Materialization", sections 1 and 2.3 (subtract
  the row maximum before exponentiating).
* Saved statistic -- same page, section 4.5: the forward pass keeps the
  output and one log-sum-exp per query row.
* Backward -- the analytic gradient of softmax attention (the function the
  recompute-based backward of section 4.5 differentiates):
  dV = P^T dO, dP = dO V^T, delta_i = sum_j P_ij dP_ij,
  dS = P * (dP - delta), dQ = scale * dS K, dK = scale * dS^T Q.

Readings where the pages are silent:

* Blocks are consecutive runs of b tokens from the start of each half; the
  last block of a half is shorter when b does not divide n.  Block
  numbering restarts in each half, so noisy block i and clean block i
  cover the same positions.
* The scale multiplies the scores before the softmax.
* The log-sum-exp is the natural logarithm and includes the scale.
* The causal yardstick is top-left causal: row i of a sequence sees keys
  0..i of the same sequence.
* Softcapping (named by Fast Diffusion Attention, "Accuracy", among what
  its tests cover; defined by flash-attention, whose interface the pages
  follow): with cap > 0 the scaled scores s become cap * tanh(s / cap)
  before the softmax; the backward multiplies dS by 1 - tanh^2(s / cap)
  (the derivative of that map).  cap = 0 leaves the scores as they are.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# Masks
# --------------------------------------------------------------------------

def block_diffusion_mask(n: int, b: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Explicit boolean mask of a [noisy | clean] sequence of 2n tokens.

    Returns M with M[r, c] True when query r may attend to key c, for the
    query rows ``rows`` (default: all 2n rows) and all 2n keys.  Rows and
    columns 0..n-1 are the noisy half, n..2n-1 the clean half.
    """
    if n < 1 or b < 1:
        raise ValueError("n and b must be positive")
    r = np.arange(2 * n) if rows is None else np.asarray(rows, dtype=np.int64)
    r = r[:, None]
    c = np.arange(2 * n)[None, :]
    r_noisy = r < n
    c_noisy = c < n
    r_block = np.where(r_noisy, r, r - n) // b   # block index inside its own half
    c_block = np.where(c_noisy, c, c - n) // b
    noisy_sees_own_block = r_noisy & c_noisy & (c_block == r_block)
    noisy_sees_earlier_clean = r_noisy & ~c_noisy & (c_block < r_block)
    clean_block_causal = ~r_noisy & ~c_noisy & (c_block <= r_block)
    return noisy_sees_own_block | noisy_sees_earlier_clean | clean_block_causal


def causal_mask(S: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Top-left causal mask of one sequence of S tokens: key c <= query r."""
    r = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    return np.arange(S)[None, :] <= r[:, None]


# --------------------------------------------------------------------------
# Dense masked softmax attention (one head)
# --------------------------------------------------------------------------

def _masked_softmax_stats(S: np.ndarray, M: np.ndarray):
    """Row max, probabilities and log-sum-exp of S restricted to M.

    Masked scores are -inf; the maximum is subtracted before exp (the
    numerically stable softmax).  Every row is required to see at least
    one key.
    """
    if not np.all(M.any(axis=1)):
        raise ValueError("a query row sees no key")
    S = np.where(M, S, -np.inf)
    m = S.max(axis=1)
    E = np.exp(S - m[:, None])                  # exp(-inf) = 0 on masked pairs
    ell = E.sum(axis=1)
    P = E / ell[:, None]
    lse = m + np.log(ell)
    return P, lse


def _scores(q, k, scale, softcap):
    """Scaled scores, softcapped when softcap > 0; also returns the factor
    d(capped)/d(scaled) = 1 - tanh^2 (None without softcap)."""
    S = scale * (q @ k.T)
    if not softcap:
        return S, None
    T = np.tanh(S / softcap)
    return softcap * T, 1.0 - T * T


def masked_attention_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                             M: np.ndarray, scale: float, softcap: float = 0.0) -> Tuple[np.ndarray, np.ndarray]:
    """O = softmax(scale * q k^T restricted to M) v and its row log-sum-exp.

    q: (Nq, D), k and v: (Nk, D), M: (Nq, Nk) boolean.  float64 throughout.
    """
    S, _ = _scores(q, k, scale, softcap)
    P, lse = _masked_softmax_stats(S, M)
    return P @ v, lse


def masked_attention_backward(q, k, v, dout, M, scale, softcap: float = 0.0):
    """Analytic gradients (dq, dk, dv) of sum(dout * O) for masked attention."""
    S, dcap = _scores(q, k, scale, softcap)
    P, _ = _masked_softmax_stats(S, M)
    dv = P.T @ dout
    dP = dout @ v.T
    delta = (P * dP).sum(axis=1)
    dS = P * (dP - delta[:, None])
    if dcap is not None:
        dS = dS * dcap
    dq = scale * (dS @ k)
    dk = scale * (dS.T @ q)
    return dq, dk, dv


# --------------------------------------------------------------------------
# Block-diffusion attention of one (sample, head): q, k, v of shape (2n, D)
# --------------------------------------------------------------------------

def _half_len(x: np.ndarray) -> int:
    if x.shape[0] % 2:
        raise ValueError("sequence length must be 2n")
    return x.shape[0] // 2


def diffusion_forward(q, k, v, b: int, scale: float, softcap: float = 0.0):
    """(O, LSE) of one head: O (2n, D), LSE (2n,), natural log."""
    n = _half_len(q)
    return masked_attention_forward(q, k, v, block_diffusion_mask(n, b), scale, softcap)


def diffusion_backward(q, k, v, dout, b: int, scale: float, softcap: float = 0.0):
    """(dq, dk, dv) of one head."""
    n = _half_len(q)
    return masked_attention_backward(q, k, v, dout, block_diffusion_mask(n, b), scale, softcap)


def diffusion_forward_rows(q, k, v, b: int, scale: float, rows: Sequence[int], softcap: float = 0.0):
    """O and LSE of the query rows ``rows`` only (same definition, fewer rows)."""
    n = _half_len(q)
    rows = np.asarray(rows, dtype=np.int64)
    M = block_diffusion_mask(n, b, rows)
    return masked_attention_forward(q[rows], k, v, M, scale, softcap)


def diffusion_grad_q_rows(q, k, v, dout, b: int, scale: float, rows: Sequence[int],
                          softcap: float = 0.0):
    """dQ of the query rows ``rows``: each row needs only its own softmax."""
    n = _half_len(q)
    rows = np.asarray(rows, dtype=np.int64)
    M = block_diffusion_mask(n, b, rows)
    S, dcap = _scores(q[rows], k, scale, softcap)
    P, _ = _masked_softmax_stats(S, M)
    dP = dout[rows] @ v.T
    delta = (P * dP).sum(axis=1)
    dS = P * (dP - delta[:, None])
    if dcap is not None:
        dS = dS * dcap
    return scale * (dS @ k)


def diffusion_grad_kv_cols(q, k, v, dout, out, lse, b: int, scale: float,
                           cols: Sequence[int], softcap: float = 0.0):
    """dK and dV of the key columns ``cols``.

    A key's gradient sums over every query that sees it, so it needs each
    query's full-row statistics: ``lse`` (the log-sum-exp of every row)
    and ``out`` (the exact output of every row, giving
    delta_i = sum_j P_ij dP_ij = dout_i . out_i).  Both must come from this
    oracle's own forward pass.  P_ij = exp(S_ij - LSE_i) is the softmax
    written with its normaliser.
    """
    n = _half_len(q)
    cols = np.asarray(cols, dtype=np.int64)
    M = block_diffusion_mask(n, b)[:, cols]
    S, dcap = _scores(q, k[cols], scale, softcap)
    P = np.where(M, np.exp(np.where(M, S, 0.0) - lse[:, None]), 0.0)
    dP = dout @ v[cols].T
    delta = (dout * out).sum(axis=1)
    dS = P * (dP - delta[:, None])
    if dcap is not None:
        dS = dS * dcap
    dv = P.T @ dout
    dk = scale * (dS.T @ q)
    return dk, dv


# --------------------------------------------------------------------------
# Causal yardstick of one sequence: q, k, v of shape (S, D)
# --------------------------------------------------------------------------

def causal_forward(q, k, v, scale: float, softcap: float = 0.0):
    return masked_attention_forward(q, k, v, causal_mask(q.shape[0]), scale, softcap)


def causal_backward(q, k, v, dout, scale: float, softcap: float = 0.0):
    return masked_attention_backward(q, k, v, dout, causal_mask(q.shape[0]), scale, softcap)


# --------------------------------------------------------------------------
# Grouped-query attention: H query heads share H_kv key/value heads
# --------------------------------------------------------------------------
#
# Fast Diffusion Attention, "Ampere and Ada" (the GQA-grouped backward):
# several query heads read one key/value head, and that head's dK / dV is
# the sum of what each of those query heads contributes (the chain rule for
# a shared input).  Which query heads form a group is not stated on the
# pages; the reading taken is flash-attention's (whose call shape the pages
# follow): H_kv consecutive runs of H / H_kv query heads, run j reading
# key/value head j.

def kv_head_of(h: int, H: int, H_kv: int) -> int:
    """Key/value head read by query head h."""
    if H_kv < 1 or H % H_kv or not 0 <= h < H:
        raise ValueError("need 1 <= H_kv, H divisible by H_kv and 0 <= h < H")
    return h // (H // H_kv)


def grouped_forward(fn: Callable, q, k, v, heads: Optional[Sequence[Tuple[int, int]]] = None, **kw):
    """(O, LSE) of q (B, T, H, D) against k, v (B, T, H_kv, D).

    ``fn`` is a one-head forward such as ``diffusion_forward``; query head h
    of sample bi runs it with key/value head ``kv_head_of(h)``.  ``heads``
    restricts the work to the listed (sample, query head) pairs (the other
    entries are NaN).
    """
    B, T, H, D = q.shape
    H_kv = k.shape[2]
    O = np.full((B, T, H, D), np.nan)
    L = np.full((B, H, T), np.nan)
    todo = heads if heads is not None else [(bi, h) for bi in range(B) for h in range(H)]
    for bi, h in todo:
        j = kv_head_of(h, H, H_kv)
        O[bi, :, h], L[bi, h] = fn(q[bi, :, h], k[bi, :, j], v[bi, :, j], **kw)
    return O, L


def grouped_backward(fn: Callable, q, k, v, dout, **kw):
    """(dq, dk, dv) for q, dout (B, T, H, D) and k, v (B, T, H_kv, D).

    ``fn`` is a one-head backward such as ``diffusion_backward``.  dq of a
    query head is that head's own; dk and dv of key/value head j sum the
    contributions of every query head of its group.
    """
    B, T, H, D = q.shape
    H_kv = k.shape[2]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for bi in range(B):
        for h in range(H):
            j = kv_head_of(h, H, H_kv)
            gq, gk, gv = fn(q[bi, :, h], k[bi, :, j], v[bi, :, j], dout[bi, :, h], **kw)
            dq[bi, :, h] = gq
            dk[bi, :, j] += gk
            dv[bi, :, j] += gv
    return dq, dk, dv


def grouped_grad_kv_cols(qs, k, v, douts, outs, lses, b: int, scale: float, cols: Sequence[int]):
    """dK and dV of the key columns ``cols`` of one key/value head.

    ``qs``, ``douts``, ``outs``, ``lses``: one entry per query head of the
    group (each as ``diffusion_grad_kv_cols`` takes them); the result is the
    sum of the heads' contributions.
    """
    dk = dv = 0.0
    for qh, dh, oh, lh in zip(qs, douts, outs, lses):
        gk, gv = diffusion_grad_kv_cols(qh, k, v, dh, oh, lh, b, scale, cols)
        dk = dk + gk
        dv = dv + gv
    return dk, dv


# --------------------------------------------------------------------------
# Variable-length batches: samples of different lengths packed in one tensor
# --------------------------------------------------------------------------
#
# Fast Diffusion Attention, "Hopper" (varlen batches: packed samples of
# different lengths) and "Try it" (the varlen function follows
# flash-attention's varlen call).  Reading taken: sample b occupies the
# packed tokens [cu[b], cu[b+1]); in the diffusion layout those are its
# noisy half followed by its clean half (2 n_b tokens), in the causal
# layout one sequence.  A sample attends only within itself, exactly as
# the batched function on that sample alone.  Per-row statistics are laid
# out [heads][total tokens].

def varlen_forward(fn: Callable, q, k, v, cu: Sequence[int], **kw):
    """(O, LSE) of packed q (total, H, D) against k, v (total, H_kv, D).

    ``fn`` is a one-head forward (``diffusion_forward`` or
    ``causal_forward``-like, taking q, k, v of one sample and head).
    Tokens outside every sample are NaN.
    """
    total, H, D = q.shape
    H_kv = k.shape[1]
    O = np.full((total, H, D), np.nan)
    L = np.full((H, total), np.nan)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 == s0:
            continue                      # an empty sample has no rows
        for h in range(H):
            j = kv_head_of(h, H, H_kv)
            O[s0:s1, h], L[h, s0:s1] = fn(q[s0:s1, h], k[s0:s1, j], v[s0:s1, j], **kw)
    return O, L


def varlen_backward(fn: Callable, q, k, v, dout, cu: Sequence[int], **kw):
    """(dq, dk, dv) of packed tensors; dk and dv of a key/value head sum over
    its query heads.  Tokens outside every sample are NaN."""
    total, H, D = q.shape
    H_kv = k.shape[1]
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 == s0:
            continue
        dk[s0:s1] = 0.0
        dv[s0:s1] = 0.0
        for h in range(H):
            j = kv_head_of(h, H, H_kv)
            gq, gk, gv = fn(q[s0:s1, h], k[s0:s1, j], v[s0:s1, j], dout[s0:s1, h], **kw)
            dq[s0:s1, h] = gq
            dk[s0:s1, j] += gk
            dv[s0:s1, j] += gv
    return dq, dk, dv


# --------------------------------------------------------------------------
# (batch, seq, heads, dim) helpers
# --------------------------------------------------------------------------

def to_f64(x) -> np.ndarray:
    """Exact upcast of a bf16/fp32 torch tensor or array to float64 NumPy."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def batched(fn: Callable, *arrays, heads: Optional[Sequence[Tuple[int, int]]] = None, **kw):
    """Apply a one-head function to every (batch, head) of (B, S, H, D) arrays.

    Returns a list, one entry per output of ``fn``, each stacked back to
    (B, S, H, D) for sequence-shaped outputs or (B, H, S) for per-row
    vectors.  ``heads`` restricts the work to the listed (batch, head)
    pairs (outputs of other pairs are left as NaN).
    """
    B, S, H, _ = arrays[0].shape
    todo = heads if heads is not None else [(bi, hi) for bi in range(B) for hi in range(H)]
    outs = None
    for bi, hi in todo:
        res = fn(*[a[bi, :, hi, :] for a in arrays], **kw)
        if not isinstance(res, tuple):
            res = (res,)
        if outs is None:
            outs = []
            for r in res:
                if r.ndim == 2:
                    outs.append(np.full((B, r.shape[0], H, r.shape[1]), np.nan))
                else:
                    outs.append(np.full((B, H, r.shape[0]), np.nan))
        for o, r in zip(outs, res):
            if r.ndim == 2:
                o[bi, :, hi, :] = r
            else:
                o[bi, hi, :] = r
    return outs
