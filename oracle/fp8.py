"""Float64 reference for the FP8 forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Fast Diffusion Attention, "Results" (the FP8 forward pass) names the
operation but not its quantisation; the readings taken here:

* q, k and v arrive as OCP FP8 E4M3 values (1 sign bit, 4 exponent bits
  with bias 7, 3 mantissa bits; no infinities, one NaN pattern per sign,
  largest finite 448), each with a float32 descale factor per (sample,
  head): the value a byte stands for is descale * e4m3(byte).
* The result approximates exact softmax attention over those dequantized
  values, which is what ``fp8_forward`` computes (with the scores scaled by
  ``scale`` as in the bf16 pass).
* The one rounding the method adds is that of the unnormalised
  probabilities P~ = 2^(s c - m) (at most 2^8 under the lazy rescale) to
  E4M3 for the P.V product, the denominator summing the unrounded values.
  ``fp8_output_bound`` bounds the error this can cause in each output
  element.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .attention import block_diffusion_mask, diffusion_forward, _half_len


def e4m3_value(code: int) -> float:
    """The real number an OCP FP8 E4M3 byte encodes (NaN for 0x7F / 0xFF)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:  # subnormal: m / 8 * 2^(1 - 7)
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3 = np.array([e4m3_value(c) for c in range(256)])


def dequantize_e4m3(codes, descale) -> np.ndarray:
    """descale * e4m3(codes) in float64; codes: uint8 array, descale: scalar
    or array broadcastable against it."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)] * np.asarray(descale, dtype=np.float64)


def fp8_forward(q8, k8, v8, q_descale, k_descale, v_descale, b: int, scale: float):
    """(O, LSE) of one head from E4M3 codes q8, k8, v8 of shape (2n, D):
    exact attention over the dequantized values."""
    q = dequantize_e4m3(q8, q_descale)
    k = dequantize_e4m3(k8, k_descale)
    v = dequantize_e4m3(v8, v_descale)
    return diffusion_forward(q, k, v, b, scale)


def fp8_output_bound(q, k, v, b: int, scale: float, rows: Optional[Sequence[int]] = None,
                     mask: Optional[np.ndarray] = None) -> np.ndarray:
    """Largest error the E4M3 rounding of P~ can cause in O[rows] (float64
    q, k, v of shape (2n, D), already dequantized).  ``mask`` (rows x keys)
    replaces the block-diffusion mask, e.g. with the causal one.

    The kernel rounds P~_ij = 2^(s_ij c - m_i) with a reference m_i at or
    below the row maximum (so P~ <= 2^8 and its row sum l_i' is at least
    the row sum l_i taken at the maximum).  A normal E4M3 value is off by
    at most 2^-4 of itself, one below 2^-6 by at most 2^-10.  Dividing by
    l_i' gives, per output element,
        |dO_id| <= 2^-4 sum_j P_ij |v_jd| + 2^-10 sum_{j visible} |v_jd| / l_i
    with P the exact probabilities and l_i = sum_j exp(s_ij - max_j s_ij).
    """
    if mask is None:
        n = _half_len(q)
        rows = np.arange(2 * n) if rows is None else np.asarray(rows, dtype=np.int64)
        M = block_diffusion_mask(n, b, rows)
    else:
        rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
        M = mask
    S = np.where(M, scale * (q[rows] @ k.T), -np.inf)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    ell = E.sum(axis=1)
    P = E / ell[:, None]
    av = np.abs(v)
    return 2.0 ** -4 * (P @ av) + 2.0 ** -10 * (M.astype(np.float64) @ av) / ell[:, None]
