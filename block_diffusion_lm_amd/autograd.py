"""PyTorch-facing functions built on the C-ABI binding.

``diffusion_attn_func(q, k, v, block_size)`` takes q, k, v of shape
(batch, 2n, heads, headdim) laid out [noisy | clean] (Fast Diffusion
Attention, "TL;DR": the same call shape as flash-attention's function, with
a block size where the causal flag would be) and returns the attention
output; its backward runs the library's backward kernels.  k and v may
carry fewer heads than q (grouped-query attention: H a multiple of H_kv,
query head h reading key/value head h // (H // H_kv)).  PyTorch only
allocates the outputs and the workspace and supplies the stream.
"""
from __future__ import annotations

import math

import torch

from . import _binding as _b


def _prep(x: torch.Tensor) -> torch.Tensor:
    return x if x.is_contiguous() else x.contiguous()


class _DiffusionAttn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, block_size, scale, softcap):
        q, k, v = _prep(q), _prep(k), _prep(v)
        B, T, H, D = q.shape
        Hkv = k.shape[2]
        if T % 2:
            raise ValueError("the sequence length must be 2n ([noisy | clean])")
        n = T // 2
        out = torch.empty_like(q)
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
        if softcap:
            _b.bdattn_fwd(_b.MODE_DIFFUSION, q, k, v, out, lse, None, B, n, 0, H, Hkv, D, block_size,
                          scale, softcap)
        elif Hkv == H:
            _b.diffusion_attn_fwd(q, k, v, out, lse, B, n, H, D, block_size, scale)
        else:
            _b.diffusion_attn_fwd_gqa(q, k, v, out, lse, B, n, H, Hkv, D, block_size, scale)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.block_size, ctx.scale, ctx.softcap = block_size, scale, softcap
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, out, lse = ctx.saved_tensors
        dout = _prep(dout)
        B, T, H, D = q.shape
        Hkv = k.shape[2]
        n = T // 2
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_bytes = _b.diffusion_attn_bwd_gqa_workspace_size(B, n, H, Hkv, D)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        if ctx.softcap:
            _b.bdattn_bwd(_b.MODE_DIFFUSION, q, k, v, out, dout, lse, dq, dk, dv, None, B, n, 0, H, Hkv,
                          D, ctx.block_size, ctx.scale, ctx.softcap, ws, ws_bytes)
        elif Hkv == H:
            _b.diffusion_attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, n, H, D, ctx.block_size,
                                  ctx.scale, ws, ws_bytes)
        else:
            _b.diffusion_attn_bwd_gqa(q, k, v, out, dout, lse, dq, dk, dv, B, n, H, Hkv, D,
                                      ctx.block_size, ctx.scale, ws, ws_bytes)
        return dq, dk, dv, None, None, None


class _CausalAttn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, scale, softcap):
        q, k, v = _prep(q), _prep(k), _prep(v)
        B, S, H, D = q.shape
        Hkv = k.shape[2]
        out = torch.empty_like(q)
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
        if softcap:
            _b.bdattn_fwd(_b.MODE_CAUSAL, q, k, v, out, lse, None, B, S, 0, H, Hkv, D, 1, scale, softcap)
        elif Hkv == H:
            _b.causal_attn_fwd(q, k, v, out, lse, B, S, H, D, scale)
        else:
            _b.causal_attn_fwd_gqa(q, k, v, out, lse, B, S, H, Hkv, D, scale)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.scale, ctx.softcap = scale, softcap
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, out, lse = ctx.saved_tensors
        dout = _prep(dout)
        B, S, H, D = q.shape
        Hkv = k.shape[2]
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_bytes = _b.causal_attn_bwd_gqa_workspace_size(B, S, H, Hkv, D)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        if ctx.softcap:
            _b.bdattn_bwd(_b.MODE_CAUSAL, q, k, v, out, dout, lse, dq, dk, dv, None, B, S, 0, H, Hkv, D, 1,
                          ctx.scale, ctx.softcap, ws, ws_bytes)
        elif Hkv == H:
            _b.causal_attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, S, H, D, ctx.scale, ws, ws_bytes)
        else:
            _b.causal_attn_bwd_gqa(q, k, v, out, dout, lse, dq, dk, dv, B, S, H, Hkv, D, ctx.scale, ws,
                                   ws_bytes)
        return dq, dk, dv, None, None


class _DiffusionAttnVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens, max_n, block_size, scale, softcap):
        q, k, v = _prep(q), _prep(k), _prep(v)
        total, H, D = q.shape
        Hkv = k.shape[1]
        B = cu_seqlens.numel() - 1
        out = torch.empty_like(q)
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
        _b.bdattn_fwd(_b.MODE_DIFFUSION, q, k, v, out, lse, cu_seqlens, B, max_n, total, H, Hkv, D,
                      block_size, scale, softcap)
        ctx.save_for_backward(q, k, v, out, lse, cu_seqlens)
        ctx.max_n, ctx.block_size, ctx.scale, ctx.softcap = max_n, block_size, scale, softcap
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, out, lse, cu_seqlens = ctx.saved_tensors
        dout = _prep(dout)
        total, H, D = q.shape
        Hkv = k.shape[1]
        B = cu_seqlens.numel() - 1
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_bytes = _b.diffusion_attn_varlen_bwd_workspace_size(B, ctx.max_n, total, H, Hkv, D)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
        _b.bdattn_bwd(_b.MODE_DIFFUSION, q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens, B, ctx.max_n,
                      total, H, Hkv, D, ctx.block_size, ctx.scale, ctx.softcap, ws, ws_bytes)
        return dq, dk, dv, None, None, None, None, None


def diffusion_attn_func(q, k, v, block_size: int, softmax_scale=None, return_lse: bool = False,
                        softcap: float = 0.0):
    """Block-diffusion attention; q: (batch, 2n, heads, headdim) bf16, k and v:
    (batch, 2n, kv_heads, headdim) with heads a multiple of kv_heads.
    softcap > 0 caps the scaled scores to softcap * tanh(s / softcap)."""
    scale = 1.0 / math.sqrt(q.shape[-1]) if softmax_scale is None else float(softmax_scale)
    out, lse = _DiffusionAttn.apply(q, k, v, int(block_size), scale, float(softcap))
    return (out, lse) if return_lse else out


def causal_attn_func(q, k, v, softmax_scale=None, return_lse: bool = False, softcap: float = 0.0):
    """Causal attention (the yardstick); q: (batch, seq, heads, headdim) bf16, k
    and v: (batch, seq, kv_heads, headdim)."""
    scale = 1.0 / math.sqrt(q.shape[-1]) if softmax_scale is None else float(softmax_scale)
    out, lse = _CausalAttn.apply(q, k, v, scale, float(softcap))
    return (out, lse) if return_lse else out


def diffusion_attn_varlen_func(q, k, v, cu_seqlens, max_n: int, block_size: int, softmax_scale=None,
                               return_lse: bool = False, softcap: float = 0.0):
    """Block-diffusion attention over packed samples of different lengths.

    q: (total, heads, headdim) bf16, k and v: (total, kv_heads, headdim);
    cu_seqlens: int32 (B + 1,) on the GPU, sample b holding the tokens
    cu_seqlens[b] .. cu_seqlens[b+1] as [noisy n_b | clean n_b]; max_n: the
    largest n_b.  Rows of the outputs and gradients outside every sample
    are left uninitialised.  Returns out (and lse of shape (heads, total))."""
    scale = 1.0 / math.sqrt(q.shape[-1]) if softmax_scale is None else float(softmax_scale)
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    out, lse = _DiffusionAttnVarlen.apply(q, k, v, cu_seqlens, int(max_n), int(block_size), scale,
                                          float(softcap))
    return (out, lse) if return_lse else out
