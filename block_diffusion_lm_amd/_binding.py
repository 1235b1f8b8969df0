"""ctypes binding of libbdattn.so: the C-ABI entry points under the same names.

Argument marshalling only: every function checks that its tensors live on
the GPU with the dtype and shape the C ABI expects, passes their device
pointers and the current HIP stream, and turns a non-zero status into an
exception.  All computation happens in the library's HIP kernels.  There is
no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# BDATTN_LIB selects another build of the same library (e.g. one compiled
# with different code-generation options) for side-by-side measurements.
LIB_PATH = os.environ.get("BDATTN_LIB") or os.path.join(_HERE, "libbdattn.so")

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_i32p = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes); mirrors include/bdattn.h
SIGNATURES = {
    "bdattn_status_string": (ctypes.c_char_p, [_i]),
    "diffusion_attn_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp]),
    "diffusion_attn_bwd_workspace_size": (_sz, [_i, _i, _i, _i]),
    "diffusion_attn_bwd": (_i, [_vp] * 9 + [_i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "diffusion_attn_bwd_noalloc": (_i, [_vp] * 9 + [_i, _i, _i, _i, _i, _f, _vp]),
    "causal_attn_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _vp]),
    "causal_attn_bwd_workspace_size": (_sz, [_i, _i, _i, _i]),
    "causal_attn_bwd": (_i, [_vp] * 9 + [_i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "bdattn_bwd_stage": (_i, [_i, _i] + [_vp] * 10 + [_i] * 7 + [_f, _f, _vp, _sz, _vp]),
    "bdattn_fwd": (_i, [_i] + [_vp] * 6 + [_i] * 7 + [_f, _f, _vp]),
    "bdattn_bwd_workspace_size": (_sz, [_i] * 8),
    "bdattn_bwd": (_i, [_i] + [_vp] * 10 + [_i] * 7 + [_f, _f, _vp, _sz, _vp]),
    "diffusion_attn_fwd_fp8": (_i, [_vp] * 8 + [_i] * 6 + [_f, _vp]),
    "causal_attn_fwd_fp8": (_i, [_vp] * 8 + [_i] * 5 + [_f, _vp]),
    "diffusion_attn_varlen_fwd": (_i, [_vp] * 6 + [_i] * 7 + [_f, _vp]),
    "diffusion_attn_varlen_bwd_workspace_size": (_sz, [_i] * 6),
    "diffusion_attn_varlen_bwd": (_i, [_vp] * 10 + [_i] * 7 + [_f, _vp, _sz, _vp]),
    "causal_attn_varlen_fwd": (_i, [_vp] * 6 + [_i] * 6 + [_f, _vp]),
    "causal_attn_varlen_bwd_workspace_size": (_sz, [_i] * 6),
    "causal_attn_varlen_bwd": (_i, [_vp] * 10 + [_i] * 6 + [_f, _vp, _sz, _vp]),
    "diffusion_attn_fwd_gqa": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp]),
    "diffusion_attn_bwd_gqa": (_i, [_vp] * 9 + [_i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "causal_attn_fwd_gqa": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp]),
    "causal_attn_bwd_gqa": (_i, [_vp] * 9 + [_i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "diffusion_attn_bwd_gqa_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "causal_attn_bwd_gqa_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "bdattn_fwd_tiles": (_i, [_i, _i, _i, _i, _i, _i, _i, _i32p, _i]),
    "bdattn_bwd_tiles": (_i, [_i, _i, _i, _i, _i, _i, _i, _i32p, _i]),
    "bdattn_row_interval": (_i, [_i, _i, _i, _i, _i, _i, _i32p, _i32p]),
    "bdattn_visible_pairs": (ctypes.c_int64, [_i, _i, _i]),
}

MODE_DIFFUSION, MODE_CAUSAL = 0, 1
NOISY, CLEAN = 0, 1

_lib = None


class BdattnError(RuntimeError):
    pass


def lib():
    """Load libbdattn.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise BdattnError(f"{LIB_PATH} is missing: build it with `python -m block_diffusion_lm_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(code: int) -> str:
    return lib().bdattn_status_string(int(code)).decode()


def _check(code: int, what: str):
    if code != 0:
        raise BdattnError(f"{what} failed: {status_string(code)} (status {code})")


def _stream_handle(t: torch.Tensor, stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _want(*specs):
    """Check (name, tensor, dtype, shape) specs: dtype, shape and layout of
    every tensor first, then that all of them live on the GPU."""
    for name, t, dtype, shape in specs:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t, _, _ in specs:
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU, got {t.device}")


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def diffusion_attn_fwd(q, k, v, out, lse, B, n, H, D, block_size, scale, stream=None):
    _want_fwd(q, k, v, out, lse, B, 2 * n, H, H, D)
    _check(lib().diffusion_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, n, H, D,
                                    block_size, float(scale), _stream_handle(q, stream)),
           "diffusion_attn_fwd")


def diffusion_attn_bwd_workspace_size(B, n, H, D) -> int:
    return int(lib().diffusion_attn_bwd_workspace_size(B, n, H, D))


def diffusion_attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, n, H, D, block_size, scale,
                       workspace, workspace_bytes=None, stream=None):
    workspace_bytes = _want_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, 2 * n, H, H, D, workspace,
                                workspace_bytes)
    _check(lib().diffusion_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                    _ptr(dq), _ptr(dk), _ptr(dv), B, n, H, D, block_size,
                                    float(scale), _ptr(workspace), int(workspace_bytes),
                                    _stream_handle(q, stream)),
           "diffusion_attn_bwd")


def diffusion_attn_bwd_noalloc(q, k, v, out, dout, lse, dq, dk, dv, B, n, H, D, block_size, scale,
                               stream=None):
    """diffusion_attn_bwd without a workspace: the library keeps the row
    statistics in its own static device array (calls that overlap on one GPU
    race; see the header)."""
    bf = torch.bfloat16
    qs = (B, 2 * n, H, D)
    _want(("q", q, bf, qs), ("k", k, bf, qs), ("v", v, bf, qs), ("out", out, bf, qs),
          ("dout", dout, bf, qs), ("lse", lse, torch.float32, (B, H, 2 * n)), ("dq", dq, bf, qs),
          ("dk", dk, bf, qs), ("dv", dv, bf, qs))
    _check(lib().diffusion_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                            _ptr(dq), _ptr(dk), _ptr(dv), B, n, H, D, block_size,
                                            float(scale), _stream_handle(q, stream)),
           "diffusion_attn_bwd_noalloc")


def causal_attn_fwd(q, k, v, out, lse, B, S, H, D, scale, stream=None):
    _want_fwd(q, k, v, out, lse, B, S, H, H, D)
    _check(lib().causal_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, S, H, D,
                                 float(scale), _stream_handle(q, stream)),
           "causal_attn_fwd")


def causal_attn_bwd_workspace_size(B, S, H, D) -> int:
    return int(lib().causal_attn_bwd_workspace_size(B, S, H, D))


def causal_attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, S, H, D, scale, workspace,
                    workspace_bytes=None, stream=None):
    workspace_bytes = _want_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, S, H, H, D, workspace,
                                workspace_bytes)
    _check(lib().causal_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                 _ptr(dq), _ptr(dk), _ptr(dv), B, S, H, D, float(scale),
                                 _ptr(workspace), int(workspace_bytes), _stream_handle(q, stream)),
           "causal_attn_bwd")


def _want_fwd(q, k, v, out, lse, B, T, H, H_kv, D):
    bf = torch.bfloat16
    _want(("q", q, bf, (B, T, H, D)), ("k", k, bf, (B, T, H_kv, D)), ("v", v, bf, (B, T, H_kv, D)),
          ("out", out, bf, (B, T, H, D)), ("lse", lse, torch.float32, (B, H, T)))


def _want_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, T, H, H_kv, D, workspace, workspace_bytes):
    """Check the backward's tensors; returns the workspace size in bytes."""
    bf = torch.bfloat16
    qs, kvs = (B, T, H, D), (B, T, H_kv, D)
    _want(("q", q, bf, qs), ("k", k, bf, kvs), ("v", v, bf, kvs), ("out", out, bf, qs),
          ("dout", dout, bf, qs), ("lse", lse, torch.float32, (B, H, T)), ("dq", dq, bf, qs),
          ("dk", dk, bf, kvs), ("dv", dv, bf, kvs))
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda":
        raise ValueError("workspace must be a tensor on the GPU")
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    return int(workspace_bytes)


def bdattn_bwd_stage(mode, stage, q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens, B, n,
                     total_tokens, H, H_kv, D, block_size, scale, softcap, workspace,
                     workspace_bytes=None, stream=None):
    """One backward stage (0: dQ, also writing -delta and lse2; 1: dK/dV).

    cu_seqlens None: batched tensors, n the half length (S in causal mode),
    total_tokens ignored.  Otherwise packed tensors as in the varlen entry
    points, n the longest sample."""
    if cu_seqlens is None:
        T = 2 * n if mode == MODE_DIFFUSION else n
        wsb = _want_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, T, H, H_kv, D, workspace,
                        workspace_bytes)
        cu = None
    else:
        wsb = _want_bwd_packed(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens, B, total_tokens, H,
                               H_kv, D, workspace, workspace_bytes)
        cu = _ptr(cu_seqlens)
    _check(lib().bdattn_bwd_stage(mode, stage, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                                  _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), cu, B, n, total_tokens,
                                  H, H_kv, D, block_size, float(scale), float(softcap),
                                  _ptr(workspace), wsb, _stream_handle(q, stream)),
           "bdattn_bwd_stage")


# The general form: mode, batched (cu_seqlens None) or packed tensors, grouped
# heads and softcapping (0: off) in one call.

def _general_checks_fwd(mode, q, k, v, out, lse, cu_seqlens, B, n, total_tokens, H, H_kv, D):
    if cu_seqlens is None:
        _want_fwd(q, k, v, out, lse, B, 2 * n if mode == MODE_DIFFUSION else n, H, H_kv, D)
        return None
    _want_fwd_packed(q, k, v, out, lse, cu_seqlens, B, total_tokens, H, H_kv, D)
    return _ptr(cu_seqlens)


def bdattn_fwd(mode, q, k, v, out, lse, cu_seqlens, B, n, total_tokens, H, H_kv, D, block_size, scale,
               softcap=0.0, stream=None):
    cu = _general_checks_fwd(mode, q, k, v, out, lse, cu_seqlens, B, n, total_tokens, H, H_kv, D)
    _check(lib().bdattn_fwd(mode, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), cu, B, n, total_tokens,
                            H, H_kv, D, block_size, float(scale), float(softcap), _stream_handle(q, stream)),
           "bdattn_fwd")


def bdattn_bwd_workspace_size(mode, packed, B, n, total_tokens, H, H_kv, D) -> int:
    return int(lib().bdattn_bwd_workspace_size(mode, int(bool(packed)), B, n, total_tokens, H, H_kv, D))


def bdattn_bwd(mode, q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens, B, n, total_tokens, H, H_kv, D,
               block_size, scale, softcap, workspace, workspace_bytes=None, stream=None):
    if cu_seqlens is None:
        wsb = _want_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, 2 * n if mode == MODE_DIFFUSION else n,
                        H, H_kv, D, workspace, workspace_bytes)
        cu = None
    else:
        wsb = _want_bwd_packed(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens, B, total_tokens, H,
                               H_kv, D, workspace, workspace_bytes)
        cu = _ptr(cu_seqlens)
    _check(lib().bdattn_bwd(mode, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq),
                            _ptr(dk), _ptr(dv), cu, B, n, total_tokens, H, H_kv, D, block_size,
                            float(scale), float(softcap), _ptr(workspace), wsb,
                            _stream_handle(q, stream)),
           "bdattn_bwd")


# Packed samples of different lengths: q / out / dout / dq [total][H][D],
# k / v / dk / dv [total][H_kv][D], lse [H][total], cu_seqlens int32 [B + 1]
# on the GPU (sample b: tokens cu[b] .. cu[b+1]).

def _want_fwd_packed(q, k, v, out, lse, cu_seqlens, B, total, H, H_kv, D):
    bf = torch.bfloat16
    _want(("q", q, bf, (total, H, D)), ("k", k, bf, (total, H_kv, D)),
          ("v", v, bf, (total, H_kv, D)), ("out", out, bf, (total, H, D)),
          ("lse", lse, torch.float32, (H, total)), ("cu_seqlens", cu_seqlens, torch.int32, (B + 1,)))


def _want_bwd_packed(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens, B, total, H, H_kv, D,
                     workspace, workspace_bytes):
    bf = torch.bfloat16
    qs, kvs = (total, H, D), (total, H_kv, D)
    _want(("q", q, bf, qs), ("k", k, bf, kvs), ("v", v, bf, kvs), ("out", out, bf, qs),
          ("dout", dout, bf, qs), ("lse", lse, torch.float32, (H, total)), ("dq", dq, bf, qs),
          ("dk", dk, bf, kvs), ("dv", dv, bf, kvs),
          ("cu_seqlens", cu_seqlens, torch.int32, (B + 1,)))
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda":
        raise ValueError("workspace must be a tensor on the GPU")
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    return int(workspace_bytes)


def diffusion_attn_varlen_fwd(q, k, v, out, lse, cu_seqlens, B, max_n, total_tokens, H, H_kv, D,
                              block_size, scale, stream=None):
    _want_fwd_packed(q, k, v, out, lse, cu_seqlens, B, total_tokens, H, H_kv, D)
    _check(lib().diffusion_attn_varlen_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                           _ptr(cu_seqlens), B, max_n, total_tokens, H, H_kv, D,
                                           block_size, float(scale), _stream_handle(q, stream)),
           "diffusion_attn_varlen_fwd")


def diffusion_attn_varlen_bwd_workspace_size(B, max_n, total_tokens, H, H_kv, D) -> int:
    return int(lib().diffusion_attn_varlen_bwd_workspace_size(B, max_n, total_tokens, H, H_kv, D))


def diffusion_attn_varlen_bwd(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens, B, max_n,
                              total_tokens, H, H_kv, D, block_size, scale, workspace,
                              workspace_bytes=None, stream=None):
    wsb = _want_bwd_packed(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens, B, total_tokens, H, H_kv,
                           D, workspace, workspace_bytes)
    _check(lib().diffusion_attn_varlen_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                                           _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens),
                                           B, max_n, total_tokens, H, H_kv, D, block_size,
                                           float(scale), _ptr(workspace), wsb,
                                           _stream_handle(q, stream)),
           "diffusion_attn_varlen_bwd")


def causal_attn_varlen_fwd(q, k, v, out, lse, cu_seqlens, B, max_S, total_tokens, H, H_kv, D, scale,
                           stream=None):
    _want_fwd_packed(q, k, v, out, lse, cu_seqlens, B, total_tokens, H, H_kv, D)
    _check(lib().causal_attn_varlen_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                        _ptr(cu_seqlens), B, max_S, total_tokens, H, H_kv, D,
                                        float(scale), _stream_handle(q, stream)),
           "causal_attn_varlen_fwd")


def causal_attn_varlen_bwd_workspace_size(B, max_S, total_tokens, H, H_kv, D) -> int:
    return int(lib().causal_attn_varlen_bwd_workspace_size(B, max_S, total_tokens, H, H_kv, D))


def causal_attn_varlen_bwd(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens, B, max_S, total_tokens,
                           H, H_kv, D, scale, workspace, workspace_bytes=None, stream=None):
    wsb = _want_bwd_packed(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens, B, total_tokens, H, H_kv,
                           D, workspace, workspace_bytes)
    _check(lib().causal_attn_varlen_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens), B, max_S,
                                        total_tokens, H, H_kv, D, float(scale), _ptr(workspace), wsb,
                                        _stream_handle(q, stream)),
           "causal_attn_varlen_bwd")


# Grouped-query attention: q / out / dout / dq carry H heads, k / v / dk / dv
# carry H_kv (H a multiple of H_kv); query head h reads key/value head
# h // (H // H_kv).

def diffusion_attn_fwd_gqa(q, k, v, out, lse, B, n, H, H_kv, D, block_size, scale, stream=None):
    _want_fwd(q, k, v, out, lse, B, 2 * n, H, H_kv, D)
    _check(lib().diffusion_attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, n, H,
                                        H_kv, D, block_size, float(scale),
                                        _stream_handle(q, stream)),
           "diffusion_attn_fwd_gqa")


def diffusion_attn_bwd_gqa_workspace_size(B, n, H, H_kv, D) -> int:
    return int(lib().diffusion_attn_bwd_gqa_workspace_size(B, n, H, H_kv, D))


def causal_attn_bwd_gqa_workspace_size(B, S, H, H_kv, D) -> int:
    return int(lib().causal_attn_bwd_gqa_workspace_size(B, S, H, H_kv, D))


def diffusion_attn_bwd_gqa(q, k, v, out, dout, lse, dq, dk, dv, B, n, H, H_kv, D, block_size,
                           scale, workspace, workspace_bytes=None, stream=None):
    wsb = _want_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, 2 * n, H, H_kv, D, workspace,
                    workspace_bytes)
    _check(lib().diffusion_attn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                                        _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, n, H, H_kv, D,
                                        block_size, float(scale), _ptr(workspace), wsb,
                                        _stream_handle(q, stream)),
           "diffusion_attn_bwd_gqa")


def causal_attn_fwd_gqa(q, k, v, out, lse, B, S, H, H_kv, D, scale, stream=None):
    _want_fwd(q, k, v, out, lse, B, S, H, H_kv, D)
    _check(lib().causal_attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, S, H,
                                     H_kv, D, float(scale), _stream_handle(q, stream)),
           "causal_attn_fwd_gqa")


def causal_attn_bwd_gqa(q, k, v, out, dout, lse, dq, dk, dv, B, S, H, H_kv, D, scale, workspace,
                        workspace_bytes=None, stream=None):
    wsb = _want_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, S, H, H_kv, D, workspace,
                    workspace_bytes)
    _check(lib().causal_attn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                     _ptr(dq), _ptr(dk), _ptr(dv), B, S, H, H_kv, D, float(scale),
                                     _ptr(workspace), wsb, _stream_handle(q, stream)),
           "causal_attn_bwd_gqa")


# ---------------------------------------------------------------------------
# Host-side geometry inspection (no GPU needed)
# ---------------------------------------------------------------------------

def _tiles(fn, mode, n, block_size, tile_m, tile_n, half, tile):
    cnt = fn(mode, n, block_size, tile_m, tile_n, half, tile, None, 0)
    if cnt < 0:
        raise ValueError("bad geometry arguments")
    buf = (ctypes.c_int32 * max(1, 3 * cnt))()
    fn(mode, n, block_size, tile_m, tile_n, half, tile, buf, cnt)
    return [(buf[3 * i], buf[3 * i + 1], buf[3 * i + 2]) for i in range(cnt)]


def bdattn_fwd_tiles(mode, n, block_size, tile_m, tile_n, qhalf, qt):
    """[(key_half, key_tile, masked)] visited by query tile qt of half qhalf."""
    return _tiles(lib().bdattn_fwd_tiles, mode, n, block_size, tile_m, tile_n, qhalf, qt)


def bdattn_bwd_tiles(mode, n, block_size, tile_m, tile_n, khalf, kt):
    """[(query_half, query_tile, masked)] that see key tile kt of half khalf."""
    return _tiles(lib().bdattn_bwd_tiles, mode, n, block_size, tile_m, tile_n, khalf, kt)


def bdattn_row_interval(mode, n, block_size, qhalf, p, khalf):
    lo, hi = ctypes.c_int32(), ctypes.c_int32()
    if lib().bdattn_row_interval(mode, n, block_size, qhalf, p, khalf, ctypes.byref(lo), ctypes.byref(hi)) != 0:
        raise ValueError("bad geometry arguments")
    return lo.value, hi.value


def bdattn_visible_pairs(mode, n, block_size) -> int:
    r = lib().bdattn_visible_pairs(mode, n, block_size)
    if r < 0:
        raise ValueError("bad geometry arguments")
    return int(r)


# ---------------------------------------------------------------------------
# FP8 (E4M3) forward: q [B][T][H][D], k / v [B][T][H_kv][D] as
# torch.float8_e4m3fn, descale factors float32 [B][H] / [B][H_kv]
# ---------------------------------------------------------------------------

def _want_fwd_fp8(q, k, v, qd, kd, vd, out, lse, B, T, H, H_kv, D):
    f8, f32 = torch.float8_e4m3fn, torch.float32
    _want(("q", q, f8, (B, T, H, D)), ("k", k, f8, (B, T, H_kv, D)), ("v", v, f8, (B, T, H_kv, D)),
          ("q_descale", qd, f32, (B, H)), ("k_descale", kd, f32, (B, H_kv)),
          ("v_descale", vd, f32, (B, H_kv)), ("out", out, torch.bfloat16, (B, T, H, D)),
          ("lse", lse, f32, (B, H, T)))


def diffusion_attn_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, out, lse, B, n, H, H_kv, D,
                           block_size, scale, stream=None):
    _want_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, out, lse, B, 2 * n, H, H_kv, D)
    _check(lib().diffusion_attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale),
                                        _ptr(v_descale), _ptr(out), _ptr(lse), B, n, H, H_kv, D,
                                        block_size, float(scale), _stream_handle(q, stream)),
           "diffusion_attn_fwd_fp8")


def causal_attn_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, out, lse, B, S, H, H_kv, D, scale,
                        stream=None):
    _want_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, out, lse, B, S, H, H_kv, D)
    _check(lib().causal_attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale),
                                     _ptr(v_descale), _ptr(out), _ptr(lse), B, S, H, H_kv, D,
                                     float(scale), _stream_handle(q, stream)),
           "causal_attn_fwd_fp8")
