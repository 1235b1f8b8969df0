"""The no-allocation backward entry point (diffusion_attn_bwd_noalloc), called
through the C ABI with ctypes: the same results, bit for bit, as
diffusion_attn_bwd with a caller workspace, on two calls in a row (the
second with a smaller problem, so it runs on statistics the first call left
in the library's static array), and the size limit."""
import ctypes
import math

import pytest
import torch

import block_diffusion_lm_amd as bd
from workloads import make_inputs

TOO_LARGE = 4


def _bwd_pair(B, n, H, D, b, seed):
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in make_inputs(B, n, H, D, seed=seed))
    scale = 1 / math.sqrt(D)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, 2 * n), dtype=torch.float32, device=dev)
    bd.diffusion_attn_fwd(q, k, v, out, lse, B, n, H, D, b, scale)
    ref = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(bd.diffusion_attn_bwd_workspace_size(B, n, H, D), dtype=torch.uint8, device=dev)
    bd.diffusion_attn_bwd(q, k, v, out, do, lse, *ref, B, n, H, D, b, scale, ws)
    got = [torch.full_like(q, 7.0) for _ in range(3)]
    lib = bd.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.diffusion_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        do.data_ptr(), lse.data_ptr(), *(t.data_ptr() for t in got),
                                        B, n, H, D, b, ctypes.c_float(scale), stream)
    assert st == 0, bd.status_string(st)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # the second call is smaller: the array still holds the first call's
    # statistics past the rows the second writes
    for B, n, H, D, b, seed in ((2, 1024, 8, 128, 16, 50001), (1, 300, 3, 64, 7, 50002)):
        ref, got = _bwd_pair(B, n, H, D, b, seed)
        for name, r, g in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(r, g), f"{name} differs (B={B} n={n} H={H} D={D} b={b})"


def test_noalloc_rejects_beyond_its_scratch():
    # 2 x 8192 x 257 query rows x heads > 4194304: refused before any GPU use
    FAKE = 0x10000
    lib = bd.lib()
    assert lib.diffusion_attn_bwd_noalloc(*([FAKE] * 9), 1, 8192, 257, 64, 4, ctypes.c_float(0.125),
                                          None) == TOO_LARGE
    assert lib.diffusion_attn_bwd_noalloc(*([FAKE] * 9), 1, 8192, 256, 80, 4, ctypes.c_float(0.125),
                                          None) == 2
    assert lib.diffusion_attn_bwd_noalloc(*([FAKE] * 8 + [None]), 1, 64, 2, 64, 4, ctypes.c_float(0.125),
                                          None) == 1
