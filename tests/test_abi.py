"""The C ABI: the library loads, exports every symbol the header declares,
and rejects bad arguments with a status code before touching the GPU.

No call here reaches a kernel launch: every case fails validation first,
so these tests run on a machine without a GPU.
"""
import ctypes
import os
import re

import pytest

import block_diffusion_lm_amd as bd
from block_diffusion_lm_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bdattn.h")

OK, INVALID, UNSUPPORTED, LAUNCH = 0, 1, 2, 3
# A fake, 16-byte aligned, non-null address: only ever passed alongside some
# other invalid argument, so the library rejects the call before using it.
FAKE = 0x10000


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"}


def test_header_and_binding_agree():
    assert _declared() == set(_binding.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bd.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in (OK, INVALID, UNSUPPORTED, LAUNCH, 99):
        assert isinstance(bd.status_string(code), str) and bd.status_string(code)


def _fwd(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, B=1, n=16, H=1, D=64, b=4, scale=0.125)
    args.update(kw)
    return bd.lib().diffusion_attn_fwd(args["q"], args["k"], args["v"], args["out"], args["lse"],
                                       args["B"], args["n"], args["H"], args["D"], args["b"],
                                       args["scale"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(lse=None), INVALID), (dict(v=FAKE + 2), INVALID),
    (dict(B=0), INVALID), (dict(n=0), INVALID), (dict(H=-1), INVALID), (dict(b=0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID), (dict(scale=0.0), INVALID),
    (dict(n=2 ** 30 + 1), INVALID), (dict(D=80), UNSUPPORTED), (dict(D=512), UNSUPPORTED),
    (dict(n=2 ** 22, H=2, D=128), UNSUPPORTED),
    # 2^31 rows in all (over the 32-bit row limit), each sample small
    (dict(B=2 ** 20, n=1024, H=1, D=64), INVALID),
])
def test_fwd_rejects(kw, want):
    assert _fwd(**kw) == want


def _bwd(**kw):
    args = dict(p=[FAKE] * 9, B=1, n=16, H=1, D=64, b=4, scale=0.125, ws=FAKE, wsb=1 << 20)
    args.update(kw)
    return bd.lib().diffusion_attn_bwd(*args["p"], args["B"], args["n"], args["H"], args["D"],
                                       args["b"], args["scale"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(p=[FAKE] * 8 + [None]), INVALID), (dict(ws=None), INVALID), (dict(wsb=4), INVALID),
    (dict(ws=FAKE + 8), INVALID), (dict(B=0), INVALID), (dict(b=-3), INVALID),
    (dict(scale=float("-inf")), INVALID), (dict(D=32), UNSUPPORTED),
])
def test_bwd_rejects(kw, want):
    assert _bwd(**kw) == want


@pytest.mark.parametrize("stage", [-1, 2, 3])
def test_bwd_stage_rejects_unknown_stage(stage):
    # stage 0 is dQ (with the row statistics), stage 1 dK/dV; nothing else
    lib = bd.lib()
    assert lib.bdattn_bwd_stage(0, stage, *([FAKE] * 9), None, 1, 16, 0, 1, 1, 64, 4, 0.125, 0.0, FAKE, 1 << 20, None) == INVALID


def test_causal_rejects():
    lib = bd.lib()
    assert lib.causal_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 64, 0.1, None) == INVALID
    assert lib.causal_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, 1, 64, 0.1, None) == INVALID
    assert lib.causal_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 80, 0.1, None) == UNSUPPORTED
    assert lib.causal_attn_bwd(*([FAKE] * 9), 1, 8, 1, 64, 0.1, FAKE, 0, None) == INVALID


def test_workspace_sizes():
    # two float32 values per query row, rounded up to 256 bytes
    assert bd.diffusion_attn_bwd_workspace_size(2, 100, 3, 64) == -(-2 * 2 * 3 * 200 * 4 // 256) * 256
    assert bd.causal_attn_bwd_workspace_size(4, 64, 2, 128) == 2 * 4 * 2 * 64 * 4
    assert bd.diffusion_attn_bwd_workspace_size(0, 100, 3, 64) == 0
    assert bd.diffusion_attn_bwd_workspace_size(1, 100, 3, 80) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError, match="on the GPU"):
        bd.diffusion_attn_fwd(x, x, x, x.clone(), lse, 1, 4, 1, 64, 2, 0.125)


@pytest.mark.parametrize("H,H_kv", [(4, 0), (4, -1), (4, 8), (6, 4), (5, 2)])
def test_grouped_entry_points_reject_bad_kv_heads(H, H_kv):
    # 1 <= H_kv <= H with H a multiple of H_kv; the rest of each call is valid
    lib = bd.lib()
    assert lib.diffusion_attn_fwd_gqa(*([FAKE] * 5), 1, 16, H, H_kv, 64, 4, 0.125, None) == INVALID
    assert lib.diffusion_attn_bwd_gqa(*([FAKE] * 9), 1, 16, H, H_kv, 64, 4, 0.125, FAKE, 1 << 20,
                                      None) == INVALID
    assert lib.causal_attn_fwd_gqa(*([FAKE] * 5), 1, 16, H, H_kv, 64, 0.125, None) == INVALID
    assert lib.causal_attn_bwd_gqa(*([FAKE] * 9), 1, 16, H, H_kv, 64, 0.125, FAKE, 1 << 20,
                                   None) == INVALID
    assert lib.bdattn_bwd_stage(0, 0, *([FAKE] * 9), None, 1, 16, 0, H, H_kv, 64, 4, 0.125, 0.0, FAKE, 1 << 20,
                                None) == INVALID


def test_grouped_entry_points_share_the_other_checks():
    lib = bd.lib()
    assert lib.diffusion_attn_fwd_gqa(*([FAKE] * 5), 1, 16, 4, 2, 160, 4, 0.125, None) == UNSUPPORTED
    assert lib.diffusion_attn_fwd_gqa(None, *([FAKE] * 4), 1, 16, 4, 2, 64, 4, 0.125, None) == INVALID
    assert lib.diffusion_attn_bwd_gqa(*([FAKE] * 9), 1, 16, 4, 2, 64, 4, 0.125, FAKE, 4, None) == INVALID


def test_grouped_binding_checks_kv_shapes():
    import torch
    q = torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16)
    kv = torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16)  # 4 heads where 2 are expected
    lse = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError, match=r"k must have shape \(1, 8, 2, 64\)"):
        bd.diffusion_attn_fwd_gqa(q, kv, kv, q.clone(), lse, 1, 4, 4, 2, 64, 2, 0.125)


def _expected_gqa_workspace(B, n, H, Hkv, D, causal=False):
    """Statistics (two float32 per query row) plus, when the dK/dV kernel
    splits the groups, float32 partial dK and dV per split.  The split count
    is the smallest divisor S of G = H / Hkv giving at least four dK/dV
    workgroups (of 128 keys, 64 at D = 256) per resident slot: 1024, or 2048
    at D = 64 and 96 where a CU holds two (all of G when none does)."""
    T = n if causal else 2 * n
    r256 = lambda x: -(-x // 256) * 256
    bkv = 64 if D == 256 else 128
    base = -(-n // bkv) * (1 if causal else 2) * B * Hkv
    G = H // Hkv
    need = 2048 if D <= 96 else 1024
    S = next((c for c in range(1, G + 1) if G % c == 0 and base * c >= need), G)
    part = 2 * S * B * T * Hkv * D * 4 if S > 1 else 0
    return r256(2 * B * H * T * 4) + r256(part), S


@pytest.mark.parametrize("B,n,H,Hkv,D", [
    (8, 1024, 32, 8, 128),   # 1024 workgroups unsplit: S = 1
    (4, 2048, 16, 1, 64),    # multi-query, 128 workgroups: S = 16
    (8, 2048, 16, 1, 64),    # 256 workgroups: S = 8
    (2, 100, 4, 2, 64),      # tiny: every query head on its own, S = G
    (1, 7, 8, 2, 128),
    (3, 5000, 12, 12, 64),   # plain multi-head
    (2, 4096, 16, 2, 256),   # 512 workgroups of 64 keys: S = 2
    (1, 1000, 8, 1, 256),
    (2, 4096, 16, 2, 192),   # 512 workgroups of 128 keys: S = 2
    (2, 900, 12, 3, 96),
    (4, 2048, 16, 2, 96),    # 256 workgroups: S = 8 (1024 would give 4)
])
def test_gqa_workspace_sizes(B, n, H, Hkv, D):
    want, S = _expected_gqa_workspace(B, n, H, Hkv, D)
    assert bd.diffusion_attn_bwd_gqa_workspace_size(B, n, H, Hkv, D) == want
    wantc, _ = _expected_gqa_workspace(B, n, H, Hkv, D, causal=True)
    assert bd.causal_attn_bwd_gqa_workspace_size(B, n, H, Hkv, D) == wantc
    if Hkv == H:
        assert want == bd.diffusion_attn_bwd_workspace_size(B, n, H, D)
    assert bd.diffusion_attn_bwd_gqa_workspace_size(B, n, H, H + 1, D) == 0
    assert bd.diffusion_attn_bwd_gqa_workspace_size(B, n, H, 0, D) == 0


def test_gqa_bwd_rejects_a_workspace_without_room_for_partials():
    # multi-query at this size splits the groups, so the statistics alone
    # are not enough workspace
    B, n, H, D = 4, 2048, 16, 64
    stats_only = bd.diffusion_attn_bwd_workspace_size(B, n, H, D)
    assert bd.diffusion_attn_bwd_gqa_workspace_size(B, n, H, 1, D) > stats_only
    assert bd.lib().diffusion_attn_bwd_gqa(*([FAKE] * 9), B, n, H, 1, D, 4, 0.125, FAKE, stats_only,
                                           None) == INVALID


def test_varlen_rejects_bad_arguments():
    lib = bd.lib()
    # (B, max_n, total, H, H_kv, D, b)
    ok = (2, 16, 40, 4, 2, 64, 4)
    fwd = lambda cu, *a: lib.diffusion_attn_varlen_fwd(*([FAKE] * 5), cu, *a, 0.125, None)
    assert fwd(None, *ok) == INVALID                       # no offsets
    assert fwd(FAKE + 2, *ok) == INVALID                   # misaligned offsets
    assert fwd(FAKE, 2, 0, 40, 4, 2, 64, 4) == INVALID     # max_n = 0 with tokens
    assert fwd(FAKE, 2, 16, -1, 4, 2, 64, 4) == INVALID    # negative total
    assert fwd(FAKE, 0, 16, 40, 4, 2, 64, 4) == INVALID    # no samples
    assert fwd(FAKE, 2, 16, 40, 4, 3, 64, 4) == INVALID    # H not a multiple of H_kv
    assert fwd(FAKE, 2, 16, 40, 4, 2, 160, 4) == UNSUPPORTED
    # all rows past the 32-bit row limit
    assert fwd(FAKE, 2, 16, 2 ** 30, 4, 2, 64, 4) == INVALID
    bwd = lambda cu, wsb, *a: lib.diffusion_attn_varlen_bwd(*([FAKE] * 9), cu, *a, 0.125, FAKE, wsb, None)
    assert bwd(None, 1 << 30, *ok) == INVALID
    assert bwd(FAKE, 16, *ok) == INVALID                   # workspace too small
    assert lib.causal_attn_varlen_fwd(*([FAKE] * 5), None, 2, 16, 40, 4, 2, 64, 0.1, None) == INVALID


def test_varlen_with_no_tokens_launches_nothing():
    # nothing to compute: OK without touching any pointer (there is no GPU here)
    lib = bd.lib()
    assert lib.diffusion_attn_varlen_fwd(*([FAKE] * 5), FAKE, 3, 0, 0, 4, 2, 64, 4, 0.125, None) == OK
    assert lib.diffusion_attn_varlen_bwd(*([FAKE] * 9), FAKE, 3, 0, 0, 4, 2, 64, 4, 0.125, FAKE, 0,
                                         None) == OK
    assert bd.diffusion_attn_varlen_bwd_workspace_size(3, 0, 0, 4, 2, 64) == 0


def test_varlen_workspace_sizes():
    # statistics per packed row and head; partials when the groups split,
    # by the same rule as the batched layout with max_n standing for n
    B, max_n, total, H, Hkv, D = 5, 300, 1234, 8, 2, 64
    want, S = _expected_gqa_workspace(B, max_n, H, Hkv, D)
    r256 = lambda x: -(-x // 256) * 256
    part = 2 * S * total * Hkv * D * 4 if S > 1 else 0
    assert bd.diffusion_attn_varlen_bwd_workspace_size(B, max_n, total, H, Hkv, D) == \
        r256(2 * H * total * 4) + r256(part)
    assert bd.diffusion_attn_varlen_bwd_workspace_size(B, max_n, total, H, H, D) == r256(2 * H * total * 4)
    assert bd.causal_attn_varlen_bwd_workspace_size(B, max_n, total, 4, 4, 128) == r256(2 * 4 * total * 4)


def test_one_more_token_past_the_largest_sample_is_rejected():
    # 2n x H x D bf16 must stay below 2 GiB: n = 16383 at H = 256, D = 128 is
    # the largest accepted half (exercised on the GPU), n = 16384 is not
    assert _fwd(n=16384, H=256, D=128) == UNSUPPORTED
    assert bd.diffusion_attn_bwd_workspace_size(1, 16383, 256, 128) > 0
    assert bd.diffusion_attn_bwd_workspace_size(1, 16384, 256, 128) == 0


def test_fp8_forward_rejects_bad_arguments():
    lib = bd.lib()
    f = lambda qd=FAKE, kd=FAKE, vd=FAKE, D=64, H_kv=2: lib.diffusion_attn_fwd_fp8(
        FAKE, FAKE, FAKE, qd, kd, vd, FAKE, FAKE, 1, 16, 4, H_kv, D, 4, 0.125, None)
    assert f(qd=None) == INVALID and f(kd=None) == INVALID and f(vd=None) == INVALID
    assert f(vd=FAKE + 2) == INVALID            # descales must be 4-byte aligned
    assert f(D=80) == UNSUPPORTED
    for D in (96, 192, 256):                    # no FP8 kernel at these widths
        assert f(D=D) == UNSUPPORTED
    assert f(H_kv=3) == INVALID
    assert lib.causal_attn_fwd_fp8(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 16, 4, 4, 64, 0.1,
                                   None) == INVALID


def test_general_entry_points_check_softcap_and_mode():
    lib = bd.lib()
    fwd = lambda mode=0, cap=0.0: lib.bdattn_fwd(mode, *([FAKE] * 5), None, 1, 16, 0, 2, 2, 64, 4, 0.125, cap, None)
    assert fwd(cap=-1.0) == INVALID
    assert fwd(cap=float("nan")) == INVALID and fwd(cap=float("inf")) == INVALID
    assert fwd(mode=2) == INVALID
    bwd = lambda cap: lib.bdattn_bwd(0, *([FAKE] * 9), None, 1, 16, 0, 2, 2, 64, 4, 0.125, cap, FAKE, 1 << 20, None)
    assert bwd(-0.5) == INVALID
    # packed with no tokens: nothing to do, in every packed entry point
    assert lib.bdattn_fwd(0, *([FAKE] * 5), FAKE, 3, 0, 0, 2, 2, 64, 4, 0.125, 1.0, None) == OK
    assert lib.bdattn_bwd(0, *([FAKE] * 9), FAKE, 3, 0, 0, 2, 2, 64, 4, 0.125, 1.0, FAKE, 0, None) == OK
    for stage in (0, 1):
        assert lib.bdattn_bwd_stage(0, stage, *([FAKE] * 9), FAKE, 3, 0, 0, 2, 2, 64, 4, 0.125, 1.0,
                                    FAKE, 0, None) == OK


def test_general_workspace_size_matches_the_specific_ones():
    W = bd.bdattn_bwd_workspace_size
    assert W(0, 0, 2, 100, 0, 8, 2, 64) == bd.diffusion_attn_bwd_gqa_workspace_size(2, 100, 8, 2, 64)
    assert W(1, 0, 2, 100, 0, 8, 8, 128) == bd.causal_attn_bwd_workspace_size(2, 100, 8, 128)
    assert W(0, 1, 5, 300, 1234, 8, 2, 64) == bd.diffusion_attn_varlen_bwd_workspace_size(5, 300, 1234, 8, 2, 64)
    assert W(1, 1, 5, 300, 1234, 4, 4, 64) == bd.causal_attn_varlen_bwd_workspace_size(5, 300, 1234, 4, 4, 64)
    assert W(2, 0, 2, 100, 0, 8, 2, 64) == 0
