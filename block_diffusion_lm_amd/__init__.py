"""Block-diffusion attention for AMD MI355X (gfx950).

The compute lives in ``libbdattn.so`` (hand-written HIP kernels behind the
C ABI of ``include/bdattn.h``); this package is its binding.
"""
from ._binding import (  # noqa: F401
    BdattnError,
    CLEAN,
    LIB_PATH,
    MODE_CAUSAL,
    MODE_DIFFUSION,
    NOISY,
    SIGNATURES,
    bdattn_bwd,
    bdattn_bwd_stage,
    bdattn_bwd_workspace_size,
    bdattn_fwd,
    bdattn_bwd_tiles,
    bdattn_fwd_tiles,
    bdattn_row_interval,
    bdattn_visible_pairs,
    causal_attn_bwd,
    causal_attn_bwd_gqa,
    causal_attn_bwd_gqa_workspace_size,
    causal_attn_bwd_workspace_size,
    causal_attn_fwd,
    causal_attn_fwd_fp8,
    causal_attn_fwd_gqa,
    causal_attn_varlen_bwd,
    causal_attn_varlen_bwd_workspace_size,
    causal_attn_varlen_fwd,
    diffusion_attn_bwd,
    diffusion_attn_bwd_gqa,
    diffusion_attn_bwd_gqa_workspace_size,
    diffusion_attn_bwd_workspace_size,
    diffusion_attn_fwd,
    diffusion_attn_fwd_fp8,
    diffusion_attn_fwd_gqa,
    diffusion_attn_varlen_bwd,
    diffusion_attn_varlen_bwd_workspace_size,
    diffusion_attn_varlen_fwd,
    lib,
    status_string,
)
from .autograd import (  # noqa: F401
    causal_attn_func,
    diffusion_attn_func,
    diffusion_attn_varlen_func,
)
