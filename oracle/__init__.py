"""Plain float64 CPU oracle for block-diffusion attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library
and its Python binding) imports, links or runs this package; only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP path: it builds
its own explicit mask and computes dense masked softmax attention and its
analytic backward with NumPy in float64.

Every function here is pinned by ``tests/test_oracle.py`` against facts
the pages and the mathematics fix (see that file); none is "parity
unpinned".
"""
from .attention import (  # noqa: F401
    block_diffusion_mask,
    causal_mask,
    masked_attention_forward,
    masked_attention_backward,
    diffusion_forward,
    diffusion_backward,
    diffusion_forward_rows,
    diffusion_grad_q_rows,
    diffusion_grad_kv_cols,
    causal_forward,
    causal_backward,
    kv_head_of,
    grouped_forward,
    grouped_backward,
    grouped_grad_kv_cols,
    varlen_forward,
    varlen_backward,
    batched,
    to_f64,
)
from .fp8 import (  # noqa: F401
    dequantize_e4m3,
    e4m3_value,
    fp8_forward,
    fp8_output_bound,
)
