"""CPU oracle for exact attention (test infrastructure only).

Only the test suite, the smoke check and the bench's CPU-baseline leg may import
this package; the GPU library never does.
"""
from .attn_ref import (  # noqa: F401
    alibi_slopes,
    attn_ref_bwd,
    attn_ref_blocksparse,
    attn_ref_keybias,
    attn_ref_fwd_fp8,
    e4m3_to_f64,
    philox4x32_10,
    philox_keep,
    dropout_threshold,
    attn_ref_dropout,
    attn_ref_bwd_loop,
    attn_ref_fwd,
    attn_ref_varlen,
    head_backward,
    head_forward,
    to_f64,
)
