"""MI355X (gfx950) fused exact attention forward: bf16 and FP8 E4M3 paths.

The compute lives in hand-written HIP kernels behind the C ABI of
``include/fa.h`` (built into ``libfa.so`` next to this file); the functions
here only marshal torch tensors into that ABI.
"""

from ._lib import (  # noqa: F401
    FaError,
    bwd_bf16,
    bwd_bf16_gqa,
    decode_splits,
    decode_workspace_bytes,
    fp8_prep,
    fp8_prep_v,
    fp8_ref_block,
    fp8_vt_ld,
    fwd_bf16,
    fwd_bf16_decode,
    fwd_bf16_decode_noalloc,
    fwd_bf16_gqa,
    fwd_bf16_varlen,
    fwd_fp8,
    load,
)

__all__ = ["fwd_bf16", "fwd_bf16_gqa", "fwd_bf16_varlen", "fwd_bf16_decode", "fwd_bf16_decode_noalloc", "decode_splits", "decode_workspace_bytes",
           "bwd_bf16", "bwd_bf16_gqa", "fp8_prep", "fp8_prep_v", "fwd_fp8", "fp8_vt_ld", "fp8_ref_block", "load", "FaError"]
