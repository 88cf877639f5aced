"""Block-sparse video-DiT attention (LVSA and Draft Attention masks) for MI355X.

The compute lives in the HIP library liblvsa.so (C ABI: include/lvsa.h);
this package is its thin Python binding plus the seeded synthetic-input
generator (``synth``). Importing the package does not load the library;
the first call of a binding function does, and raises if it is missing.
"""
from ._lib import (  # noqa: F401
    LvsaError,
    block_sparse_attn_fwd,
    block_sparse_attn_fwd_fp8,
    dense_attn_fwd,
    dense_attn_fwd_fp8,
    draft_attn_fwd,
    draft_attn_fwd_fp8,
    draft_grid_info,
    draft_mask_and_perm,
    draft_scores,
    draft_workspace_bytes,
    fp8_pitch,
    load,
    lvsa_mask,
    lvsa_mask_capacity,
    quantize_fp8_e4m3,
    quantize_qkv_fp8,
    token_permute,
)

__version__ = "0.1.0"
