"""Block-sparse GQA attention with a pooled, page-aware block cache, for AMD MI355X (gfx950).

The compute path is the HIP library ``libbsg.so`` (C ABI in ``include/bsg.h``); this package
only marshals torch tensors into its calls.  Build it with
``python -m block_sparse_gqa_pool_amd.build``.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, BsgDims, BsgError, block_pool, block_pool_fp8, decode_step, decode_step_fp8, decode_step_gated,
    decode_step_noalloc, decode_step_tokens, decode_step_workspace_bytes, decode_workspace_bytes, dims, group_score,
    noalloc_scratch_bytes, quantize_pages_fp8, debug_errors,
    sparse_attn_decode_tokens, token_topk, token_topk_prefill, sparse_attn_prefill_tokens,
    group_score_topk, group_score_topk_workspace_bytes, lib, sparse_attn_decode, sparse_attn_prefill,
    sparse_attn_prefill_gated, topk_blocks,
)

__version__ = "1.0.0"
