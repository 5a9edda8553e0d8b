"""MI355X-native compressed-sparse-attention (CSA) layer step.

The hot path lives in libcsa.so (hand-written HIP for gfx950 behind the C ABI
declared in include/csa.h).  This package is its thin binding: ``_lib`` has one
function per C entry point, ``runner.CsaStep`` holds device buffers for a
whole step.  There is no CPU fallback: without the built library every call
raises.
"""
from ._lib import (  # noqa: F401
    CsaError, EXPORTS, LIB_PATH, load,
    csa_status_string, csa_materialize_rope_rows, csa_index_score, csa_topk,
    csa_topk_workspace_bytes, csa_sparse_attn_decode, csa_sparse_attn_prefill,
    csa_sparse_attn_workspace_bytes, csa_candidate_blocks, csa_candidate_blocks_workspace_bytes,
    csa_index_score_candidates, csa_topk_candidates, csa_topk_candidates_workspace_bytes,
    csa_index_score_mxfp4, csa_sparse_attn_decode_noalloc, csa_sparse_attn_noalloc_max_bytes,
    csa_sparse_attn_decode_mx, csa_sparse_attn_mx_workspace_bytes, csa_index_score_fp8,
    csa_inverse_rope, csa_compress_pairs, csa_sparse_attn_decode_rope,
    csa_sparse_attn_decode_mx_rope, csa_compress_pairs_rope,
)
from .runner import CsaStep, step_for_config  # noqa: F401
