"""CPU oracle of the CSA layer step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never import, call or link it, and it shares no code with them.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against values the pages fix (worked examples under ``tests/golden/``), closed
forms, textbook special cases and brute force on tiny inputs.
"""
from .csa_oracle import (  # noqa: F401
    PAGE, EFLAG_POS_RANGE, EFLAG_BLOCK_RANGE, EFLAG_TOPK_RANGE, EFLAG_META,
    bf16_to_f64, visible_count, window_positions, owner_request,
    rotate_adjacent_pairs, materialize_rope_rows, inverse_rope, index_scores, topk,
    kv_rows_for_query, deterministic_selection, sparse_attn,
    candidate_blocks, candidate_positions, index_scores_in_candidates, topk_in_candidates,
    decode_e2m1, decode_e8m0, mx_rows, index_scores_mxfp4,
    decode_e4m3, KvPlane, bf16_plane, mxfp8_plane, mxfp4_e4m3_plane, index_scores_fp8,
    f64_to_bf16, compress_pairs,
)
