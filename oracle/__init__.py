"""CPU oracle of the index-selection sparse attention layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  Every function is pinned
by CPU tests against exact arithmetic, brute force, closed forms and library
routines (see tests/test_oracle.py)."""
from .lisfa_oracle import (  # noqa: F401
    decode_bf16, decode_e4m3, e4m3_table, decode_e8m0, decode_mx, encode_e4m3, mx_quantize, slots, indexer_keys, latent_rows,
    decode_tile_scaled, KV_TILE,
    indexer_query, mla_query, indexer_scores, select_topk, sparse_mla,
    layer_row, attend_row, scores_row,
)
from .cp_oracle import (  # noqa: F401
    shard_candidates, merge_candidates, combine_partials, zigzag_segments,
    zigzag_share, zigzag_order, zigzag_restore,
)
from .prolog_oracle import layer_norm, fp8_token_quantize, quantize_q, bf16_round  # noqa: F401
