"""CPU oracle for the DSA hot path (test infrastructure only; see dsa_oracle)."""
from .dsa_oracle import (  # noqa: F401
    decode_bf16_bits, e4m3fn_table, decode_e4m3, decode_e8m0, decode_values,
    query_position, paged_rows, indexer_scores, topk_select, sparse_attention,
    zigzag_units, indexer_query, sfa_query, run_query,
    round_bf16_bits, e4m3_encode, fp8_quantise, mx_quantise, layer_norm, prolog_token,
    quantise_query, quantise_key, append_position,
)
