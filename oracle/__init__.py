"""fp64 CPU oracle for block-sparse attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the product path never does.
"""
from .sparge_oracle import (  # noqa: F401
    NEG_INF, attend, block_map, block_mean, block_self_similarity,
    block_sparse_attention, block_sparse_attention_pv_skip,
    block_sparse_attention_qk_fp8, block_sparse_attention_qk_int8, causal_valid, cdf_count, combine, dense_attention, dequantize_int8, e4m3_code, e4m3_value, quantize_block_fp8, quantize_fp8, round_e4m3, E4M3_MAX,
    lut_from_selection, pool_and_gate, pooled_scores, pv_skip_blocks, quantize_block_int8, quantize_int8, row_softmax,
    select_from_probs, select_row, selection_order, smooth_keys,
    token_list_attention, topk_count,
)
