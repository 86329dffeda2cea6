"""CPU oracle for index-selected sparse attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this package. The
product (the HIP library and its binding) never does, and the two share no code.
"""
from .oracle import (  # noqa: F401
    build, load, index_scores, block_scores, topk, topk_in_blocks, sparse_attn, decode_step,
    two_level_select, bf16_decode, e4m3_decode, e4m3_encode, mx_exponent, mx_quantize_bf16,
    cache_append, indexer_prolog, max_threads, LN_EPS,
    NEG_INF,
)
