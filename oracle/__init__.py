"""CPU oracle for the fused Indexer-TopK -- TEST INFRASTRUCTURE ONLY.

Imported only by the tests, the smoke check and the benchmark's CPU-baseline
leg.  It shares no code with the GPU library and never imports it.
"""
from .oracle import (  # noqa: F401
    bf16_to_f64,
    decode,
    dsa_gather,
    dsa_pack,
    e4m3fn_table,
    first_copy,
    key_table,
    indexer_row_scores,
    indexer_scores,
    next_sample,
    oracle_indexer,
    oracle_retrieval,
    retrieval_row_scores,
    retrieval_scores,
    topk_row,
    valid_keys,
)
from . import model  # noqa: F401
