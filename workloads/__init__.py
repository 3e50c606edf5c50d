"""Seeded synthetic inputs shared by the CPU oracle, the tests and the benchmark.

Nothing in this package scores, bins or selects: it draws random numbers and
rounds them to the storage formats the kernels read.
"""
from .gen import (  # noqa: F401
    INDEXER_WORKLOADS,
    WORKLOADS,
    indexer_keys,
    indexer_workload,
    indexer_inputs,
    prefill_queries,
    random_retrieval_sample_of,
    random_sample,
    retrieval_workload,
    retrieval_inputs,
    retrieval_queries,
    selection_rows,
    to_storage,
)
