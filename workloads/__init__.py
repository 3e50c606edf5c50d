"""Seeded synthetic inputs shared by the CPU oracle, the tests and the benchmark.

Nothing in this package scores, bins or selects: it draws random numbers and
rounds them to the storage formats the kernels read.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    indexer_config,
    indexer_inputs,
    random_sample,
    retrieval_config,
    retrieval_inputs,
    to_storage,
)
