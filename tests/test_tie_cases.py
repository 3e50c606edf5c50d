"""The exact-tie inputs of the GPU tie tests, checked on the CPU: in every
query row the k-th score falls inside a group of bit-identical scores that
the result cuts, and no other score value lies within GAP * max|I| of it, so
the GPU tests can require the oracle's index sets exactly."""
import numpy as np
import pytest

import oracle as O
from tests.tie_cases import GAP, boundary_stats, tied_indexer_inputs, tied_retrieval_inputs

INDEXER_TIE_CASES = [
    # (T, L, H, D, dtype, topk, n_src, tag)
    (40, 6000, 64, 128, "fp8", 200, 37, 3),
    (40, 6000, 64, 128, "bf16", 200, 37, 4),
    (24, 3001, 4, 64, "f32", 100, 29, 5),
]
DECODE_TIE_CASES = [(1, 65536, 64, 128, "fp8", 512, 150, 6), (8, 65536, 64, 128, "fp8", 512, 150, 6)]
RETRIEVAL_TIE_CASE = (64, 50000, 128, 256, 300, 7)   # (T, N, D, topk, n_src, tag)


@pytest.mark.parametrize("case", INDEXER_TIE_CASES + DECODE_TIE_CASES, ids=lambda c: f"T{c[0]}_L{c[1]}_{c[4]}")
def test_indexer_tie_fixture(case):
    inp = tied_indexer_inputs(*case[:7], tag=case[7])
    keys = O.key_table(inp)
    for t in range(inp["T"]):
        _, s = O.indexer_row_scores(inp, t, keys)
        split, gap = boundary_stats(s, inp["topk"])
        assert split and gap >= GAP, (t, split, gap)


def test_retrieval_tie_fixture():
    T, N, D, k, n_src, tag = RETRIEVAL_TIE_CASE
    qb, dbb, _ = tied_retrieval_inputs(T, N, D, k, n_src, tag)
    rep = O.first_copy(dbb)
    for t in range(T):
        s = O.retrieval_row_scores(qb, dbb, t, rep=rep)
        split, gap = boundary_stats(s, k)
        assert split and gap >= GAP, (t, split, gap)
