"""Exact ties at the k-th score on the GPU: every path must return the
oracle's index sets exactly, with no acceptance band.  The inputs (see
tests/tie_cases.py) are built so that the k-th score of every query row lies
inside a group of bit-identical scores that the result cuts, and the lower
key indices of that group must win (the oracle's tie rule).

Covered: the fused path (default, forced overflow so that the exact fallback
decides, one bin, several key splits), the unfused baseline, decode-shape
calls (key range split over many workgroups with shared thresholds) and the
retrieval path (default and forced overflow)."""
import numpy as np
import pytest

from tests.gpu_util import check_rows, say, to_dev
from tests.tie_cases import tied_indexer_inputs, tied_retrieval_inputs
from tests.test_tie_cases import DECODE_TIE_CASES, INDEXER_TIE_CASES, RETRIEVAL_TIE_CASE

pytestmark = pytest.mark.gpu


def _exact(ref, got, where):
    ref, got = np.sort(ref, axis=1), np.sort(np.asarray(got), axis=1)
    bad = np.nonzero(np.any(ref != got, axis=1))[0]
    assert len(bad) == 0, f"{where}: rows {bad[:8].tolist()} differ from the oracle's exact sets"


@pytest.mark.parametrize("case", INDEXER_TIE_CASES, ids=lambda c: f"T{c[0]}_L{c[1]}_{c[4]}_k{c[5]}")
def test_exact_ties_fused_and_unfused(lib, case):
    import indexer_topk_long_amd as ltk
    from oracle import oracle_indexer
    inp = tied_indexer_inputs(*case[:7], tag=case[7])
    k = inp["topk"]
    ref, _ = oracle_indexer(inp)
    d = to_dev(inp)
    for name, opts in [("default", None), ("forced_overflow", ltk.Opts(cand_capacity=1)),
                       ("one_bin", ltk.Opts(nbins=1)), ("splits8", ltk.Opts(l_splits=8)),
                       ("sorted", ltk.Opts(sorted_output=True))]:
        say("ties fused", case, name)
        idx, sc = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=d["sample"], q_scale=d["q_scale"],
                                   k_scale=d["k_scale"], opts=opts, return_scores=True)
        _exact(ref, idx.cpu().numpy(), f"fused {name}")
        check_rows(inp, idx.cpu().numpy(), sc.cpu().numpy(), range(inp["T"]), f"fused {name}")
    say("ties unfused", case)
    uidx = lib.unfused_score_select(d["q"], d["k"], d["w"], d["pos"], k, q_scale=d["q_scale"], k_scale=d["k_scale"])
    _exact(ref, uidx.cpu().numpy(), "unfused")


@pytest.mark.parametrize("case", DECODE_TIE_CASES, ids=lambda c: f"T{c[0]}_L{c[1]}_{c[4]}_k{c[5]}")
def test_exact_ties_decode_shape(lib, case):
    from oracle import oracle_indexer
    inp = tied_indexer_inputs(*case[:7], tag=case[7])
    k = inp["topk"]
    ref, _ = oracle_indexer(inp)
    d = to_dev(inp)
    say("ties decode", case)
    idx, st = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=d["sample"], q_scale=d["q_scale"],
                               k_scale=d["k_scale"], return_stats=True)
    _exact(ref, idx.cpu().numpy(), "decode")
    # the step sampled from its own result, as a decode loop runs
    idx2 = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=idx.flatten(), q_scale=d["q_scale"],
                            k_scale=d["k_scale"])
    _exact(ref, idx2.cpu().numpy(), "decode, previous-result sample")


def test_exact_ties_retrieval(lib):
    import torch
    import indexer_topk_long_amd as ltk
    from oracle import oracle_retrieval
    T, N, D, k, n_src, tag = RETRIEVAL_TIE_CASE
    qb, dbb, smp = tied_retrieval_inputs(T, N, D, k, n_src, tag)
    ref, _ = oracle_retrieval(qb, dbb, k)
    q = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)
    db = torch.from_numpy(dbb.view(np.int16)).cuda().view(torch.bfloat16)
    s = torch.from_numpy(smp).cuda()
    for name, opts in [("default", None), ("forced_overflow", ltk.Opts(cand_capacity=64)),
                       ("sorted", ltk.Opts(sorted_output=True))]:
        say("ties retrieval", name)
        idx = lib.retrieve(q, db, k, sample=s, opts=opts)
        _exact(ref, idx.cpu().numpy(), f"retrieval {name}")
