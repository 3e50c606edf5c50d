"""The Sample -> Filter -> Select model equals the plain definition for every
sample, bin count, refresh period, split count and capacity (the method's
exactness claim), and the double-counting reading it avoids really breaks it."""
import numpy as np
import pytest

from oracle import indexer_row_scores, oracle_indexer, topk_row
from oracle.model import sfs_row, threshold_from_hist
from workloads import indexer_workload, random_sample


@pytest.fixture(scope="module")
def cfg0():
    inp = indexer_workload("tiny-4k-fp32")
    prev = indexer_workload("tiny-4k-fp32", chunk=-1)
    pi, _ = oracle_indexer(prev)
    L = inp["L"]
    cnt = np.bincount(pi[pi >= 0].ravel(), minlength=L)
    prev_sample = np.lexsort((np.arange(L), -cnt))[:768]          # previous chunk's top-3k by frequency
    return inp, prev_sample


def _samples(inp, prev_sample, t, s_all, v):
    k = inp["topk"]
    worst = v[np.lexsort((v, s_all))[: 3 * k]]                    # the 3k lowest-scoring valid keys
    return {
        "previous_chunk": prev_sample,
        "random": random_sample(3 * k, inp["L"], tag=99),
        "empty": np.zeros(0, np.int64),
        "worst": worst,
        "duplicates": np.concatenate([prev_sample[:100]] * 5),
        "invalid_and_noncausal": np.concatenate([prev_sample, [-5, -1, inp["L"], inp["L"] + 7],
                                                 np.arange(inp["pos"][t] + 1, inp["L"])]),
        "single": prev_sample[:1],
    }


@pytest.mark.parametrize("nbins", [1, 2, 7, 256, 4096])
def test_model_exact_over_samples_and_bins(cfg0, nbins):
    inp, prev_sample = cfg0
    for t in (0, 31, 63):
        v, s = indexer_row_scores(inp, t)
        ref_i, ref_s = topk_row(s, v, inp["topk"])
        for name, smp in _samples(inp, prev_sample, t, s, v).items():
            got_i, got_s = sfs_row(v, s, smp, inp["topk"], nbins=nbins)
            assert np.array_equal(got_i, ref_i), (name, nbins, t)
            assert np.array_equal(got_s, ref_s)


@pytest.mark.parametrize("refresh_every", [1, 3, 0])
@pytest.mark.parametrize("n_splits", [1, 3])
@pytest.mark.parametrize("tile", [32, 256])
def test_model_exact_over_refresh_splits_tiles(cfg0, refresh_every, n_splits, tile):
    inp, prev_sample = cfg0
    for t in (5, 40):
        v, s = indexer_row_scores(inp, t)
        ref_i, _ = topk_row(s, v, inp["topk"])
        for smp in (prev_sample, random_sample(768, inp["L"], tag=7)):
            got_i, _ = sfs_row(v, s, smp, inp["topk"], refresh_every=refresh_every, n_splits=n_splits, tile=tile)
            assert np.array_equal(got_i, ref_i)


@pytest.mark.parametrize("capacity", [1, 300, None])
def test_model_overflow_fallback_exact(cfg0, capacity):
    inp, prev_sample = cfg0
    v, s = indexer_row_scores(inp, 10)
    ref_i, _ = topk_row(s, v, inp["topk"])
    tr = {}
    got_i, _ = sfs_row(v, s, prev_sample, inp["topk"], capacity=capacity, trace=tr)
    assert np.array_equal(got_i, ref_i)
    if capacity == 1:
        assert tr["overflow"]


def test_model_ties_and_small_rows():
    g = np.random.default_rng(3)
    for trial in range(40):
        n = int(g.integers(1, 400))
        k = int(g.integers(1, 120))
        s = g.integers(0, 6, n).astype(np.float64)                 # heavy ties
        v = np.arange(n)
        smp = g.integers(-3, n + 3, int(g.integers(0, 3 * k + 1)))
        for nbins in (1, 3, 64):
            got, _ = sfs_row(v, s, smp, k, nbins=nbins, flush=int(g.choice([8, 64])), tile=int(g.choice([4, 32])))
            ref, _ = topk_row(s, v, k)
            assert np.array_equal(got, ref), (trial, nbins)


def test_model_good_sample_keeps_few_candidates(cfg0):
    """With the previous chunk's sample the scan keeps about k candidates, not L."""
    inp, prev_sample = cfg0
    v, s = indexer_row_scores(inp, 63)
    tr = {}
    sfs_row(v, s, prev_sample, inp["topk"], trace=tr)
    assert inp["topk"] <= tr["n_cand"] < 4 * inp["topk"] < len(v)
    assert tr["thr0"] > 0


def test_seeding_histogram_with_sample_breaks_exactness():
    """Counting the sample keys in the histogram and again during the scan can
    push the threshold above the true k-th key's bin (the reading the model rejects)."""
    g = np.random.default_rng(11)
    n, k = 3000, 100
    s = g.standard_normal(n)
    order = np.argsort(-s)
    kth = order[k - 1]
    # move the true k-th best key to the last index, so the scan meets it last
    s[[kth, n - 1]] = s[[n - 1, kth]]
    v = np.arange(n)
    top = np.argsort(-s)[:k]
    assert top[k - 1] == n - 1
    sample = top[: k - 1]                                          # the k-1 best keys, without the k-th
    ref, _ = topk_row(s, v, k)
    good, _ = sfs_row(v, s, sample, k, nbins=64)
    bad, _ = sfs_row(v, s, sample, k, nbins=64, seed_hist=True)
    assert np.array_equal(good, ref)
    assert not np.array_equal(bad, ref)


def test_threshold_from_hist():
    assert threshold_from_hist(np.array([5, 0, 3, 2]), 4) == 2
    assert threshold_from_hist(np.array([5, 0, 3, 2]), 2) == 3
    assert threshold_from_hist(np.array([5, 0, 3, 2]), 11) == 0
    assert threshold_from_hist(np.array([0, 0, 0]), 1) == 0
