"""GPU parity of the fused retrieval path (inner-product top-k) against the
CPU oracle, and bit-exact independence from sample, bins, splits and capacity."""
import numpy as np
import pytest

from tests.gpu_util import canon, check_row, say, spaced_rows
from workloads import retrieval_inputs, retrieval_workload

pytestmark = pytest.mark.gpu


def _q_dev(r):
    import torch
    return torch.from_numpy(np.ascontiguousarray(r["q"]).view(np.int16)).cuda().view(torch.bfloat16)


def _db_host_bits(db):
    import torch
    return db.view(torch.int16).cpu().numpy().view(np.uint16)


def _check(r, idx, sc, rows, where):
    from oracle import first_copy, retrieval_row_scores
    dbh = _db_host_bits(r["db"])
    N = r["N"]
    v = np.arange(N)
    rep = first_copy(dbh)
    rows = [int(t) for t in rows]
    swaps = 0
    for i0 in range(0, len(rows), 16):   # 16 queries' scores per pass over the database
        part = rows[i0:i0 + 16]
        scores = retrieval_row_scores(r["q"], dbh, part, rep=rep)
        for t, s in zip(part, scores):
            swaps += check_row(idx[t], None if sc is None else sc[t], v, s, r["topk"], "bf16",
                               f"{where} row {t}") or 0
    return swaps


SMALL = [(40, 5000, 64, 100), (33, 7001, 128, 64), (20, 3000, 768, 50), (70, 4500, 256, 300), (9, 2100, 512, 2000),
         (12, 30000, 256, 4096), (6, 40000, 768, 8192)]   # the k-sweep's upper end


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: f"T{s[0]}_N{s[1]}_D{s[2]}_k{s[3]}")
def test_retrieval_small(lib, shape):
    import torch
    T, N, D, k = shape
    say("retrieval small", shape)
    r = retrieval_inputs(T, N, D, k, n_centres=max(2, N // 400), sigma=0.3, n_sample=3 * k if 3 * k < N else N // 2,
                         device="cuda", block=4096)
    q = _q_dev(r)
    smp = torch.from_numpy(r["sample"]).cuda()
    idx, sc = lib.retrieve(q, r["db"], k, sample=smp, return_scores=True)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    _check(r, idx, sc, range(T), f"retrieve {shape}")


def test_retrieval_degenerate_sizes(lib):
    """No queries (nothing launched), a one-row database, and fewer rows than
    k (-1 padding): every valid row is returned with its exact score."""
    import torch
    r = retrieval_inputs(0, 500, 128, 16, n_centres=4, n_sample=0, device="cuda")
    idx, sc = lib.retrieve(_q_dev(r), r["db"], 16, return_scores=True)
    assert tuple(idx.shape) == (0, 16) and tuple(sc.shape) == (0, 16)
    for T, N, D, k in [(3, 1, 64, 1), (3, 1, 64, 5), (37, 20, 128, 50), (5, 31, 768, 31)]:
        say("retrieval degenerate", (T, N, D, k))
        r = retrieval_inputs(T, N, D, k, n_centres=4, n_sample=min(N, 3 * k) // 2, device="cuda")
        smp = torch.from_numpy(r["sample"]).cuda()
        idx, sc = lib.retrieve(_q_dev(r), r["db"], k, sample=smp, return_scores=True)
        idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
        _check(r, idx, sc, range(T), f"retrieve degenerate {(T, N, D, k)}")
        for t in range(T):   # all N rows, then padding
            assert sorted(idx[t].tolist()) == [-1] * max(0, k - N) + list(range(min(N, k)))


def test_retrieval_independence(lib):
    import torch
    import indexer_topk_long_amd as ltk
    T, N, D, k = 45, 9000, 128, 80
    r = retrieval_inputs(T, N, D, k, n_centres=20, sigma=0.3, n_sample=240, device="cuda", block=4096)
    q = _q_dev(r)
    smp = torch.from_numpy(r["sample"]).cuda()
    ref, ref_sc = canon(*[x.cpu().numpy() for x in lib.retrieve(q, r["db"], k, sample=smp, return_scores=True)])
    _check(r, *[x.cpu().numpy() for x in lib.retrieve(q, r["db"], k, sample=smp, return_scores=True)], range(T), "ref")
    cases = [
        ("empty_sample", torch.zeros(0, dtype=torch.int32, device="cuda"), None),
        ("dups_invalid", torch.tensor([5, 5, 5, -1, N, N + 9, 17, 17], dtype=torch.int32, device="cuda"), None),
        ("nbins1", smp, ltk.Opts(nbins=1)),
        ("nbins1024", smp, ltk.Opts(nbins=1024)),
        ("splits1", smp, ltk.Opts(l_splits=1)),
        ("splits7", smp, ltk.Opts(l_splits=7)),
        ("ccap1", smp, ltk.Opts(cand_capacity=1)),
        ("ccap100", smp, ltk.Opts(cand_capacity=100)),
        ("sorted", smp, ltk.Opts(sorted_output=True)),
    ]
    for name, s_, o in cases:
        say("variant", name)
        got, got_sc = canon(*[x.cpu().numpy() for x in lib.retrieve(q, r["db"], k, sample=s_, opts=o, return_scores=True)])
        assert np.array_equal(got, ref), name
        assert np.array_equal(got_sc.view(np.uint32), ref_sc.view(np.uint32)), name


@pytest.mark.timeout(900)
def test_retrieval_full_size(lib):
    """The 8M x 768 retrieval workload at full size: sampled queries against the
    oracle, structure and candidate counts on every query."""
    import torch
    say("retrieval-8m-d768-bf16: generating on the GPU")
    r = retrieval_workload(device="cuda")
    T, N, k = r["T"], r["N"], r["topk"]
    q = _q_dev(r)
    smp = torch.from_numpy(r["sample"]).cuda()
    say("retrieval-8m-d768-bf16: fused")
    idx, sc, st = lib.retrieve(q, r["db"], k, sample=smp, return_scores=True, return_stats=True)
    idx_h, sc_h = idx.cpu().numpy(), sc.cpu().numpy()
    s = np.sort(idx_h, axis=1)
    assert np.all(s >= 0) and np.all(np.diff(s, axis=1) > 0) and np.all(s < N)
    say(f"retrieval-8m-d768-bf16: candidates/query {st.cand_written / T:.0f}, max {st.max_cand_per_query}, overflow rows {st.overflow_rows}")
    rows = spaced_rows(T, 64)
    say(f"retrieval-8m-d768-bf16: oracle rows {rows[:4]} ... {rows[-2:]} ({len(rows)})")
    _check(r, idx_h, sc_h, rows, "retrieval-8m")


def test_retrieval_earlier_batch_sample(lib):
    """k = 2,048 with the sample built from an earlier batch's results (the
    rows that batch's queries selected most often): exact, and bit-identical to
    the random-sample run."""
    import torch
    from workloads import retrieval_queries
    T, N, D, k = 24, 50000, 256, 2048
    r = retrieval_inputs(T, N, D, k, n_centres=60, sigma=0.3, n_sample=3 * k, device="cuda", block=8192)
    qp_raw, _ = retrieval_queries(T, D, 60, 0.3, tag=4, batch=-1)
    qp = torch.from_numpy(np.ascontiguousarray(qp_raw).view(np.int16)).cuda().view(torch.bfloat16)
    prev = lib.retrieve(qp, r["db"], k, sample=torch.from_numpy(r["sample"]).cuda())
    smp = lib.next_sample(prev, N, 3 * k)
    q = _q_dev(r)
    idx, sc = lib.retrieve(q, r["db"], k, sample=smp, return_scores=True)
    ref, ref_sc = lib.retrieve(q, r["db"], k, sample=torch.from_numpy(r["sample"]).cuda(), return_scores=True)
    a, a_sc = canon(idx.cpu().numpy(), sc.cpu().numpy())
    b, b_sc = canon(ref.cpu().numpy(), ref_sc.cpu().numpy())
    assert np.array_equal(a, b) and np.array_equal(a_sc.view(np.uint32), b_sc.view(np.uint32))
    _check(r, idx.cpu().numpy(), sc.cpu().numpy(), range(0, T, 5), "earlier-batch sample")


UNFUSED = [(40, 5000, 64, 100), (33, 7001, 128, 64), (70, 4500, 256, 300), (20, 3000, 768, 50), (9, 2100, 512, 2000)]


@pytest.mark.parametrize("shape", UNFUSED, ids=lambda s: f"T{s[0]}_N{s[1]}_D{s[2]}_k{s[3]}")
def test_unfused_retrieval(lib, shape):
    """The unfused path (full score matrix, radix select per row) returns the
    fused path's sets and bit-identical scores, and the oracle's sets."""
    import torch
    T, N, D, k = shape
    say("unfused retrieval", shape)
    r = retrieval_inputs(T, N, D, k, n_centres=max(2, N // 400), sigma=0.3, n_sample=3 * k if 3 * k < N else N // 2,
                         device="cuda", block=4096)
    q = _q_dev(r)
    idx, sc = lib.unfused_retrieve(q, r["db"], k, return_scores=True)
    ref, ref_sc = lib.retrieve(q, r["db"], k, sample=torch.from_numpy(r["sample"]).cuda(), return_scores=True)
    a, a_sc = canon(idx.cpu().numpy(), sc.cpu().numpy())
    b, b_sc = canon(ref.cpu().numpy(), ref_sc.cpu().numpy())
    assert np.array_equal(a, b) and np.array_equal(a_sc.view(np.uint32), b_sc.view(np.uint32))
    _check(r, idx.cpu().numpy(), sc.cpu().numpy(), range(0, T, 3), f"unfused {shape}")


def test_unfused_retrieval_large(lib):
    """256 queries over 1M rows of 768 dimensions (a 1 GB score matrix): the
    fused path's sets and scores, sorted output included."""
    import torch
    T, N, D, k = 256, 1 << 20, 768, 512
    say("unfused retrieval large", (T, N, D, k))
    r = retrieval_inputs(T, N, D, k, n_centres=500, sigma=0.3, n_sample=3 * k, device="cuda", block=1 << 16)
    q = _q_dev(r)
    opts = lib.Opts(sorted_output=1)
    idx, sc = lib.unfused_retrieve(q, r["db"], k, opts=opts, return_scores=True)
    ref, ref_sc = lib.retrieve(q, r["db"], k, sample=torch.from_numpy(r["sample"]).cuda(), opts=opts,
                               return_scores=True)
    assert torch.equal(idx, ref) and torch.equal(sc.view(torch.int32), ref_sc.view(torch.int32))
    _check(r, idx.cpu().numpy(), sc.cpu().numpy(), [0, 127, 255], "unfused large")
