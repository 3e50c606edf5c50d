"""GPU parity of the fused indexer path and the unfused baseline against the
CPU oracle, and bit-exact agreement of the GPU paths with each other."""
import numpy as np
import pytest

from tests.gpu_util import canon, check_rows, oracle_prev_chunk_sample, say, to_dev
from workloads import selection_rows, indexer_inputs, indexer_workload, random_sample

pytestmark = pytest.mark.gpu


def _run_fused(lib, d, topk, opts=None, sample="default"):
    smp = d["sample"] if isinstance(sample, str) else sample
    idx, sc = lib.score_select(d["q"], d["k"], d["w"], d["pos"], topk, sample=smp, q_scale=d["q_scale"],
                               k_scale=d["k_scale"], opts=opts, return_scores=True)
    return idx.cpu().numpy(), sc.cpu().numpy()


def _run_unfused(lib, d, topk):
    idx, sc = lib.unfused_score_select(d["q"], d["k"], d["w"], d["pos"], topk, q_scale=d["q_scale"],
                                       k_scale=d["k_scale"], return_scores=True)
    return idx.cpu().numpy(), sc.cpu().numpy()


@pytest.fixture(scope="module")
def tiny():
    """The tiny workload as stated: 64 queries at positions 4032..4095, sampled
    by the top-768 of the previous 64-query chunk (positions 3968..4031)."""
    inp = indexer_workload("tiny-4k-fp32", with_prev=True)
    inp["sample"] = oracle_prev_chunk_sample(inp)
    return inp


def test_tiny_previous_chunk_sample(tiny):
    """The previous chunk's top-768 covers most of this chunk's top-256."""
    from oracle import oracle_indexer
    ref = oracle_indexer(tiny, with_scores=False)
    assert len(tiny["sample"]) == 768 and len(np.unique(tiny["sample"])) == 768
    hit = np.isin(ref, tiny["sample"]).mean()
    say("tiny: previous-chunk sample holds", hit, "of the top-k")
    assert hit > 0.8


def test_device_is_gfx950(lib):
    assert lib.device_check() == 0


def test_unfused_tiny_vs_oracle(lib, tiny):
    say("unfused tiny-4k-fp32")
    d = to_dev(tiny)
    idx, sc = _run_unfused(lib, d, tiny["topk"])
    check_rows(tiny, idx, sc, range(tiny["T"]), "unfused tiny")


def test_fused_tiny_vs_oracle_and_unfused(lib, tiny):
    say("fused tiny-4k-fp32")
    d = to_dev(tiny)
    idx, sc = _run_fused(lib, d, tiny["topk"])
    check_rows(tiny, idx, sc, range(tiny["T"]), "fused tiny")
    uidx, usc = _run_unfused(lib, d, tiny["topk"])
    a, asc = canon(idx, sc)
    b, bsc = canon(uidx, usc)
    assert np.array_equal(a, b)
    assert np.array_equal(asc.view(np.uint32), bsc.view(np.uint32))   # identical fp32 scores


SMALL = [
    # (T, L, H, D, dtype, topk, n_hot) -- ragged T and L, padded heads
    (37, 3001, 64, 128, "bf16", 100, 200),
    (37, 3001, 64, 128, "fp8", 100, 200),
    (19, 2500, 20, 64, "bf16", 64, 100),
    (16, 1100, 33, 64, "fp8", 300, 50),
    (9, 777, 8, 128, "f32", 50, 40),
    (37, 3001, 64, 128, "f32", 100, 200),   # two head blocks: fragments read in pieces, 32 KB tiles
    (19, 2500, 40, 64, "f32", 64, 100),     # two head blocks, 64 KB tiles
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: f"T{s[0]}_L{s[1]}_H{s[2]}_D{s[3]}_{s[4]}_k{s[5]}")
def test_fused_small_shapes(lib, shape):
    T, L, H, D, dt, k, nh = shape
    say("small", shape)
    inp = indexer_inputs(T, L, H, D, dt, k, nh, drift=True, tag=21, n_sample=3 * k)
    d = to_dev(inp)
    idx, sc = _run_fused(lib, d, k)
    check_rows(inp, idx, sc, range(T), f"fused {shape}")
    uidx, usc = _run_unfused(lib, d, k)
    check_rows(inp, uidx, usc, range(T), f"unfused {shape}")
    a, asc = canon(idx, sc)
    b, bsc = canon(uidx, usc)
    assert np.array_equal(a, b) and np.array_equal(asc.view(np.uint32), bsc.view(np.uint32))


def _variants(inp):
    L, k = inp["L"], inp["topk"]
    base = inp["sample"]
    worst = np.arange(0, min(3 * k, L), dtype=np.int32)
    return {
        "random": base,
        "empty": np.zeros(0, np.int32),
        "single": base[:1],
        "low_index_keys": worst,
        "dups_invalid": np.concatenate([base[:50]] * 4 + [np.array([-7, -1, L, L + 100], np.int32)]).astype(np.int32),
        "other_seed": random_sample(3 * k, L, tag=77),
        # 16,384 entries: the largest sample de-duplicated in one workgroup's hash table
        "hash_table_full": np.resize(random_sample(min(4000, L), L, tag=78), 16384).astype(np.int32),
        # past that size the key bitmap de-duplicates (duplicates and invalid entries included)
        "bitmap_path": np.concatenate([np.resize(random_sample(min(3000, L), L, tag=79), 20000),
                                       np.array([-3, L, L + 9], np.int32)]).astype(np.int32),
    }


def test_sample_with_many_distinct_keys(lib):
    """More distinct sample keys than the statistics hold in registers (16 per
    thread of 1,024): the statistics loop over the sample, and the result is
    exact and equal to the unfused path's."""
    import torch
    T, L, k = 12, 40000, 300
    inp = indexer_inputs(T, L, 64, 128, "fp8", k, 600, drift=True, tag=82)
    d = to_dev(inp)
    smp = np.concatenate([random_sample(20000, L, tag=83), random_sample(5000, L, tag=84)]).astype(np.int32)
    say("distinct sample keys", len(np.unique(smp)))
    idx, sc = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=torch.from_numpy(smp).cuda(),
                               q_scale=d["q_scale"], k_scale=d["k_scale"], return_scores=True)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    check_rows(inp, idx, sc, range(T), "many distinct sample keys")
    uidx, usc = _run_unfused(lib, d, k)
    a, asc = canon(idx, sc)
    b, bsc = canon(uidx, usc)
    assert np.array_equal(a, b) and np.array_equal(asc.view(np.uint32), bsc.view(np.uint32))


@pytest.mark.parametrize("dt,H,D", [("bf16", 64, 128), ("fp8", 64, 128), ("fp8", 20, 64), ("f32", 20, 64)])
def test_sample_scored_by_the_scan(lib, dt, H, D):
    """Calls of 2,048 queries or more score their sample with the scan's
    full-score form over the gathered sample rows.  Samples whose distinct
    count is not a multiple of the tile, with duplicates and invalid entries,
    none, and 16,384 entries, and bin counts that select the scan's other
    tile variants: exact on sampled rows, and every row equal to the unfused
    path's, scores bit for bit."""
    import torch
    import indexer_topk_long_amd as ltk
    T, L, k = 2048, 6000, 200
    inp = indexer_inputs(T, L, H, D, dt, k, 400, drift=True, tag=86, n_sample=3 * k)
    d = to_dev(inp)
    uidx, usc = canon(*_run_unfused(lib, d, k))
    rows = list(range(0, T, 128)) + [T - 2, T - 1]
    cases = [(name, smp, None) for name, smp in _variants(inp).items()
             if name in ("random", "empty", "dups_invalid", "hash_table_full")]
    cases += [(f"random_nbins{nb}", _variants(inp)["random"], ltk.Opts(nbins=nb)) for nb in (800, 1024)]
    for name, smp, o in cases:
        say("sample", name, len(smp))
        idx, sc = _run_fused(lib, d, k, opts=o, sample=torch.from_numpy(np.asarray(smp, np.int32)).cuda())
        check_rows(inp, idx, sc, rows, f"{dt} H{H} D{D} sample {name}")
        a, asc = canon(idx, sc)
        assert np.array_equal(a, uidx), name
        assert np.array_equal(asc.view(np.uint32), usc.view(np.uint32)), name


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_sample_bins_refresh_capacity_independence(lib, dt):
    """The result does not depend on the sample, the bin count, the refresh
    period, the key split or the buffer capacity (forced overflow included):
    the GPU output is bit-identical across all of them, although the scan's
    gate threshold differs per case."""
    inp = indexer_inputs(24, 5000, 64, 128, dt, 200, 300, drift=True, tag=31, n_sample=600)
    d = to_dev(inp)
    import indexer_topk_long_amd as ltk
    ref, ref_sc = canon(*_run_fused(lib, d, 200))
    check_rows(inp, *_run_fused(lib, d, 200), range(24), "reference")
    import torch
    cases = []
    for name, smp in _variants(inp).items():
        cases.append((name, torch.from_numpy(smp).cuda(), None))
    # 800 bins: the wide tiles no longer fit the LDS, three 32 KB stages do
    # (1,024 bins: two); each bin count below takes its own scan variant
    for nb in (1, 2, 7, 800, 1024):
        cases.append((f"nbins{nb}", d["sample"], ltk.Opts(nbins=nb)))
    for r in (3, -1):
        cases.append((f"refresh{r}", d["sample"], ltk.Opts(refresh_every=r)))
    for sp in (1, 3, 8):
        cases.append((f"splits{sp}", d["sample"], ltk.Opts(l_splits=sp)))
    for cap in (1, 64, 250):
        cases.append((f"ccap{cap}", d["sample"], ltk.Opts(cand_capacity=cap)))
    cases.append(("flush32", d["sample"], ltk.Opts(flush_batch=32)))
    cases.append(("flush32_ccap250_refresh3", d["sample"], ltk.Opts(flush_batch=32, cand_capacity=250, refresh_every=3)))
    cases.append(("nbins1_ccap1_empty", torch.zeros(0, dtype=torch.int32, device="cuda"),
                  ltk.Opts(nbins=1, cand_capacity=1, refresh_every=-1)))
    for name, smp, o in cases:
        say("variant", name)
        got, got_sc = canon(*_run_fused(lib, d, 200, opts=o, sample=smp))
        assert np.array_equal(got, ref), name
        assert np.array_equal(got_sc.view(np.uint32), ref_sc.view(np.uint32)), name


@pytest.mark.parametrize("w_range", [(-1.0, 1.0), (-1.0, 0.0)], ids=["mixed_sign", "non_positive"])
def test_fp8_signed_head_weights(lib, w_range):
    """Head weights of either sign, so that scores can be negative: fused =
    oracle = unfused, bit-identical scores."""
    say("fp8 signed weights", w_range)
    inp = indexer_inputs(40, 6000, 64, 128, "fp8", 150, 300, drift=True, w_range=w_range, tag=43, n_sample=450)
    d = to_dev(inp)
    idx, sc = _run_fused(lib, d, 150)
    check_rows(inp, idx, sc, range(40), f"fused {w_range}")
    uidx, usc = _run_unfused(lib, d, 150)
    a, asc = canon(idx, sc)
    b, bsc = canon(uidx, usc)
    assert np.array_equal(a, b) and np.array_equal(asc.view(np.uint32), bsc.view(np.uint32))


def test_forced_overflow_reports_stats(lib):
    import indexer_topk_long_amd as ltk
    inp = indexer_inputs(16, 2000, 64, 128, "fp8", 64, 100, drift=True, tag=41, n_sample=192)
    d = to_dev(inp)
    idx, st = lib.score_select(d["q"], d["k"], d["w"], d["pos"], 64, sample=d["sample"], q_scale=d["q_scale"],
                               k_scale=d["k_scale"], opts=ltk.Opts(cand_capacity=8), return_stats=True)
    assert st.overflow_rows == 16
    check_rows(inp, idx.cpu().numpy(), None, range(16), "overflow")
    idx2, st2 = lib.score_select(d["q"], d["k"], d["w"], d["pos"], 64, sample=d["sample"], q_scale=d["q_scale"],
                                 k_scale=d["k_scale"], return_stats=True)
    assert st2.overflow_rows == 0 and 64 * 16 <= st2.cand_written and st2.max_cand_per_query >= 64
    assert np.array_equal(canon(idx.cpu().numpy()), canon(idx2.cpu().numpy()))
    # bytes written: 8 per stored candidate, 4 per (query, distinct sample key), 4 per output index
    smp = np.asarray(inp["sample"])
    nu = len(np.unique(smp[(smp >= 0) & (smp < inp["L"])]))
    assert st2.bytes_written == 8 * st2.cand_written + 4 * nu * 16 + 4 * 64 * 16
    # an overflowed row stores only its capacity (8 entries), in the first pass
    # and again in its rescan, whose buffer overflows too (the exact fallback)
    assert st.bytes_written == 2 * 8 * 8 * 16 + 4 * nu * 16 + 4 * 64 * 16


def test_edge_positions_and_small_k(lib):
    """Rows with fewer valid keys than k (padding), no valid key, k = 1, unsorted
    and repeated positions, positions past the context."""
    T, L = 12, 700
    pos = np.array([0, 5, 699, 3, 350, -1, 1000, 63, 64, 65, 5, 200], np.int32)
    for k in (1, 10, 128):
        inp = indexer_inputs(T, L, 64, 128, "bf16", k, 40, tag=51, pos=pos, n_sample=3 * k)
        d = to_dev(inp)
        say("edge k", k)
        idx, sc = _run_fused(lib, d, k)
        check_rows(inp, idx, sc, range(T), f"edge k={k}")
        uidx, usc = _run_unfused(lib, d, k)
        check_rows(inp, uidx, usc, range(T), f"edge unfused k={k}")


def test_degenerate_sizes(lib):
    """No queries (empty outputs, nothing launched) and a one-key context in
    every dtype: positions 0, -1 and past the context, k above the one valid
    key, and sample entries past the context (dropped by the preparation)."""
    for dt in ("f32", "bf16", "fp8"):
        inp = indexer_inputs(0, 500, 64, 128, dt, 16, 10, tag=55, pos=np.zeros(0, np.int32), n_sample=48)
        d = to_dev(inp)
        say("degenerate T=0", dt)
        idx, sc = _run_fused(lib, d, 16)
        assert idx.shape == (0, 16) and sc.shape == (0, 16)
        uidx, usc = _run_unfused(lib, d, 16)
        assert uidx.shape == (0, 16) and usc.shape == (0, 16)
        pos = np.array([0, -1, 7, 0, 3], np.int32)
        for k in (1, 4):
            inp = indexer_inputs(5, 1, 64, 128, dt, k, 1, tag=56, pos=pos, n_sample=3 * k)
            d = to_dev(inp)
            say("degenerate L=1", dt, "k", k)
            idx, sc = _run_fused(lib, d, k)
            check_rows(inp, idx, sc, range(5), f"L=1 {dt} k={k}")
            for t in range(5):   # the one key, or nothing, then padding
                assert sorted(idx[t].tolist()) == [-1] * (k - (pos[t] >= 0)) + [0] * int(pos[t] >= 0)
            uidx, usc = _run_unfused(lib, d, k)
            check_rows(inp, uidx, usc, range(5), f"L=1 unfused {dt} k={k}")


def test_sorted_output(lib):
    """Sorted rows, (score desc, index asc), with and without the scores
    returned, through the finalize and through the overflow fallback."""
    import indexer_topk_long_amd as ltk
    inp = indexer_inputs(10, 3000, 64, 128, "bf16", 150, 200, tag=61, n_sample=450)
    d = to_dev(inp)
    for cap in (0, 1):
        o = ltk.Opts(sorted_output=True, cand_capacity=cap)
        idx, sc = _run_fused(lib, d, 150, opts=o)
        for t in range(10):
            keys = list(zip(-sc[t].astype(np.float64), idx[t]))
            assert keys == sorted(keys)
        check_rows(inp, idx, sc, range(10), "sorted")
        only = lib.score_select(d["q"], d["k"], d["w"], d["pos"], 150, sample=d["sample"], opts=o).cpu().numpy()
        assert np.array_equal(only, idx), f"sorted without scores, capacity {cap}"


def test_determinism(lib, tiny):
    d = to_dev(tiny)
    a = _run_fused(lib, d, tiny["topk"])
    for _ in range(5):
        b = _run_fused(lib, d, tiny["topk"])
        assert np.array_equal(canon(a[0]), canon(b[0]))


def _next_sample_cases():
    g = np.random.default_rng(3)
    cases = [("random", g.integers(-1, 500, size=(64, 40)).astype(np.int32), 500, 120)]
    # the 1M-context chunk shape: 2,048 overlapping top-2,048 rows, 6,144 keys
    cases.append(("chunk_1m", selection_rows(2048, 2048, 1 << 20, tag=81), 1 << 20, 6144))
    # every row the same 3,000 keys, spread over several workgroups' ranges:
    # the threshold cuts a tie of 3,000 keys, taken in index order
    keys = np.sort(g.choice(40000, 3000, replace=False)).astype(np.int32)
    cases.append(("one_big_tie", np.tile(keys, (50, 1)), 40000, 1234))
    # fewer selected keys than samples: keys never selected fill in by index
    cases.append(("zeros_fill", g.integers(0, 70000, size=(3, 100)).astype(np.int32), 70000, 5000))
    # counts past the histogram's range (20,000 rows): the ranking fallback
    hot = np.tile(np.array([7, 3, 900, 12], np.int32), (20000, 1))
    hot[::3, 1] = 5   # counts 13,333 and 6,667 below and 20,000 above the range end
    cases.append(("counts_past_range", hot, 1000, 3))
    # repeated keys within rows, invalid entries, a ragged key range
    rep = g.integers(-3, 12305, size=(40, 64)).astype(np.int32)
    rep[:, 32:] = rep[:, :32]
    cases.append(("repeats_ragged", rep, 12305, 777))
    cases.append(("no_rows", np.zeros((0, 16), np.int32), 300, 50))
    return cases


@pytest.mark.parametrize("case", _next_sample_cases(), ids=lambda c: c[0])
def test_next_sample_vs_oracle(lib, case):
    import torch
    from oracle import next_sample
    name, prev, L, n = case
    say("next_sample", name, prev.shape, L, n)
    got = lib.next_sample(torch.from_numpy(np.ascontiguousarray(prev)).cuda(), L, n).cpu().numpy()
    assert got.shape == (n,)
    assert np.array_equal(np.sort(got), np.sort(next_sample(prev, L, n))), name


def test_no_sample_draws_its_own(lib):
    """With no sample the library samples 3k evenly spaced causal keys itself:
    at a long context the gate is no longer open, so no row overflows, and the
    result is exact."""
    T, L, k = 24, 200000, 256
    inp = indexer_inputs(T, L, 64, 128, "fp8", k, 2000, drift=True, tag=44)
    d = to_dev(inp)
    idx, st = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, q_scale=d["q_scale"], k_scale=d["k_scale"],
                               return_stats=True)
    say("no sample: candidates/query", st.cand_written / T, "overflow rows", st.overflow_rows)
    assert st.overflow_rows == 0
    check_rows(inp, idx.cpu().numpy(), None, [0, 11, T - 1], "no sample")


@pytest.mark.parametrize("H,D", [(64, 128), (33, 64)], ids=["H64_D128", "H33_D64"])
def test_fp8_score_precision(lib, H, D):
    """fp8 scores carry the linear term as four fp8 parts (about 16
    significant bits): every returned score is within 1e-4 of the row's
    largest |score| of the oracle's fp64 value, far inside the 2e-2 fp8
    tolerance, so a part dropped or mis-scaled fails here first."""
    from oracle import indexer_row_scores, key_table
    inp = indexer_inputs(40, 6000, H, D, "fp8", 150, 300, drift=True, w_range=(-0.2, 1.0), tag=47, n_sample=450)
    d = to_dev(inp)
    idx, sc = _run_fused(lib, d, 150)
    uidx, usc = _run_unfused(lib, d, 150)
    keys = key_table(inp)
    worst = 0.0
    for t in range(40):
        v, s = indexer_row_scores(inp, t, keys)
        for gi, gs in ((idx[t], sc[t]), (uidx[t], usc[t])):
            m = gi >= 0
            err = np.abs(gs[m].astype(np.float64) - s[gi[m]]) / np.abs(s).max()
            worst = max(worst, float(err.max()))
    say("fp8 worst score error / max|I|:", worst)
    assert worst <= 1e-4


def test_overflow_rescan_resolves_rows(lib):
    """A weak (random) sample lets about k ln(N / k) keys per key split through
    the early, low gate, so a small buffer overflows; the rescan of those rows,
    gated at their first pass's final threshold bin, fits.  Exact against the
    oracle and bit-identical to the unfused path."""
    import indexer_topk_long_amd as ltk
    T, L, k, cap = 32, 200000, 512, 3000
    inp = indexer_inputs(T, L, 64, 128, "fp8", k, 2000, drift=True, tag=71, n_sample=3 * k)
    d = to_dev(inp)
    idx, sc, st = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=d["sample"], q_scale=d["q_scale"],
                                   k_scale=d["k_scale"], opts=ltk.Opts(cand_capacity=cap), return_scores=True,
                                   return_stats=True)
    say("rescan: overflow rows", st.overflow_rows, "candidates/query", st.cand_written / T)
    assert st.overflow_rows > 0
    smp = np.asarray(inp["sample"])
    nu = len(np.unique(smp))
    # some rescanned row stored fewer than its capacity: the rescan, not the
    # exact fallback, resolved it
    assert st.bytes_written < 8 * 2 * cap * T + 4 * nu * T + 8 * k * T
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    check_rows(inp, idx, sc, [0, 7, 19, T - 1], "rescan")
    uidx, usc = _run_unfused(lib, d, k)
    a, asc = canon(idx, sc)
    b, bsc = canon(uidx, usc)
    assert np.array_equal(a, b) and np.array_equal(asc.view(np.uint32), bsc.view(np.uint32))
