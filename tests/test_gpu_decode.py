"""Decode and speculative-decode steps (LiteTopK pages, "Significance": the
method is said to extend to decode and speculative decoding).

A step is T = 1..8 queries at the newest positions of a long context.  Its
key range is split over many workgroups whose per-query threshold
histograms are shared in device memory.  Every row is checked against the
oracle and the index sets are checked against the unfused path bit for bit.
This is done with a good sample (the previous step's result), with a poor
one (seeded random keys), with sharing forced on and off, over a chain of
steps, and under HIP graph capture.
"""
import numpy as np
import pytest

from tests.gpu_util import canon, check_rows, say, to_dev
from workloads import indexer_inputs

pytestmark = pytest.mark.gpu


def _step_inputs(T, L, H, D, dt, k, nh, step, keys=None, tag=61):
    """Queries of decode step `step` (0 = the newest T positions, -1 the T before, ...)."""
    return indexer_inputs(T, L, H, D, dt, k, nh, drift=True, tag=tag, chunk=step, keys=keys, n_sample=6144)


def _keys(inp):
    return (inp["k"], inp["k_scale"], inp["hot"])


CASES = [
    # (T, L, H, D, dtype, k, n_hot, sample) -- 32 splits of 4K keys for L = 128K
    (1, 131072, 64, 128, "fp8", 2048, 8192, "prev"),
    (3, 131072, 64, 128, "fp8", 2048, 8192, "random"),
    (8, 131072, 64, 128, "bf16", 512, 8192, "prev"),
    (1, 70001, 20, 64, "f32", 100, 1000, "random"),    # 16 splits, ragged last split and tile
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c[0]}_L{c[1]}_H{c[2]}_D{c[3]}_{c[4]}_k{c[5]}_{c[7]}")
def test_decode_step_vs_oracle_and_unfused(lib, case):
    import torch
    T, L, H, D, dt, k, nh, smp = case
    say("decode", case)
    inp = _step_inputs(T, L, H, D, dt, k, nh, 0)
    d = to_dev(inp)
    if smp == "prev":
        prev = _step_inputs(T, L, H, D, dt, k, nh, -1, keys=_keys(inp))
        pd = to_dev(prev)
        sample = lib.score_select(pd["q"], d["k"], pd["w"], pd["pos"], k, sample=pd["sample"], q_scale=pd["q_scale"],
                                  k_scale=d["k_scale"]).reshape(-1)
    else:
        sample = d["sample"]
    idx, sc, st = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=sample, q_scale=d["q_scale"],
                                   k_scale=d["k_scale"], return_scores=True, return_stats=True)
    say("  candidates/query", st.cand_written / T, "max", st.max_cand_per_query, "overflow rows", st.overflow_rows)
    if smp == "prev":
        # k sample keys score >= the sample's minimum: the gate starts there, not at -inf
        assert st.overflow_rows == 0
    check_rows(inp, idx.cpu().numpy(), sc.cpu().numpy(), range(T), f"decode {case}")
    uidx, usc = lib.unfused_score_select(d["q"], d["k"], d["w"], d["pos"], k, q_scale=d["q_scale"],
                                         k_scale=d["k_scale"], return_scores=True)
    gi, gs = canon(idx.cpu().numpy(), sc.cpu().numpy())
    ui, us = canon(uidx.cpu().numpy(), usc.cpu().numpy())
    assert np.array_equal(gi, ui)
    assert np.array_equal(gs.view(np.uint32), us.view(np.uint32))   # bit-identical scores
    # sharing the threshold changes the work, never the result
    for shared in (1, -1):
        o = lib.Opts(shared_threshold=shared)
        idx2, st2 = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=sample, q_scale=d["q_scale"],
                                     k_scale=d["k_scale"], opts=o, return_stats=True)
        say(f"  shared={shared}: candidates/query", st2.cand_written / T, "overflow rows", st2.overflow_rows)
        assert np.array_equal(canon(idx2.cpu().numpy()), gi)


def test_decode_shared_threshold_small_splits(lib):
    """Sharing forced on with a handful of uneven splits and a tiny k: every split
    flushes and refreshes from the shared counts many times."""
    T, L, H, D, dt, k = 3, 5000, 20, 64, "f32", 64
    inp = indexer_inputs(T, L, H, D, dt, k, 300, drift=True, tag=62, n_sample=96)
    d = to_dev(inp)
    o = lib.Opts(shared_threshold=1, l_splits=7)
    idx, sc, st = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=d["sample"], opts=o,
                                   return_scores=True, return_stats=True)
    check_rows(inp, idx.cpu().numpy(), sc.cpu().numpy(), range(T), "shared 7 splits")
    o2 = lib.Opts(shared_threshold=-1, l_splits=7)
    idx2, st2 = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=d["sample"], opts=o2,
                                 return_stats=True)
    assert np.array_equal(canon(idx.cpu().numpy()), canon(idx2.cpu().numpy()))
    say("  shared", st.cand_written, "unshared", st2.cand_written)


VARIANTS = [
    # (T, H, D, dtype, k, opts) -- 2 or 4 waves per query, every tile geometry
    (1, 64, 64, "bf16", 128, {}),
    (1, 20, 64, "fp8", 150, {}),
    (2, 20, 64, "fp8", 200, {}),
    (3, 64, 128, "bf16", 64, {}),
    (1, 20, 128, "f32", 100, {}),                 # one 64-key block per tile: one wave per query
    (1, 64, 128, "fp8", 256, {"nbins": 1024}),    # four tile stages do not fit: one wave per query
    (4, 33, 128, "fp8", 300, {"l_splits": 5}),
    (1, 20, 64, "fp8", 3200, {}),                 # 9,600 sample slots: statistics by their own kernel
]


@pytest.mark.parametrize("case", VARIANTS, ids=lambda c: f"T{c[0]}_H{c[1]}_D{c[2]}_{c[3]}_k{c[4]}_{len(c[5])}")
def test_decode_waves_per_query_variants(lib, case):
    T, H, D, dt, k, ok = case
    L = 20011
    inp = indexer_inputs(T, L, H, D, dt, k, 600, drift=True, tag=65, n_sample=3 * k)
    d = to_dev(inp)
    idx, sc = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=d["sample"], q_scale=d["q_scale"],
                               k_scale=d["k_scale"], opts=lib.Opts(**ok), return_scores=True)
    check_rows(inp, idx.cpu().numpy(), sc.cpu().numpy(), range(T), f"variant {case}")
    uidx = lib.unfused_score_select(d["q"], d["k"], d["w"], d["pos"], k, q_scale=d["q_scale"], k_scale=d["k_scale"])
    assert np.array_equal(canon(idx.cpu().numpy()), canon(uidx.cpu().numpy()))


def _messy_sample(n, L, pos, seed):
    """n sample entries with repeats, empty (-1) slots, keys past the context
    and keys that only the later of the call's positions can see."""
    g = np.random.default_rng(seed)
    s = g.integers(0, L, size=n).astype(np.int32)
    h = n // 4
    s[:h] = s[h:2 * h]          # the second quarter's keys twice
    s[3::37] = -1
    s[5::41] = L + 3
    p = np.clip(np.asarray(pos, np.int64), 0, L - 1)
    m = len(s[7::43])
    s[7::43] = p.max() - g.integers(0, p.max() - p.min() + 1, size=m)
    return s


FRONT = [
    # (T, H, D, dtype, k, sample entries, positions): calls of at most 8
    # queries with at most 6,144 sample slots take the sample steps in one
    # launch; the neighbours keep the separate launches
    (1, 64, 128, "fp8", 512, 0, None),          # no sample: the library's evenly spaced keys
    (6, 64, 128, "fp8", 300, 6144, "mixed"),    # the largest such sample; unsorted, repeated, outside positions
    (8, 20, 64, "bf16", 200, 3000, None),
    (8, 20, 64, "bf16", 200, 6145, None),       # one slot more: separate launches
    (9, 20, 64, "fp8", 200, 3000, None),        # nine queries: separate launches
    (2, 64, 128, "f32", 128, 1000, None),       # fp32 rows of 128 in two head blocks: separate launches
    (3, 20, 128, "f32", 64, 0, "mixed3"),
]


@pytest.mark.parametrize("case", FRONT, ids=lambda c: f"T{c[0]}_H{c[1]}_D{c[2]}_{c[3]}_k{c[4]}_s{c[5]}_{c[6]}")
def test_sample_steps_in_one_launch(lib, case):
    """Exact against the oracle, bit-identical to the unfused path, and the same
    sets sorted through the overflow fallback, whichever sample path runs."""
    import torch
    T, H, D, dt, k, ns, pk = case
    L = 30011
    pos = {None: None,
           "mixed": np.array([L - 1, 100, L - 1, L + 20000, 15000, -1], np.int32),
           "mixed3": np.array([7, 29000, L + 9000], np.int32)}[pk]
    say("sample steps", case)
    inp = indexer_inputs(T, L, H, D, dt, k, 600, drift=True, tag=67, pos=pos)
    d = to_dev(inp)
    sample = torch.from_numpy(_messy_sample(ns, L, inp["pos"], 67)).cuda() if ns else None
    # a workspace full of 0x7f bytes (floats of 3.4e38): a score slot left
    # unwritten would raise the sample's threshold above the true one
    code = {"f32": 0, "bf16": 1, "fp8": 2}[dt]
    nb = lib.workspace_bytes(lib.KIND_SCORE_SELECT, T, H, D, L, k, ns, code)
    ws = torch.full((nb,), 0x7f, dtype=torch.uint8, device="cuda")
    idx, sc, st = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=sample, q_scale=d["q_scale"],
                                   k_scale=d["k_scale"], return_scores=True, return_stats=True, workspace=ws)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    say("  candidates/query", st.cand_written / T, "overflow rows", st.overflow_rows)
    check_rows(inp, idx, sc, range(T), f"sample steps {case}")
    # bytes written: candidates, sample scores, indices and scores.  The one
    # launch stores a whole score row per query (a score or NaN per sample
    # slot); the separate launches store every distinct in-range key's score
    # for every query.
    one_launch = T <= 8 and (ns if ns else min(3 * k, L, 16384)) <= 6144 and not (dt == "f32" and D == 128 and H > 32)
    if ns:
        keys = np.unique(sample.cpu().numpy())
        keys = keys[(keys >= 0) & (keys < L)]
    else:
        kmax = int(np.clip(inp["pos"], -1, L - 1).max()) + 1
        nw = min(min(3 * k, L, 16384), kmax)
        keys = (np.arange(nw, dtype=np.int64) * kmax) // nw
    slots = ns if ns else min(3 * k, L, 16384)
    n_scores = T * slots if one_launch else T * len(keys)
    if st.overflow_rows == 0:
        assert st.bytes_written == 8 * st.cand_written + 4 * n_scores + 8 * k * T
    uidx, usc = lib.unfused_score_select(d["q"], d["k"], d["w"], d["pos"], k, q_scale=d["q_scale"],
                                         k_scale=d["k_scale"], return_scores=True)
    gi, gs = canon(idx, sc)
    ui, us = canon(uidx.cpu().numpy(), usc.cpu().numpy())
    assert np.array_equal(gi, ui)
    assert np.array_equal(gs.view(np.uint32), us.view(np.uint32))
    o = lib.Opts(sorted_output=True, cand_capacity=1)
    sidx, ssc = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=sample, q_scale=d["q_scale"],
                                 k_scale=d["k_scale"], opts=o, return_scores=True)
    si, ss = canon(sidx.cpu().numpy(), ssc.cpu().numpy())
    assert np.array_equal(si, gi)
    assert np.array_equal(ss.view(np.uint32), gs.view(np.uint32))


def test_decode_chain_of_steps(lib):
    """Four speculative-decode steps of T = 4: each step's sample is the previous step's result.
    The same chain again with the results kept in a ring that every step samples whole and
    writes one slot of (the output overlaps the sample) gives the same sets."""
    import torch
    T, L, H, D, dt, k, nh = 4, 65536, 64, 128, "fp8", 1024, 4096
    first = _step_inputs(T, L, H, D, dt, k, nh, -4, tag=63)
    keys = _keys(first)
    ins = [first] + [_step_inputs(T, L, H, D, dt, k, nh, s, keys=keys, tag=63) for s in (-3, -2, -1)]
    ds = [to_dev(x) for x in ins]
    sample = ds[0]["sample"]
    plain = []
    for s, (inp, d) in enumerate(zip(ins, ds)):
        idx = lib.score_select(d["q"], ds[0]["k"], d["w"], d["pos"], k, sample=sample, q_scale=d["q_scale"],
                               k_scale=ds[0]["k_scale"])
        check_rows(inp, idx.cpu().numpy(), None, range(T), f"chain step {s}")
        plain.append(canon(idx.cpu().numpy()))
        sample = idx.reshape(-1)
    ring = torch.full((2, T, k), -1, dtype=torch.int32, device="cuda")
    for s, d in enumerate(ds):
        smp = ds[0]["sample"] if s == 0 else ring
        out = lib.score_select(d["q"], ds[0]["k"], d["w"], d["pos"], k, sample=smp.reshape(-1),
                               q_scale=d["q_scale"], k_scale=ds[0]["k_scale"], out=ring[s % 2])
        assert out.data_ptr() == ring[s % 2].data_ptr()
        assert np.array_equal(canon(out.cpu().numpy()), plain[s]), f"ring step {s}"


def test_decode_graph_capture_replays(lib):
    """Three decode steps captured as one HIP graph: every replay, with eager work
    and synchronisations in between, equals the eager chain."""
    import torch
    T, L, H, D, dt, k, nh = 2, 65536, 64, 128, "fp8", 512, 4096
    ins = [_step_inputs(T, L, H, D, dt, k, nh, -3, tag=64)]
    keys = _keys(ins[0])
    ins += [_step_inputs(T, L, H, D, dt, k, nh, s, keys=keys, tag=64) for s in (-2, -1)]
    ds = [to_dev(x) for x in ins]
    kk, ks = ds[0]["k"], ds[0]["k_scale"]
    ws = torch.empty(lib.workspace_bytes(lib.KIND_SCORE_SELECT, T, H, D, L, k, 6144, 2), dtype=torch.uint8,
                     device="cuda")

    def chain(sample):
        outs = []
        for d in ds:
            sample = lib.score_select(d["q"], kk, d["w"], d["pos"], k, sample=sample.reshape(-1),
                                      q_scale=d["q_scale"], k_scale=ks, workspace=ws)
            outs.append(sample)
        return outs

    s0 = ds[0]["sample"].clone()
    eager = [o.clone() for o in chain(s0)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain(s0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gouts = chain(s0)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(gouts, eager):   # row order follows atomic order: compare the sets
            assert np.array_equal(canon(a.cpu().numpy()), canon(b.cpu().numpy())), f"replay {rep}"
        # eager work on the same workspace between replays
        lib.score_select(ds[1]["q"], kk, ds[1]["w"], ds[1]["pos"], k, sample=s0, q_scale=ds[1]["q_scale"],
                         k_scale=ks, workspace=ws)
        torch.cuda.synchronize()
    check_rows(ins[2], gouts[2].cpu().numpy(), None, range(T), "graph replay, last step")


def test_keys_past_two_gib_uniform_tile_addresses(lib):
    """A 2.1 GB key array, so that some tile base addresses have bit 31 of their
    low word set and others not: the tile loads that take a wave-uniform base
    in scalar registers must give the same result as the unfused path (which
    addresses every lane separately)."""
    import torch
    L, H, D, k = (1 << 24) + 77, 64, 128, 512
    g = torch.Generator(device="cuda")
    g.manual_seed(81)
    codes = torch.randint(0, 126, (L, D), generator=g, device="cuda", dtype=torch.uint8)   # finite e4m3 codes
    codes |= (torch.randint(0, 2, (L, D), generator=g, device="cuda", dtype=torch.uint8) << 7)
    kk = codes.view(torch.float8_e4m3fn)
    ks = torch.rand(L, generator=g, device="cuda") + 0.5
    q = torch.randint(0, 126, (2, H, D), generator=g, device="cuda", dtype=torch.uint8).view(torch.float8_e4m3fn)
    qs = torch.rand(2, generator=g, device="cuda") + 0.5
    w = torch.rand(2, H, generator=g, device="cuda")
    for T in (1, 2):   # four and two waves per query
        pos = torch.tensor([L - 1, L - 2][:T], dtype=torch.int32, device="cuda")
        idx = lib.score_select(q[:T].contiguous(), kk, w[:T].contiguous(), pos, k, q_scale=qs[:T].contiguous(),
                               k_scale=ks)
        uidx = lib.unfused_score_select(q[:T].contiguous(), kk, w[:T].contiguous(), pos, k,
                                        q_scale=qs[:T].contiguous(), k_scale=ks)
        assert np.array_equal(canon(idx.cpu().numpy()), canon(uidx.cpu().numpy())), T
    say("2.1 GB keys: fused == unfused")
