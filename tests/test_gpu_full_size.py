"""The prefill workloads at full size on the GPU, launched as the benchmark
launches them: 64 evenly spaced rows and the edge rows against the CPU oracle, every row against the
unfused baseline (bit-identical sets and scores), structural checks on all
rows, and the bytes written per query."""
import numpy as np
import pytest

from tests.gpu_util import canon, check_rows, say, spaced_rows, to_dev
from workloads import indexer_workload

pytestmark = pytest.mark.gpu


def _prev_sample(lib, inp, d):
    """The previous chunk (bootstrapped with a seeded random sample) through the
    library, then its top-3k by selection count: the sample of this chunk."""
    import torch
    prev = dict(inp["prev"])
    prev.update(k=inp["k"], k_scale=inp["k_scale"])
    pd = to_dev(prev)
    pidx = lib.score_select(pd["q"], d["k"], pd["w"], pd["pos"], inp["topk"], sample=pd["sample"],
                            q_scale=pd["q_scale"], k_scale=d["k_scale"])
    return lib.next_sample(pidx, inp["L"], 3 * inp["topk"]), torch


@pytest.mark.parametrize("name", ["prefill-64k-bf16", "prefill-256k-bf16", "prefill-1m-fp8"])
def test_full_size_prefill(lib, name):
    import torch
    say(f"{name}: generating")
    inp = indexer_workload(name, with_prev=True)
    d = to_dev(inp)
    sample, _ = _prev_sample(lib, inp, d)
    T, L, k = inp["T"], inp["L"], inp["topk"]
    say(f"{name}: fused")
    idx, sc, st = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=sample, q_scale=d["q_scale"],
                                   k_scale=d["k_scale"], return_scores=True, return_stats=True)
    idx_h, sc_h = idx.cpu().numpy(), sc.cpu().numpy()
    # structure on every row: k distinct causal keys
    s = np.sort(idx_h, axis=1)
    assert np.all(s >= 0) and np.all(np.diff(s, axis=1) > 0)
    assert np.all(s[:, -1] <= inp["pos"])
    assert st.overflow_rows == 0
    # bytes written against the full score matrix (4 L bytes per query): the
    # filter's own write-back (candidates and outputs) at least 5x below it on
    # every chunk, and everything the call writes (sample scores included) at
    # least 5x below it on the 1M-context chunk, where the target is stated
    bytes_q = st.bytes_written / T
    filt_q = (8.0 * st.cand_written + 8.0 * T * k) / T
    say(f"{name}: candidates/query {st.cand_written / T:.0f}, bytes/query {bytes_q:.0f} "
        f"(candidates and outputs {filt_q:.0f}) vs {4 * L}")
    assert st.bytes_written >= 8 * st.cand_written + 4 * T * k * 2
    assert filt_q * 5 <= 4 * L
    if L == 1 << 20:
        assert bytes_q * 5 <= 4 * L
    # 64 evenly spaced rows (and the edges) against the oracle
    rows = spaced_rows(T, 64)
    say(f"{name}: {len(rows)} oracle rows")
    check_rows(inp, idx_h, sc_h, rows, name)
    # every row against the unfused baseline
    say(f"{name}: unfused")
    uidx, usc = lib.unfused_score_select(d["q"], d["k"], d["w"], d["pos"], k, q_scale=d["q_scale"],
                                         k_scale=d["k_scale"], return_scores=True)
    a, asc = canon(idx_h, sc_h)
    b, bsc = canon(uidx.cpu().numpy(), usc.cpu().numpy())
    del uidx, usc
    torch.cuda.empty_cache()
    assert np.array_equal(a, b)
    assert np.array_equal(asc.view(np.uint32), bsc.view(np.uint32))


@pytest.mark.parametrize("T", [1, 8], ids=["decode", "specdecode"])
def test_full_size_decode(lib, T):
    """Decode steps over the 1M-context fp8 keys, launched as the benchmark
    launches them (the key range split over every CU, shared thresholds): the
    newest T queries of the chunk, a bootstrap step on a random sample, then a
    step sampled from its result.  Every row against the oracle, and
    bit-identical to the unfused baseline."""
    from workloads import random_sample
    import torch
    say(f"decode T={T}: generating")
    full = indexer_workload("prefill-1m-fp8")
    inp = dict(full)
    for f in ("q", "q_scale", "w", "pos"):
        inp[f] = np.ascontiguousarray(full[f][-T:])
    inp["T"] = T
    del full
    d = to_dev(inp, sample=random_sample(3 * inp["topk"], inp["L"], tag=91))
    k = inp["topk"]
    say(f"decode T={T}: bootstrap step")
    first = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=d["sample"], q_scale=d["q_scale"],
                             k_scale=d["k_scale"])
    say(f"decode T={T}: sampled step")
    idx, sc, st = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=first.flatten(),
                                   q_scale=d["q_scale"], k_scale=d["k_scale"], return_scores=True,
                                   return_stats=True)
    assert st.overflow_rows == 0
    idx_h, sc_h = idx.cpu().numpy(), sc.cpu().numpy()
    check_rows(inp, idx_h, sc_h, range(T), f"decode T={T}")
    uidx, usc = lib.unfused_score_select(d["q"], d["k"], d["w"], d["pos"], k, q_scale=d["q_scale"],
                                         k_scale=d["k_scale"], return_scores=True)
    a, asc = canon(idx_h, sc_h)
    b, bsc = canon(uidx.cpu().numpy(), usc.cpu().numpy())
    del uidx, usc
    torch.cuda.empty_cache()
    assert np.array_equal(a, b)
    assert np.array_equal(asc.view(np.uint32), bsc.view(np.uint32))
