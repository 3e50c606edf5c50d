"""Chunked prefill driver (LiteTopK pages, "Sampling": each chunk's sample is the
previous chunk's top-3k): every chunk's result against the oracle on sampled
rows, and bit-identical to the unfused path on all rows, whatever sample was
carried in."""
import numpy as np
import pytest

from tests.gpu_util import canon, check_rows, say, to_dev
from workloads import indexer_inputs

pytestmark = pytest.mark.gpu


CASES = [
    # (L, chunk, H, D, dtype, topk, n_hot) -- a ragged last chunk, padded heads
    (3000, 512, 20, 64, "bf16", 64, 150),
    (2048, 512, 64, 128, "fp8", 100, 200),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"L{c[0]}_chunk{c[1]}_H{c[2]}_D{c[3]}_{c[4]}_k{c[5]}")
def test_prefill_chunked_vs_oracle_and_unfused(lib, case):
    import torch
    L, chunk, H, D, dt, k, nh = case
    say("prefill", case)
    # every position of the context is a query; the chunks cover them in order
    inp = indexer_inputs(L, L, H, D, dt, k, nh, drift=True, tag=51, pos=np.arange(L), n_sample=3 * k)
    d = to_dev(inp)
    res = lib.prefill_chunked((d["q"], d["w"], d["q_scale"]), d["k"], k, L, chunk=chunk, n_sample=3 * k,
                              k_scale=d["k_scale"], keep_outputs=True)
    ch = res["chunks"]
    assert len(ch) == (L + chunk - 1) // chunk
    assert [r["queries"] for r in ch] == [min(chunk, L - c0) for c0 in range(0, L, chunk)]
    assert ch[0]["sample_hit_rate"] is None and all(r["sample_hit_rate"] is not None for r in ch[1:])
    assert all(r["overflow_rows"] == 0 for r in ch)
    idx = torch.cat(res["outputs"]).cpu().numpy()
    assert idx.shape == (L, k)
    rows = np.unique(np.concatenate([np.arange(0, L, 41), np.arange(chunk - 2, L, chunk), [L - 1]]))
    check_rows(inp, idx, None, rows, f"prefill {case}")
    uidx = lib.unfused_score_select(d["q"], d["k"], d["w"], d["pos"], k, q_scale=d["q_scale"],
                                    k_scale=d["k_scale"]).cpu().numpy()
    assert np.array_equal(canon(idx), canon(uidx))


def test_prefill_without_diagnostics_same_sets(lib):
    """The driver enqueued back to back (no per-chunk events, statistics or
    synchronisation) selects the same key sets, chunk by chunk, and counts the
    same causal pairs."""
    L, chunk, H, D, dt, k, nh = 2048, 512, 64, 128, "fp8", 100, 200
    inp = indexer_inputs(L, L, H, D, dt, k, nh, drift=True, tag=52, pos=np.arange(L), n_sample=3 * k)
    d = to_dev(inp)
    args = ((d["q"], d["w"], d["q_scale"]), d["k"], k, L)
    kw = dict(chunk=chunk, n_sample=3 * k, k_scale=d["k_scale"], keep_outputs=True)
    a = lib.prefill_chunked(*args, **kw)
    b = lib.prefill_chunked(*args, diagnostics=False, **kw)
    assert [r["pairs"] for r in a["chunks"]] == [r["pairs"] for r in b["chunks"]]
    assert [r["queries"] for r in a["chunks"]] == [r["queries"] for r in b["chunks"]]
    for x, y in zip(a["outputs"], b["outputs"]):
        assert np.array_equal(canon(x.cpu().numpy()), canon(y.cpu().numpy()))

