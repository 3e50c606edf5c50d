"""The seeded generators: shapes, formats, determinism and workload structure."""
import numpy as np
import pytest

from oracle import decode, indexer_row_scores, oracle_indexer
from workloads import WORKLOADS, indexer_inputs, indexer_keys, indexer_workload, retrieval_inputs, to_storage


def test_tiny_workload_shapes():
    inp = indexer_workload("tiny-4k-fp32")
    c = WORKLOADS["tiny-4k-fp32"]
    assert inp["q"].shape == (c["T"], c["H"], c["D"]) and inp["q"].dtype == np.float32
    assert inp["k"].shape == (c["L"], c["D"])
    assert inp["w"].shape == (c["T"], c["H"]) and inp["w"].min() >= 0.5 and inp["w"].max() <= 1.0
    assert inp["pos"].tolist() == list(range(4032, 4096))
    assert len(inp["hot"]) == 128 and len(np.unique(inp["hot"])) == 128
    assert len(inp["sample"]) == 768 and len(np.unique(inp["sample"])) == 768
    prev = indexer_workload("tiny-4k-fp32", chunk=-1)
    assert prev["pos"].tolist() == list(range(3968, 4032))
    assert np.array_equal(prev["k"], inp["k"]) and not np.array_equal(prev["q"], inp["q"])


def test_determinism():
    a = indexer_inputs(8, 300, 4, 32, "bf16", 10, 20, tag=5)
    b = indexer_inputs(8, 300, 4, 32, "bf16", 10, 20, tag=5)
    c = indexer_inputs(8, 300, 4, 32, "bf16", 10, 20, tag=6)
    for key in ("q", "k", "w", "pos"):
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["k"], c["k"])


@pytest.mark.parametrize("dtype,rel", [("bf16", 2.0 ** -8), ("fp8", 2.0 ** -4)])
def test_rounding_error_bound(dtype, rel):
    """Round-to-nearest into bf16 (8 significant bits) / e4m3fn (4 bits, scaled to amax/448)."""
    g = np.random.default_rng(0)
    x = g.standard_normal((50, 64)).astype(np.float32)
    raw, scale = to_storage(x, dtype, axes=(1,))
    y = decode(raw, dtype, scale)
    err = np.abs(y - x)
    if dtype == "fp8":
        sub = scale.astype(np.float64)[:, None] * 2.0 ** -10       # half the smallest subnormal step
        assert np.all(err <= rel * np.abs(x) + sub)
        assert np.all(np.abs(raw.astype(np.int32) & 0x7F) <= 0x7E)   # never NaN, never above 448
        assert np.allclose(np.abs(y).max(1), np.abs(x).max(1), rtol=2 ** -4)
    else:
        assert np.all(err <= rel * np.abs(x))


def test_fp8_scales_per_token():
    inp = indexer_inputs(6, 200, 4, 32, "fp8", 10, 10, tag=8)
    assert inp["q_scale"].shape == (6,) and inp["k_scale"].shape == (200,)
    q = decode(inp["q"], "fp8", inp["q_scale"])
    assert np.all(np.abs(q).reshape(6, -1).max(1) <= 448 * inp["q_scale"] * (1 + 1e-6))


def test_score_concentration_and_chunk_overlap():
    """Most scores sit in a narrow band far below the top (the curse-of-dimensionality
    concentration the method exploits); adjacent chunks share top sets."""
    inp = indexer_workload("tiny-4k-fp32")
    v, s = indexer_row_scores(inp, 0)
    kth = np.sort(s)[-inp["topk"]]
    assert np.percentile(s, 90) < kth < s.max()
    assert (np.percentile(s, 75) - np.percentile(s, 25)) < 0.25 * (s.max() - np.percentile(s, 25))
    cur, _ = oracle_indexer(inp, rows=[0, 63])
    prev, _ = oracle_indexer(indexer_workload("tiny-4k-fp32", chunk=-1))
    cnt = np.bincount(prev[prev >= 0].ravel(), minlength=inp["L"])
    top3k = np.lexsort((np.arange(inp["L"]), -cnt))[: 3 * inp["topk"]]
    for row in cur:                        # the previous chunk's top-3k covers most of this top-k
        assert np.isin(row, top3k).mean() > 0.6
    hot = set(inp["hot"].tolist())
    assert np.mean([i in hot for i in cur[0]]) > 10 * len(hot) / inp["L"]


def test_retrieval_generator_small():
    r = retrieval_inputs(T=16, N=5000, D=64, topk=10, n_centres=20, sigma=0.3, n_sample=30, block=1000)
    db = r["db"].float().numpy()
    assert r["db"].shape == (5000, 64) and str(r["db"].dtype) == "torch.bfloat16"
    assert np.allclose(np.linalg.norm(db, axis=1), 1.0, atol=1e-2)
    q = decode(r["q"], "bf16")
    assert np.allclose(np.linalg.norm(q, axis=1), 1.0, atol=1e-2)
    assert len(np.unique(r["sample"])) == 30
    r2 = retrieval_inputs(T=16, N=5000, D=64, topk=10, n_centres=20, sigma=0.3, n_sample=30, block=1000)
    assert (r2["db"] == r["db"]).all()


def test_indexer_keys_match_the_workload():
    k, ks = indexer_keys("tiny-4k-fp32")
    full = indexer_workload("tiny-4k-fp32")
    assert np.array_equal(k, full["k"]) and ks is None
    assert all(WORKLOADS[c["keys"]]["kind"] == "indexer" for c in WORKLOADS.values() if c["kind"] == "decode")
