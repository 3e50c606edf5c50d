"""The allocation-free entry point (litetopk_score_select_static) against
litetopk_score_select, through the C ABI: two calls in a row on the shared
static workspace, the second smaller, each bit-identical (indices and
scores) to the workspace-argument call on the same inputs."""
import numpy as np
import pytest

from tests.gpu_util import canon, check_rows, say, to_dev
from workloads import indexer_inputs

pytestmark = pytest.mark.gpu


def _both(lib, inp, sample, opts=None):
    d = to_dev(inp, sample=sample)
    k = inp["topk"]
    kw = dict(sample=d["sample"], q_scale=d["q_scale"], k_scale=d["k_scale"], opts=opts, return_scores=True,
              return_stats=True)
    i0, s0, st0 = lib.score_select(d["q"], d["k"], d["w"], d["pos"], k, **kw)
    i1, s1, st1 = lib.score_select_static(d["q"], d["k"], d["w"], d["pos"], k, **kw)
    return (i0.cpu().numpy(), s0.cpu().numpy(), st0), (i1.cpu().numpy(), s1.cpu().numpy(), st1)


def test_static_workspace_matches_workspace_call(lib):
    import torch
    cases = [
        # a speculative-decode step over a long context (key splits share thresholds), then a smaller call
        indexer_inputs(8, 131072, 64, 128, "fp8", 2048, 8192, drift=True, tag=91, n_sample=6144),
        indexer_inputs(3, 70001, 20, 64, "bf16", 100, 1000, drift=True, tag=92, n_sample=300),
    ]
    for inp in cases:
        say("static workspace", inp["T"], inp["L"], inp["dtype"])
        (i0, s0, st0), (i1, s1, st1) = _both(lib, inp, inp["sample"])
        a, asc = canon(i0, s0)
        b, bsc = canon(i1, s1)
        assert np.array_equal(a, b) and np.array_equal(asc.view(np.uint32), bsc.view(np.uint32))
        # (candidate counts may differ: with shared thresholds the work depends
        # on the timing of the splits' refreshes, the result does not)
        assert st0.overflow_rows == st1.overflow_rows == 0
        check_rows(inp, i1, s1, range(inp["T"]), "static")
    torch.cuda.synchronize()


def test_static_workspace_rejects_oversized_calls(lib):
    """A call whose workspace exceeds the static array is refused before any launch."""
    import indexer_topk_long_amd as ltk
    inp = indexer_inputs(1024, 200000, 64, 128, "fp8", 2048, 1000, tag=93, n_sample=6144)
    d = to_dev(inp)
    assert ltk.workspace_bytes(0, 1024, 64, 128, 200000, 2048, 6144, 2) > 96 << 20
    with pytest.raises(ltk.LtkError) as e:
        lib.score_select_static(d["q"], d["k"], d["w"], d["pos"], 2048, sample=d["sample"], q_scale=d["q_scale"],
                                k_scale=d["k_scale"])
    assert e.value.status == -3
