"""Helpers of the GPU parity tests: device copies of generator inputs and the
acceptance rule comparing a GPU result with the CPU oracle.

Acceptance (per row t, oracle scores I in fp64): the GPU set G holds
min(k, |V_t|) distinct valid keys and -1 elsewhere; every key in the
symmetric difference of G and the oracle set A scores within
eps_t = 1e-3 * max_s |I[t, s]| of the oracle's k-th score; every returned
score is within tol * max(|I[t, s]|, eps_t) of the oracle's (tol = 2e-3 for
fp32/bf16 inputs, 2e-2 for fp8).
"""
from __future__ import annotations

import sys

import numpy as np

TOL = {"f32": 2e-3, "bf16": 2e-3, "fp8": 2e-2}
BAND = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(inp: dict, sample=None):
    """Device tensors (q, k, w, pos, q_scale, k_scale, sample) of an indexer input dict."""
    import torch
    dt = inp["dtype"]

    def raw(x):
        if dt == "f32":
            return torch.from_numpy(np.ascontiguousarray(x)).cuda()
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x)).cuda().view(torch.float8_e4m3fn)

    q, k = raw(inp["q"]), raw(inp["k"])
    w = torch.from_numpy(inp["w"]).cuda()
    pos = torch.from_numpy(inp["pos"].astype(np.int32)).cuda()
    qs = ks = None
    if dt == "fp8":
        qs = torch.from_numpy(inp["q_scale"]).cuda()
        ks = torch.from_numpy(inp["k_scale"]).cuda()
    smp = inp.get("sample") if sample is None else sample
    s = None if smp is None else torch.from_numpy(np.asarray(smp, dtype=np.int32)).cuda()
    return dict(q=q, k=k, w=w, pos=pos, q_scale=qs, k_scale=ks, sample=s)


def check_row(g_idx, g_sc, v, s, k, dtype, where=""):
    """Check one GPU row (idx, scores or None) against the oracle row scores s over keys v."""
    from oracle import topk_row
    a_idx, a_sc = topk_row(s, v, k)
    n = min(k, len(v))
    g_idx = np.asarray(g_idx)
    sel = g_idx[g_idx >= 0]
    assert len(sel) == n, f"{where}: {len(sel)} results, expected {n}"
    assert np.all(g_idx[g_idx < 0] == -1)
    assert len(np.unique(sel)) == n, f"{where}: duplicate indices"
    if n == 0:
        return
    assert sel.min() >= v[0] and sel.max() <= v[-1], f"{where}: index outside the causal range"
    eps = BAND * np.abs(s).max()
    A = set(a_idx[:n].tolist())
    G = set(sel.tolist())
    diff = sorted(A ^ G)
    if diff:
        kth = a_sc[n - 1]
        off = np.abs(s[np.searchsorted(v, diff)] - kth)
        assert np.all(off <= eps), f"{where}: {len(diff)} keys differ, worst {off.max():.3g} from the k-th (band {eps:.3g})"
    if g_sc is not None:
        g_sc = np.asarray(g_sc, dtype=np.float64)
        m = g_idx >= 0
        ref = s[np.searchsorted(v, g_idx[m])]
        tol = TOL[dtype] * np.maximum(np.abs(ref), eps)
        err = np.abs(g_sc[m] - ref)
        assert np.all(err <= tol), f"{where}: score error {err.max():.3g} > tol"
        assert np.all(np.isnan(g_sc[~m]))
    return len(diff)


def check_rows(inp, g_idx, g_sc, rows, where=""):
    """Acceptance rule on the given query rows (oracle scored on the CPU)."""
    from oracle import indexer_row_scores, key_table
    keys = key_table(inp)
    swaps = 0
    for t in rows:
        v, s = indexer_row_scores(inp, int(t), keys)
        swaps += check_row(g_idx[t], None if g_sc is None else g_sc[t], v, s, inp["topk"], inp["dtype"],
                           f"{where} row {t}") or 0
    return swaps


def oracle_prev_chunk_sample(inp: dict) -> np.ndarray:
    """The sample of an indexer chunk as the pages define it: the previous
    chunk's top-k selections (from the oracle), ranked by how many of its rows
    selected each key, the first 3k ("Sampling")."""
    from oracle import next_sample, oracle_indexer
    pidx = oracle_indexer(inp["prev"], with_scores=False)
    return next_sample(pidx, inp["L"], 3 * inp["topk"])


def spaced_rows(T: int, n: int = 64) -> list:
    """n evenly spaced query rows plus the first two and the last two."""
    return sorted(set(np.linspace(0, T - 1, n).round().astype(int).tolist() + [0, 1, T - 2, T - 1]))


def canon(idx, sc=None):
    """Rows as sorted (index) arrays, for bit-exact set comparisons between GPU paths."""
    o = np.sort(np.asarray(idx), axis=1)
    if sc is None:
        return o
    order = np.argsort(np.asarray(idx), axis=1)
    return o, np.take_along_axis(np.asarray(sc), order, axis=1)
