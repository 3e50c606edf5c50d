"""Inputs with exact score ties at the k-th boundary, for the tie-breaking
parity tests (lower key index wins: the reading the pages leave open and the
oracle implements by a full lexicographic sort).

Every key row is a bit-for-bit copy of one of a few source rows (its fp8
per-key scale included), so each query's scores take only a few distinct
values, each shared by many keys spread over every tile and key split.  With
k not a multiple of the group sizes, the k-th score falls inside a group of
exact ties, and only the lowest indices of that group belong to the result.

The checks below hold on the CPU, so a GPU parity test built on these inputs
compares index sets exactly, with no acceptance band: a distinct score value
never lies within fp32 rounding of the k-th score.
"""
from __future__ import annotations

import numpy as np

from workloads import indexer_inputs

GAP = 1e-5   # distinct values are at least GAP * max|I| away from the k-th score


def tied_indexer_inputs(T, L, H, D, dtype, topk, n_src, tag, pos=None):
    """Indexer inputs whose L keys are copies of n_src source rows, assigned
    at random (seeded) positions."""
    inp = indexer_inputs(T, L, H, D, dtype, topk, max(L // 8, 1), drift=True, tag=tag, pos=pos,
                         n_sample=3 * topk)
    g = np.random.default_rng(np.random.SeedSequence([20260713, tag, 99]))
    src = g.choice(L, size=n_src, replace=False)
    which = src[g.integers(0, n_src, size=L)]
    which[src] = src                       # the source rows keep themselves
    inp["k"] = np.ascontiguousarray(inp["k"][which])
    if inp.get("k_scale") is not None:
        inp["k_scale"] = np.ascontiguousarray(inp["k_scale"][which])
    inp["src_of_key"] = which
    return inp


def tied_retrieval_inputs(T, N, D, topk, n_src, tag):
    """bf16 unit database rows that are copies of n_src source rows; queries
    are perturbed source rows.  Returns (q bits [T, D], db bits [N, D], sample)."""
    import torch
    g = np.random.default_rng(np.random.SeedSequence([20260713, tag, 98]))
    base = g.standard_normal((n_src, D)).astype(np.float32)
    base /= np.linalg.norm(base, axis=1, keepdims=True)
    which = g.integers(0, n_src, size=N)
    db = base[which]
    q = base[g.integers(0, n_src, size=T)] + 0.6 * g.standard_normal((T, D)).astype(np.float32) / np.sqrt(D)
    q /= np.linalg.norm(q, axis=1, keepdims=True)

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    sample = np.sort(g.choice(N, size=min(3 * topk, N), replace=False)).astype(np.int32)
    return bits(q), bits(db), sample


def boundary_stats(s, k):
    """(split tie at the k-th score?, smallest gap from a distinct value to the
    k-th score relative to max|I|) for one row of fp64 scores s."""
    if len(s) <= k:
        return False, np.inf
    srt = np.sort(s)[::-1]
    vk = srt[k - 1]
    split = (s > vk).sum() < k < (s >= vk).sum()
    other = s[s != vk]
    gap = np.abs(other - vk).min() / np.abs(s).max() if len(other) else np.inf
    return bool(split), float(gap)
