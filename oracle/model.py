"""Step-by-step CPU model of LiteTopK's Sample -> Filter -> Select -- TEST INFRASTRUCTURE ONLY.

Where ``oracle.py`` is the plain definition, this module walks the method's
three phases in the order the LiteTopK pages give them ("Methodology"), in
fp64, one query row at a time, so that the method's exactness claim can be
checked on the CPU against the plain definition for any sample, bin count,
refresh period, split count and buffer capacity:

1. Sample ("Sampling"): score the sample keys (the previous chunk's top-3k,
   reused), take their range [s_min, s_max], split it into ``nbins``
   equal-width bins, and set the initial threshold bin to the bin holding the
   sample's k-th largest score.
2. Filter ("Filtering"): for every key, in tiles, map the score to a bin with
   the affine map B = (I - s_min) * delta (delta = nbins / (s_max - s_min));
   keep the key only if its bin is >= the current threshold bin; kept keys go
   to a small local list that is appended to the candidate buffer in batches
   of ``flush`` entries; every ``refresh_every`` batches the threshold bin is
   recomputed by accumulating the histogram of kept keys from the top bin
   down (a plain overwrite that can only raise it).
3. Select ("Selection"): keys in bins strictly above the final threshold bin
   go straight to the output; a standard top-k runs only inside that bin.

Readings where the pages are silent (stated again in the design notes):
causal boundary inclusive; sample de-duplicated and restricted to valid keys;
the main histogram starts empty (seeding it with the sample's counts while
scanning the sample keys again would count them twice -- ``seed_hist=True``
reproduces that mistake for the tests); scores outside [s_min, s_max] are
clamped into the first/last bin; a degenerate range is widened; fewer than k
valid sample keys give threshold bin 0; the final threshold bin is the recount
of the candidates' bins from the top; a buffer that overflows its capacity
falls back to the plain top-k of the row.
"""
from __future__ import annotations

import numpy as np

from .oracle import topk_row


def bin_map(I, s_min: float, delta: float, nbins: int):
    """Equal-width bin of a score: clamp(floor((I - s_min) * delta), 0, nbins - 1)."""
    B = (np.asarray(I, dtype=np.float64) - s_min) * delta
    return np.clip(np.floor(B), 0, nbins - 1).astype(np.int64)


def threshold_from_hist(hist: np.ndarray, k: int) -> int:
    """Largest bin b whose count of entries in bins >= b reaches k (0 if none)."""
    acc = 0
    for b in range(len(hist) - 1, -1, -1):
        acc += int(hist[b])
        if acc >= k:
            return b
    return 0


def sample_range(sample_scores: np.ndarray, nbins: int):
    """(s_min, s_max, delta) of the sample scores; degenerate ranges are widened."""
    if len(sample_scores) == 0:
        s_min, s_max = 0.0, 1.0
    else:
        s_min, s_max = float(sample_scores.min()), float(sample_scores.max())
    width = s_max - s_min
    floor_w = 1e-6 * max(1.0, abs(s_max))
    if not width >= floor_w:
        width = floor_w
    return s_min, s_min + width, nbins / width


def sfs_row(keys_idx: np.ndarray, scores: np.ndarray, sample: np.ndarray, k: int, nbins: int = 256,
            tile: int = 32, flush: int = 64, refresh_every: int = 1, capacity: int | None = None,
            n_splits: int = 1, seed_hist: bool = False, trace: dict | None = None):
    """Sample-Filter-Select on one query row.

    keys_idx / scores: the valid keys of the row (increasing index) and their
    fp64 scores.  sample: raw sample indices (may hold duplicates, invalid or
    non-causal entries).  refresh_every <= 0 disables the refresh.  Returns
    (idx int32 [k], scores fp64 [k]) exactly as ``topk_row`` would for the
    same row when the method is exact.
    """
    n = len(keys_idx)

    # --- 1. Sample -------------------------------------------------------
    su = np.unique(np.asarray(sample, dtype=np.int64))       # de-duplicate
    at = np.searchsorted(keys_idx, su)
    ok = at < n
    ok[ok] = keys_idx[at[ok]] == su[ok]                      # keep valid (causal, in-range) keys only
    ss = scores[at[ok]]
    s_min, s_max, delta = sample_range(ss, nbins)
    sample_bins = bin_map(ss, s_min, delta, nbins)
    shist = np.bincount(sample_bins, minlength=nbins)
    thr0 = threshold_from_hist(shist, k) if len(ss) >= k else 0

    # --- 2. Filter -------------------------------------------------------
    bins = bin_map(scores, s_min, delta, nbins)
    cand = []            # the candidate buffer (index, score)
    tail = 0             # buffer tail: counts every appended entry, kept or not
    cap = capacity if capacity is not None else n + 1
    bounds = np.linspace(0, n, n_splits + 1).astype(np.int64)
    for sp in range(n_splits):
        hist = shist.copy() if seed_hist else np.zeros(nbins, dtype=np.int64)
        thr = thr0
        local = []
        flushes = 0
        for t0 in range(bounds[sp], bounds[sp + 1], tile):
            t1 = min(t0 + tile, bounds[sp + 1])
            for i in range(t0, t1):          # one tile: gate against the threshold read at tile start
                if bins[i] >= thr:
                    local.append(i)
                    hist[bins[i]] += 1
            while len(local) >= flush:       # batched write-back
                batch, local = local[:flush], local[flush:]
                for i in batch:
                    if tail < cap:
                        cand.append(i)
                    tail += 1
                flushes += 1
                if refresh_every > 0 and flushes % refresh_every == 0:
                    thr = max(thr, threshold_from_hist(hist, k))   # top-down recount
        for i in local:                      # final partial batch
            if tail < cap:
                cand.append(i)
            tail += 1
        if trace is not None:
            trace.setdefault("thr_final", []).append(thr)
    if trace is not None:
        trace.update(s_min=s_min, s_max=s_max, delta=delta, thr0=thr0, n_cand=tail,
                     overflow=tail > cap)

    # --- 3. Select -------------------------------------------------------
    if tail > cap:                           # overflow: exact fallback on the whole row
        return topk_row(scores, keys_idx, k)
    cand = np.array(sorted(cand), dtype=np.int64)
    if len(cand) <= k:                       # only when the row has <= k valid keys
        return topk_row(scores[cand], keys_idx[cand], k)
    cbins = bins[cand]
    chist = np.bincount(cbins, minlength=nbins)
    b_star = threshold_from_hist(chist, k)   # final threshold bin
    above = cand[cbins > b_star]
    inbin = cand[cbins == b_star]
    r = k - len(above)
    sel_i, _ = topk_row(scores[inbin], keys_idx[inbin], r)   # standard top-k inside the bin
    out_idx = np.concatenate([keys_idx[above], sel_i.astype(np.int64)])
    out_sc = np.concatenate([scores[above], scores[np.searchsorted(keys_idx, sel_i)]])
    order = np.lexsort((out_idx, -out_sc))
    res_i = np.full(k, -1, dtype=np.int32)
    res_s = np.full(k, np.nan)
    res_i[: len(order)] = out_idx[order]
    res_s[: len(order)] = out_sc[order]
    if trace is not None:
        trace.update(b_star=b_star, n_above=len(above), n_inbin=len(inbin))
    return res_i, res_s


def expected_candidates(scores: np.ndarray, s_min: float, delta: float, nbins: int, thr: int) -> int:
    """Number of keys whose bin is >= thr (what a static-threshold scan keeps)."""
    return int((bin_map(scores, s_min, delta, nbins) >= thr).sum())


__all__ = ["bin_map", "threshold_from_hist", "sample_range", "sfs_row", "expected_candidates"]
