"""Chunk-to-chunk carry of the sample (LiteTopK pages, "Sampling": the
previous chunk's top-3k tokens serve as the next chunk's sample)."""
from __future__ import annotations

import ctypes

from ._binding import KIND_NEXT_SAMPLE, LtkError, _dev, _ptr, _stream, library


def next_sample_workspace_bytes(L: int) -> int:
    """Workspace bytes litetopk_next_sample needs for L keys."""
    n = library().litetopk_workspace_bytes(KIND_NEXT_SAMPLE, 0, 0, 0, L, 1, 0, 0, None)
    if n == 0:
        raise ValueError(f"invalid key count {L}")
    return int(n)


def next_sample(prev_idx, L: int, n_sample: int, workspace=None):
    """int32 [n_sample] keys most often selected by the rows of prev_idx [T, k]
    (ties to the lower index; in no particular order), computed on the device
    by litetopk_next_sample."""
    import torch
    if prev_idx.dim() != 2:
        raise ValueError(f"prev_idx must be [T, k], got {tuple(prev_idx.shape)}")
    if not 0 <= n_sample <= L:
        raise ValueError(f"n_sample must lie in [0, L = {L}], got {n_sample}")
    _dev(prev_idx, "prev_idx", torch.int32)
    T, k = prev_idx.shape
    lib = library()
    fn = lib.litetopk_next_sample
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    out = torch.empty(n_sample, dtype=torch.int32, device=prev_idx.device)
    ws = workspace if workspace is not None else torch.empty(next_sample_workspace_bytes(L), dtype=torch.uint8,
                                                             device=prev_idx.device)
    rc = fn(_ptr(prev_idx), T, k, L, n_sample, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream())
    if rc != 0:
        raise LtkError(rc, "litetopk_next_sample")
    return out


def prefill_workspace_bytes(n_queries: int, chunk: int, H: int, D: int, L: int, topk: int, n_sample: int,
                            dtype_code: int, opts=None) -> int:
    """Workspace of `prefill_chunked`: the largest that any of its calls needs.
    A short last chunk can need more than a full one (fewer query groups get
    more key splits, which can switch on shared thresholds and a larger
    candidate capacity), and the first chunk runs without a sample."""
    from ._binding import KIND_SCORE_SELECT, workspace_bytes
    sizes = {min(chunk, n_queries)}
    if n_queries % chunk:
        sizes.add(n_queries % chunk)
    need = 0
    for T in sizes:
        for ns in (0, n_sample):
            b = workspace_bytes(KIND_SCORE_SELECT, T, H, D, L, topk, ns, dtype_code, opts)
            if b == 0:
                raise ValueError("invalid prefill sizes")
            need = max(need, b)
    return need


def prefill_chunked(queries, k, topk: int, n_queries: int, chunk: int = 8192, n_sample: int | None = None,
                    k_scale=None, first_pos: int = 0, opts=None, keep_outputs: bool = False,
                    diagnostics: bool = True):
    """Whole-prefill driver: the queries at positions first_pos .. first_pos+n_queries-1
    in chunks of `chunk`, each chunk scored against every key at or before its
    queries, with the previous chunk's most-selected 3k keys as its sample (the
    LiteTopK pages, "Sampling"); the first chunk has no sample.

    `queries` is either (q [n_queries, H, D], w [n_queries, H], q_scale or None)
    or a function (c0, c1) -> that triple for the queries c0 .. c1-1, so a long
    prefill need not hold every query at once.  One workspace, sized for the
    largest call (`prefill_workspace_bytes`), serves every chunk; the sample
    size is clamped to L.

    Returns {"chunks": [per-chunk dict], "workspace_bytes": int, "last": int32
    [rows, topk] of the last chunk, "outputs": list of every chunk's indices if
    keep_outputs}.  Per chunk: queries, causal pairs, and with `diagnostics`
    the ms of the select call (device events), candidates per query, overflow
    rows, and the sample hit rate (fraction of the chunk's selected keys that
    were in its sample).  Without `diagnostics` the chunks are enqueued back to
    back with no host synchronisation between them.
    """
    import torch
    from ._binding import _dtype_code, score_select

    L = k.shape[0]
    n_sample = min(3 * topk if n_sample is None else n_sample, L)

    def get(c0, c1):
        if callable(queries):
            return queries(c0, c1)
        q, w, qs = queries
        return q[c0:c1], w[c0:c1], None if qs is None else qs[c0:c1]

    q0, _, _ = get(0, min(chunk, n_queries))
    H, D = q0.shape[1], q0.shape[2]
    nbytes = prefill_workspace_bytes(n_queries, chunk, H, D, L, topk, n_sample, _dtype_code(q0), opts)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=k.device)
    ws_sample = torch.empty(next_sample_workspace_bytes(L), dtype=torch.uint8, device=k.device)
    records, outputs, prev = [], [], None
    for c0 in range(0, n_queries, chunk):
        c1 = min(n_queries, c0 + chunk)
        q, w, qs = get(c0, c1)
        pos = torch.arange(first_pos + c0, first_pos + c1, dtype=torch.int32, device=k.device)
        sample = next_sample(prev, L, n_sample, workspace=ws_sample) if prev is not None else None
        if not diagnostics:
            idx = score_select(q, k, w, pos, topk, sample=sample, q_scale=qs, k_scale=k_scale, opts=opts,
                               workspace=ws)
            # causal pairs: query at position p sees min(p, L - 1) + 1 keys
            p0, p1 = first_pos + c0, first_pos + c1
            below = max(0, min(p1, L) - p0)
            pairs = below * (p0 + 1) + below * (below - 1) // 2 + (c1 - c0 - below) * L
            records.append({"chunk": c0 // chunk, "queries": c1 - c0, "pairs": pairs})
            if keep_outputs:
                outputs.append(idx)
            prev = idx
            continue
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        idx, st = score_select(q, k, w, pos, topk, sample=sample, q_scale=qs, k_scale=k_scale, opts=opts,
                               return_stats=True, workspace=ws)
        e1.record()
        e1.synchronize()
        valid = idx >= 0
        if sample is not None and sample.numel() > 0:
            hit = float((torch.isin(idx, sample) & valid).sum().item()) / max(1, int(valid.sum().item()))
        else:
            hit = None
        ends = torch.clamp(pos.to(torch.int64), max=L - 1) + 1
        records.append({"chunk": c0 // chunk, "queries": c1 - c0, "pairs": int(ends.sum().item()),
                        "ms": e0.elapsed_time(e1), "candidates_per_query": st.cand_written / (c1 - c0),
                        "max_candidates": st.max_cand_per_query, "overflow_rows": st.overflow_rows,
                        "sample_hit_rate": hit})
        if keep_outputs:
            outputs.append(idx)
        prev = idx
    return {"chunks": records, "workspace_bytes": nbytes, "last": prev, "outputs": outputs if keep_outputs else None}
