"""MI355X (gfx950) fused Indexer-TopK: Python binding of liblitetopk.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library (see include/litetopk.h for the C ABI).  PyTorch
provides device memory and the current stream.

    import indexer_topk_long_amd as ltk
    idx = ltk.score_select(q, k, w, pos, topk=2048, sample=prev_top3k)

If the library has not been built, every call raises; there is no fallback.
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    KIND_RETRIEVE,
    KIND_SCORE_SELECT,
    KIND_UNFUSED,
    KIND_UNFUSED_RETRIEVE,
    HipEvents,
    LtkError,
    Opts,
    Stats,
    device_check,
    dsa_gather,
    dsa_pack,
    exported_symbols,
    library,
    retrieve,
    score_select,
    score_select_static,
    strerror,
    unfused_retrieve,
    unfused_score_select,
    workspace_bytes,
)
from .prefill import next_sample, prefill_chunked, prefill_workspace_bytes  # noqa: F401

__all__ = [
    "score_select", "retrieve", "unfused_score_select", "workspace_bytes", "strerror", "device_check",
    "Opts", "Stats", "LtkError", "next_sample", "prefill_chunked", "library", "exported_symbols",
    "dsa_pack", "dsa_gather", "prefill_workspace_bytes", "score_select_static", "unfused_retrieve",
]
