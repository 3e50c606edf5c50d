"""Chunk-to-chunk carry of the sample (LiteTopK pages, "Sampling": the
previous chunk's top-3k tokens serve as the next chunk's sample)."""
from __future__ import annotations

import ctypes

from ._binding import LtkError, _dev, _ptr, _stream, library


def next_sample(prev_idx, L: int, n_sample: int, workspace=None):
    """int32 [n_sample] keys most often selected by the rows of prev_idx [T, k]
    (ties to the lower index), computed on the device by litetopk_next_sample."""
    import torch
    _dev(prev_idx, "prev_idx", torch.int32)
    T, k = prev_idx.shape
    lib = library()
    fn = lib.litetopk_next_sample
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    out = torch.empty(n_sample, dtype=torch.int32, device=prev_idx.device)
    ws = workspace if workspace is not None else torch.empty(max(4 * L, 256), dtype=torch.uint8,
                                                             device=prev_idx.device)
    rc = fn(_ptr(prev_idx), T, k, L, n_sample, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream())
    if rc != 0:
        raise LtkError(rc, "litetopk_next_sample")
    return out
