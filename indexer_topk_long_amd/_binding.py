"""ctypes binding of liblitetopk.so (same names as the C ABI, minus the prefix)."""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

from .build import INCLUDE, lib_path

KIND_SCORE_SELECT, KIND_RETRIEVE, KIND_UNFUSED, KIND_NEXT_SAMPLE, KIND_UNFUSED_RETRIEVE = 0, 1, 2, 3, 4
_STATUS = {0: "LTK_OK", -1: "LTK_EINVAL", -2: "LTK_EUNSUPPORTED", -3: "LTK_EWORKSPACE", -4: "LTK_EHIP"}

_c_i32, _c_i64, _c_sz, _c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p


class _COpts(ctypes.Structure):
    _fields_ = [("nbins", _c_i32), ("refresh_every", _c_i32), ("l_splits", _c_i32),
                ("sorted_output", _c_i32), ("cand_capacity", _c_i64),
                ("scan_event_start", _c_p), ("scan_event_stop", _c_p), ("shared_threshold", _c_i32),
                ("flush_batch", _c_i32)]


@dataclass
class Opts:
    """Tuning options (none changes the result): see ltk_opts in litetopk.h."""
    nbins: int = 0
    refresh_every: int = 0
    l_splits: int = 0
    sorted_output: bool = False
    cand_capacity: int = 0
    scan_event_start: int | None = None   # raw hipEvent_t handles (profiling)
    scan_event_stop: int | None = None
    shared_threshold: int = 0             # 0 auto (>= 16 key splits), 1 always, -1 never
    flush_batch: int = 0                  # candidates per write-back batch: 32 or 64 (0 = 64)

    def c(self) -> _COpts:
        return _COpts(self.nbins, self.refresh_every, self.l_splits, int(bool(self.sorted_output)),
                      self.cand_capacity, self.scan_event_start, self.scan_event_stop, self.shared_threshold,
                      self.flush_batch)


@dataclass
class Stats:
    cand_written: int
    bytes_written: int
    max_cand_per_query: int
    overflow_rows: int


class LtkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({strerror(status)})")


_LIB = None


def library() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (no fallback path exists)."""
    global _LIB
    if _LIB is None:
        # torch ships its own HIP runtime with the same SONAME as the system one;
        # importing torch first makes the library bind to that already-loaded copy,
        # so one process never holds two HIP runtimes.
        import torch  # noqa: F401
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m indexer_topk_long_amd.build`")
        lib = ctypes.CDLL(path)
        lib.litetopk_workspace_bytes.restype = _c_sz
        lib.litetopk_workspace_bytes.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_i32, _c_p]
        lib.litetopk_score_select.restype = ctypes.c_int
        lib.litetopk_score_select.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i64,
                                              _c_i32, _c_i32, _c_p, _c_i32, _c_p, _c_p, _c_p, _c_sz, _c_p, _c_p, _c_p]
        lib.litetopk_score_select_static.restype = ctypes.c_int
        lib.litetopk_score_select_static.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                                     _c_i64, _c_i32, _c_i32, _c_p, _c_i32, _c_p, _c_p, _c_p, _c_p,
                                                     _c_p]
        lib.litetopk_unfused_score_select.restype = ctypes.c_int
        lib.litetopk_unfused_score_select.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                                      _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_sz, _c_p]
        lib.litetopk_retrieve.restype = ctypes.c_int
        lib.litetopk_retrieve.argtypes = [_c_p, _c_p, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_p, _c_i32, _c_p,
                                          _c_p, _c_p, _c_sz, _c_p, _c_p, _c_p]
        lib.litetopk_unfused_retrieve.restype = ctypes.c_int
        lib.litetopk_unfused_retrieve.argtypes = [_c_p, _c_p, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_p, _c_p,
                                                  _c_p, _c_sz, _c_p, _c_p]
        lib.litetopk_strerror.restype = ctypes.c_char_p
        lib.litetopk_strerror.argtypes = [ctypes.c_int]
        lib.litetopk_device_check.restype = ctypes.c_int
        lib.litetopk_device_check.argtypes = []
        lib.litetopk_dsa_pack.restype = ctypes.c_int
        lib.litetopk_dsa_pack.argtypes = [_c_p, _c_i32, _c_i32, _c_i64, _c_i32, _c_p, _c_p, _c_p, _c_p]
        lib.litetopk_dsa_gather.restype = ctypes.c_int
        lib.litetopk_dsa_gather.argtypes = [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i32, _c_i32, _c_p, _c_p]
        _LIB = lib
    return _LIB


def exported_symbols() -> list[str]:
    """Function names declared in include/litetopk.h."""
    with open(os.path.join(INCLUDE, "litetopk.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(litetopk_\w+)\s*\(", src, flags=re.M)))


def strerror(status: int) -> str:
    return library().litetopk_strerror(int(status)).decode()


def device_check() -> int:
    return int(library().litetopk_device_check())


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: 0, torch.bfloat16: 1, torch.float8_e4m3fn: 2}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, bfloat16 or float8_e4m3fn")
    return codes[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtype=None):
    import torch
    if t is None:
        return None
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _expect(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _same_device(ref, **named):
    for name, t in named.items():
        if t is not None:
            _expect(t.device == ref.device, f"{name} is on {t.device}, q on {ref.device}: all tensors must share one device")


def _check_indexer_args(q, k, w, pos, q_scale=None, k_scale=None, sample=None):
    """Shapes, dtypes and devices of an indexer call, checked before anything
    reaches the library (a mismatch would make the kernels read past the end
    of a buffer).  Returns (T, H, D, L, dtype code)."""
    import torch
    _expect(q.dim() == 3, f"q must be [T, H, D], got shape {tuple(q.shape)}")
    _expect(k.dim() == 2, f"k must be [L, D], got shape {tuple(k.shape)}")
    _expect(q.dtype == k.dtype, f"q ({q.dtype}) and k ({k.dtype}) must share one dtype")
    T, H, D = q.shape
    L = k.shape[0]
    _expect(k.shape[1] == D, f"k rows have {k.shape[1]} elements, q rows {D}")
    _expect(tuple(w.shape) == (T, H), f"w must be [{T}, {H}], got {tuple(w.shape)}")
    _expect(w.dtype == torch.float32, f"w must be float32, got {w.dtype}")
    _expect(tuple(pos.shape) == (T,), f"pos must be [{T}], got {tuple(pos.shape)}")
    _expect(pos.dtype == torch.int32, f"pos must be int32, got {pos.dtype}")
    dt = _dtype_code(q)
    if dt == 2:
        _expect(q_scale is not None and k_scale is not None, "fp8 needs q_scale [T] and k_scale [L]")
        _expect(tuple(q_scale.shape) == (T,), f"q_scale must be [{T}], got {tuple(q_scale.shape)}")
        _expect(tuple(k_scale.shape) == (L,), f"k_scale must be [{L}], got {tuple(k_scale.shape)}")
        _expect(q_scale.dtype == torch.float32 and k_scale.dtype == torch.float32, "scales must be float32")
    else:
        _expect(q_scale is None and k_scale is None, "q_scale and k_scale are for float8_e4m3fn inputs only")
    if sample is not None:
        _expect(sample.dtype == torch.int32, f"sample must be int32, got {sample.dtype}")
    _same_device(q, k=k, w=w, pos=pos, q_scale=q_scale, k_scale=k_scale, sample=sample)
    for name, t in (("q", q), ("k", k), ("w", w), ("pos", pos), ("q_scale", q_scale), ("k_scale", k_scale),
                    ("sample", sample)):
        _dev(t, name)
    return T, H, D, L, dt


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_bytes(kind: int, T: int, H: int, D: int, L: int, topk: int, n_sample: int, dtype_code: int,
                    opts: Opts | None = None) -> int:
    o = opts.c() if opts is not None else None
    return int(library().litetopk_workspace_bytes(kind, T, H, D, L, topk, n_sample, dtype_code,
                                                  ctypes.byref(o) if o is not None else None))


def _workspace(nbytes: int, device, ws=None):
    import torch
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small")
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _stats_buf(device):
    import torch
    return torch.zeros(3, dtype=torch.int64, device=device)   # ltk_stats: u64, u64, u32, u32


def _read_stats(buf) -> Stats:
    v = buf.cpu()
    return Stats(int(v[0]), int(v[1]), int(v[2]) & 0xFFFFFFFF, (int(v[2]) >> 32) & 0xFFFFFFFF)


def score_select(q, k, w, pos, topk: int, sample=None, q_scale=None, k_scale=None, opts: Opts | None = None,
                 return_scores: bool = False, return_stats: bool = False, workspace=None, out=None):
    """Fused indexer top-k (litetopk_score_select).

    q [T, H, D] and k [L, D] in float32 / bfloat16 / float8_e4m3fn (fp8 needs
    q_scale [T] and k_scale [L] fp32); w [T, H] fp32; pos [T] int32; sample
    int32 key indices (the previous chunk's top-3k).  Returns int32 [T, topk]
    (-1 padded; written into ``out`` when given, which may overlap the
    sample), plus fp32 scores and/or Stats when asked.
    """
    import torch
    T, H, D, L, dt = _check_indexer_args(q, k, w, pos, q_scale, k_scale, sample)
    ns = 0 if sample is None else sample.numel()
    lib = library()
    o = opts.c() if opts is not None else None
    nbytes = lib.litetopk_workspace_bytes(KIND_SCORE_SELECT, T, H, D, L, topk, ns, dt,
                                          ctypes.byref(o) if o is not None else None)
    if nbytes == 0:
        raise LtkError(-1, "litetopk_workspace_bytes")
    ws = _workspace(nbytes, q.device, workspace)
    if out is None:
        out = torch.empty((T, topk), dtype=torch.int32, device=q.device)
    elif tuple(out.shape) != (T, topk):
        raise ValueError(f"out must be [{T}, {topk}]")
    else:
        _dev(out, "out", torch.int32)
    osc = torch.empty((T, topk), dtype=torch.float32, device=q.device) if return_scores else None
    st = _stats_buf(q.device) if return_stats else None
    rc = lib.litetopk_score_select(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), _ptr(pos), T, H, D, L,
                                   dt, topk, _ptr(sample), ns, _ptr(out), _ptr(osc), _ptr(ws),
                                   ws.numel() * ws.element_size(), ctypes.byref(o) if o is not None else None,
                                   _ptr(st), _stream())
    if rc != 0:
        raise LtkError(rc, "litetopk_score_select")
    res = [out]
    if return_scores:
        res.append(osc)
    if return_stats:
        res.append(_read_stats(st))
    return res[0] if len(res) == 1 else tuple(res)


def score_select_static(q, k, w, pos, topk: int, sample=None, q_scale=None, k_scale=None, opts: Opts | None = None,
                        return_scores: bool = False, return_stats: bool = False, out=None, out_score=None):
    """litetopk_score_select_static: score_select on the library's static
    workspace (no workspace allocation).  With `out` (and `out_score`) given,
    the call allocates nothing at all: the caller owns every buffer."""
    import torch
    T, H, D, L, dt = _check_indexer_args(q, k, w, pos, q_scale, k_scale, sample)
    ns = 0 if sample is None else sample.numel()
    if out is None:
        out = torch.empty((T, topk), dtype=torch.int32, device=q.device)
    _expect(tuple(out.shape) == (T, topk), f"out must be [{T}, {topk}]")
    _dev(out, "out", torch.int32)
    osc = out_score
    if return_scores and osc is None:
        osc = torch.empty((T, topk), dtype=torch.float32, device=q.device)
    if osc is not None:
        _expect(tuple(osc.shape) == (T, topk), f"out_score must be [{T}, {topk}]")
        _dev(osc, "out_score", torch.float32)
    st = _stats_buf(q.device) if return_stats else None
    o = opts.c() if opts is not None else None
    rc = library().litetopk_score_select_static(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), _ptr(pos),
                                                T, H, D, L, dt, topk, _ptr(sample), ns, _ptr(out), _ptr(osc),
                                                ctypes.byref(o) if o is not None else None, _ptr(st), _stream())
    if rc != 0:
        raise LtkError(rc, "litetopk_score_select_static")
    res = [out]
    if return_scores:
        res.append(osc)
    if return_stats:
        res.append(_read_stats(st))
    return res[0] if len(res) == 1 else tuple(res)


def unfused_score_select(q, k, w, pos, topk: int, q_scale=None, k_scale=None, return_scores: bool = False,
                         workspace=None):
    """Unfused comparison path (full score matrix + radix select)."""
    import torch
    T, H, D, L, dt = _check_indexer_args(q, k, w, pos, q_scale, k_scale)
    lib = library()
    nbytes = lib.litetopk_workspace_bytes(KIND_UNFUSED, T, H, D, L, topk, 0, dt, None)
    ws = _workspace(nbytes, q.device, workspace)
    out = torch.empty((T, topk), dtype=torch.int32, device=q.device)
    osc = torch.empty((T, topk), dtype=torch.float32, device=q.device) if return_scores else None
    rc = lib.litetopk_unfused_score_select(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), _ptr(pos), T, H,
                                           D, L, dt, topk, _ptr(out), _ptr(osc), _ptr(ws),
                                           ws.numel() * ws.element_size(), _stream())
    if rc != 0:
        raise LtkError(rc, "litetopk_unfused_score_select")
    return (out, osc) if return_scores else out


def _check_retrieve_args(q, db):
    _expect(q.dim() == 2 and db.dim() == 2, f"q must be [T, D] and db [N, D], got {tuple(q.shape)}, {tuple(db.shape)}")
    _expect(q.dtype == db.dtype, f"q ({q.dtype}) and db ({db.dtype}) must share one dtype")
    _expect(db.shape[1] == q.shape[1], f"db rows have {db.shape[1]} elements, q rows {q.shape[1]}")


def unfused_retrieve(q, db, topk: int, opts: Opts | None = None, return_scores: bool = False, workspace=None):
    """Unfused retrieval comparison path (litetopk_unfused_retrieve): the full
    T x N score matrix in the workspace, then a radix select per row."""
    import torch
    _check_retrieve_args(q, db)
    _same_device(q, db=db)
    _dev(q, "q"), _dev(db, "db")
    T, D = q.shape
    N = db.shape[0]
    dt = _dtype_code(q)
    lib = library()
    o = opts.c() if opts is not None else None
    nbytes = lib.litetopk_workspace_bytes(KIND_UNFUSED_RETRIEVE, T, 1, D, N, topk, 0, dt, None)
    if nbytes == 0:
        raise LtkError(-1, "litetopk_workspace_bytes")
    ws = _workspace(nbytes, q.device, workspace)
    out = torch.empty((T, topk), dtype=torch.int32, device=q.device)
    osc = torch.empty((T, topk), dtype=torch.float32, device=q.device) if return_scores else None
    rc = lib.litetopk_unfused_retrieve(_ptr(q), _ptr(db), T, D, N, dt, topk, _ptr(out), _ptr(osc), _ptr(ws),
                                       ws.numel() * ws.element_size(),
                                       ctypes.byref(o) if o is not None else None, _stream())
    if rc != 0:
        raise LtkError(rc, "litetopk_unfused_retrieve")
    return (out, osc) if return_scores else out


def retrieve(q, db, topk: int, sample=None, opts: Opts | None = None, return_scores: bool = False,
             return_stats: bool = False, workspace=None):
    """Fused inner-product retrieval top-k (litetopk_retrieve); q [T, D], db [N, D] bfloat16."""
    import torch
    _check_retrieve_args(q, db)
    if sample is not None:
        _expect(sample.dtype == torch.int32, f"sample must be int32, got {sample.dtype}")
    _same_device(q, db=db, sample=sample)
    _dev(q, "q"), _dev(db, "db"), _dev(sample, "sample")
    T, D = q.shape
    N = db.shape[0]
    dt = _dtype_code(q)
    ns = 0 if sample is None else sample.numel()
    lib = library()
    o = opts.c() if opts is not None else None
    nbytes = lib.litetopk_workspace_bytes(KIND_RETRIEVE, T, 1, D, N, topk, ns, dt,
                                          ctypes.byref(o) if o is not None else None)
    if nbytes == 0:
        raise LtkError(-1, "litetopk_workspace_bytes")
    ws = _workspace(nbytes, q.device, workspace)
    out = torch.empty((T, topk), dtype=torch.int32, device=q.device)
    osc = torch.empty((T, topk), dtype=torch.float32, device=q.device) if return_scores else None
    st = _stats_buf(q.device) if return_stats else None
    rc = lib.litetopk_retrieve(_ptr(q), _ptr(db), T, D, N, dt, topk, _ptr(sample), ns, _ptr(out), _ptr(osc),
                               _ptr(ws), ws.numel() * ws.element_size(),
                               ctypes.byref(o) if o is not None else None, _ptr(st), _stream())
    if rc != 0:
        raise LtkError(rc, "litetopk_retrieve")
    res = [out]
    if return_scores:
        res.append(osc)
    if return_stats:
        res.append(_read_stats(st))
    return res[0] if len(res) == 1 else tuple(res)


def dsa_pack(idx, L: int, group: int):
    """LiteDSA packing (litetopk_dsa_pack): for groups of `group` consecutive
    rows of idx [T, k] (int32 selected keys), the ascending shared list of
    their distinct keys, the per-entry masks (bit i: row g*group + i selected
    the key) and the list lengths.  Returns (shared int32 [G, group*k],
    masks uint32 [G, group*k], lens int32 [G])."""
    import torch
    _expect(idx.dim() == 2, f"idx must be [T, k], got {tuple(idx.shape)}")
    _dev(idx, "idx", torch.int32)
    T, k = idx.shape
    ng = (T + group - 1) // group
    shared = torch.empty((ng, group * k), dtype=torch.int32, device=idx.device)
    masks = torch.empty((ng, group * k), dtype=torch.uint32, device=idx.device)
    lens = torch.empty((ng,), dtype=torch.int32, device=idx.device)
    rc = library().litetopk_dsa_pack(_ptr(idx), T, k, L, group, _ptr(shared), _ptr(masks), _ptr(lens), _stream())
    if rc != 0:
        raise LtkError(rc, "litetopk_dsa_pack")
    return shared, masks, lens


def dsa_gather(kv, shared, lens, out=None):
    """The key/value rows of each group's shared list, contiguous
    (litetopk_dsa_gather): out[g, j] = kv[shared[g, j]] for j < lens[g]; kv is
    [L, ...] with 16-byte-multiple rows.  Returns out [G, cap, *kv.shape[1:]]."""
    import torch
    _expect(shared.dim() == 2 and lens.dim() == 1 and lens.shape[0] == shared.shape[0] and kv.dim() >= 1,
            f"shared must be [G, cap], lens [G] and kv [L, ...]; got {tuple(shared.shape)}, {tuple(lens.shape)}, "
            f"{tuple(kv.shape)}")
    _same_device(kv, shared=shared, lens=lens, out=out)
    _dev(kv, "kv"), _dev(shared, "shared", torch.int32), _dev(lens, "lens", torch.int32)
    L = kv.shape[0]
    row_bytes = kv[0].numel() * kv.element_size() if L else 0
    ng, cap = shared.shape
    if out is None:
        out = torch.empty((ng, cap) + tuple(kv.shape[1:]), dtype=kv.dtype, device=kv.device)
    else:
        _expect(tuple(out.shape) == (ng, cap) + tuple(kv.shape[1:]),
                f"out must be {(ng, cap) + tuple(kv.shape[1:])}, got {tuple(out.shape)}")
        _dev(out, "out", kv.dtype)
    rc = library().litetopk_dsa_gather(_ptr(kv), L, row_bytes, _ptr(shared), _ptr(lens), ng, cap, _ptr(out),
                                       _stream())
    if rc != 0:
        raise LtkError(rc, "litetopk_dsa_gather")
    return out


class HipEvents:
    """hipEvent_t pairs from the HIP runtime already loaded by torch (for timing one kernel)."""

    def __init__(self, n: int):
        library()
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(a)) or self.hip.hipEventCreate(ctypes.byref(b)):
                raise RuntimeError("hipEventCreate failed")
            self.pairs.append((a.value, b.value))

    def elapsed_ms(self, i: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.pairs[i][0], self.pairs[i][1])
        if rc:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)
        self.pairs = []
