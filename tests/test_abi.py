"""The C ABI without a GPU: the library loads, exports every function the
header declares, the header is plain C with the struct layout the binding
uses, and every argument error is reported before any device call."""
import ctypes
import os
import subprocess

import pytest

import indexer_topk_long_amd as ltk
from indexer_topk_long_amd import build as B

OK, EINVAL, EUNSUP, EWS, EHIP = 0, -1, -2, -3, -4
F32, BF16, FP8 = 0, 1, 2
P = ctypes.c_void_p
A16 = P(0x10000)          # a 16-byte-aligned fake device address (never dereferenced)
MIS = P(0x10004)          # a misaligned one


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.lib_path()):
        B.build()
    return ltk.library()


def test_every_declared_symbol_is_exported(L):
    names = ltk.exported_symbols()
    assert len(names) == 11
    for n in names:
        assert hasattr(L, n), n


def test_header_is_c_and_matches_binding_layout(tmp_path):
    src = tmp_path / "probe.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "litetopk.h"\n'
        'int main(void){printf("%zu %zu %zu %zu %zu\\n", sizeof(ltk_opts), offsetof(ltk_opts, cand_capacity),'
        ' offsetof(ltk_opts, scan_event_stop), sizeof(ltk_stats), offsetof(ltk_stats, overflow_rows));'
        ' printf("%zu %zu %zu\\n", offsetof(ltk_opts, shared_threshold), offsetof(ltk_opts, flush_batch),'
        ' offsetof(ltk_stats, bytes_written)); return 0;}\n')
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", B.INCLUDE, str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    from indexer_topk_long_amd._binding import _COpts
    assert got[0] == ctypes.sizeof(_COpts)
    assert got[1] == _COpts.cand_capacity.offset and got[2] == _COpts.scan_event_stop.offset
    assert got[3] == 24 and got[4] == 20     # Stats: u64 + u64 + u32 + u32, read as three int64 by the binding
    assert got[5] == _COpts.shared_threshold.offset and got[6] == _COpts.flush_batch.offset and got[7] == 8


def test_strerror(L):
    for code in (OK, EINVAL, EUNSUP, EWS, EHIP):
        assert len(ltk.strerror(code)) >= 2 and ltk.strerror(code) != "unknown status"
    assert ltk.strerror(12345) == "unknown status"


def test_workspace_decode_shape_reserves_shared_histograms(L):
    # one fp8 query over 128K keys: 32 splits of 4K keys share T x nbins counters
    # and get at least 256 candidate slots per split
    ws = lambda o=None: ltk.workspace_bytes(0, 1, 64, 128, 131072, 2048, 2048, 2, o)
    on, off = ws(), ws(ltk.Opts(shared_threshold=-1))
    assert on - off >= 32 * 256 * 8 - 16384 * 8 + 256 * 4 - 256
    assert ws(ltk.Opts(shared_threshold=1)) == on
    # an explicit capacity is kept; sharing then adds only the histograms
    c_on = ws(ltk.Opts(cand_capacity=4096))
    c_off = ws(ltk.Opts(cand_capacity=4096, shared_threshold=-1))
    assert 0 < c_on - c_off <= 1024 + 256
    # a prefill chunk (2 splits) does not share
    p = lambda o=None: ltk.workspace_bytes(0, 8192, 64, 128, 1 << 20, 2048, 6144, 2, o)
    assert p() == p(ltk.Opts(shared_threshold=-1)) < p(ltk.Opts(shared_threshold=1))


def test_workspace_sizes(L):
    ws = lambda *a: ltk.workspace_bytes(*a)
    a = ws(0, 64, 4, 64, 4096, 256, 768, F32)
    b = ws(0, 128, 4, 64, 4096, 256, 768, F32)
    c = ws(0, 64, 4, 64, 4096, 256, 1536, F32)
    assert 0 < a < b and a < c
    assert 100 * 1000 * 4 <= ws(2, 100, 4, 64, 1000, 10, 0, F32) < 100 * 1000 * 4 + 256
    assert ws(1, 1024, 1, 768, 8_000_000, 1024, 3072, BF16) > 1024 * 131072 * 8
    assert ws(0, -1, 4, 64, 4096, 256, 0, F32) == 0 and ws(0, 4, 4, 64, 0, 256, 0, F32) == 0
    assert ws(0, 4, 4, 64, 100, 256, 0, F32, ltk.Opts(nbins=5000)) == 0
    # 1M-context fp8 chunk workspace: candidates (8192 x 16384 x 8 B) dominate, about the pages' 1.5 GB of auxiliary memory
    assert 1.0e9 < ws(0, 8192, 64, 128, 1 << 20, 2048, 6144, FP8) < 1.6e9


def _ss(L, **kw):
    a = dict(q=A16, qs=None, k=A16, ks=None, w=A16, pos=A16, T=4, H=4, D=64, Lk=100, dt=F32, topk=8,
             sample=None, ns=0, out=A16, osc=None, ws=A16, wsb=1 << 30, opts=None, stats=None, stream=None)
    a.update(kw)
    o = a["opts"].c() if a["opts"] is not None else None
    return L.litetopk_score_select(a["q"], a["qs"], a["k"], a["ks"], a["w"], a["pos"], a["T"], a["H"], a["D"],
                                   a["Lk"], a["dt"], a["topk"], a["sample"], a["ns"], a["out"], a["osc"], a["ws"],
                                   a["wsb"], ctypes.byref(o) if o is not None else None, a["stats"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), EINVAL), (dict(H=0), EUNSUP), (dict(H=65), EUNSUP), (dict(D=96), EUNSUP),
    (dict(dt=7), EINVAL), (dict(topk=0), EINVAL), (dict(topk=65537), EINVAL), (dict(Lk=0), EINVAL),
    (dict(q=None), EINVAL), (dict(k=None), EINVAL), (dict(w=None), EINVAL), (dict(pos=None), EINVAL),
    (dict(out=None), EINVAL), (dict(ws=None), EINVAL), (dict(q=MIS), EINVAL), (dict(k=MIS), EINVAL),
    (dict(ws=MIS), EINVAL), (dict(dt=FP8), EINVAL), (dict(dt=FP8, qs=A16), EINVAL), (dict(qs=A16), EINVAL),
    (dict(ns=3), EINVAL), (dict(ns=-1), EINVAL), (dict(wsb=100), EWS),
    (dict(opts=ltk.Opts(nbins=1025)), EINVAL), (dict(opts=ltk.Opts(l_splits=-2)), EINVAL),
    (dict(opts=ltk.Opts(sorted_output=True), topk=9000), EINVAL), (dict(opts=ltk.Opts(cand_capacity=-5)), EINVAL),
    (dict(opts=ltk.Opts(flush_batch=48)), EINVAL), (dict(opts=ltk.Opts(flush_batch=128)), EINVAL),
    (dict(T=0, opts=ltk.Opts(flush_batch=32)), OK), (dict(T=0, opts=ltk.Opts(flush_batch=64)), OK),
    (dict(T=0), OK),
    # no queries: the per-query arrays (query scales included) may be NULL; key scales may not
    (dict(T=0, q=None, w=None, pos=None, out=None, dt=FP8, ks=A16), OK),
    (dict(T=0, dt=FP8, qs=A16), EINVAL),
])
def test_score_select_argument_errors(L, kw, code):
    assert _ss(L, **kw) == code


def _rt(L, **kw):
    a = dict(q=A16, db=A16, T=4, D=128, N=1000, dt=BF16, topk=8, sample=None, ns=0, out=A16, osc=None, ws=A16,
             wsb=1 << 30, opts=None, stats=None, stream=None)
    a.update(kw)
    return L.litetopk_retrieve(a["q"], a["db"], a["T"], a["D"], a["N"], a["dt"], a["topk"], a["sample"], a["ns"],
                               a["out"], a["osc"], a["ws"], a["wsb"], None, a["stats"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dt=FP8), EUNSUP), (dict(dt=F32), EUNSUP), (dict(dt=9), EINVAL), (dict(D=100), EUNSUP),
    (dict(D=1024), EUNSUP), (dict(N=0), EINVAL), (dict(topk=0), EINVAL), (dict(db=None), EINVAL),
    (dict(db=MIS), EINVAL), (dict(ns=5), EINVAL), (dict(wsb=10), EWS), (dict(T=0), OK),
])
def test_retrieve_argument_errors(L, kw, code):
    assert _rt(L, **kw) == code


def test_retrieve_split_size_limit(L):
    """An explicit split count that leaves more than 2^26 rows in a split is
    rejected (a queue entry of the scan packs the row's offset in its split
    in 26 bits); the automatic count respects the limit.  No queries: nothing
    is launched."""
    o = ltk.Opts(l_splits=1).c()
    big = (1 << 26) + 1
    f = L.litetopk_retrieve
    assert f(A16, A16, 0, 128, big, BF16, 8, None, 0, A16, None, A16, 1 << 40, ctypes.byref(o), None, None) == EINVAL
    o2 = ltk.Opts(l_splits=2).c()
    assert f(A16, A16, 0, 128, big, BF16, 8, None, 0, A16, None, A16, 1 << 40, ctypes.byref(o2), None, None) == OK
    assert f(A16, A16, 0, 128, big, BF16, 8, None, 0, A16, None, A16, 1 << 40, None, None, None) == OK
    u = L.litetopk_unfused_retrieve
    assert u(A16, A16, 0, 128, big, BF16, 8, A16, None, A16, 1 << 40, ctypes.byref(o), None) == EINVAL


def test_unfused_retrieve_argument_errors(L):
    u = L.litetopk_unfused_retrieve
    need = L.litetopk_workspace_bytes(4, 4, 1, 128, 1000, 8, 0, BF16, None)   # LTK_KIND_UNFUSED_RETRIEVE
    assert 4 * 1000 * 4 <= need < 4 * 1000 * 4 + 256                          # the T x N fp32 matrix
    assert u(A16, A16, 4, 128, 1000, BF16, 8, A16, None, A16, need - 1, None, None) == EWS
    assert u(A16, A16, 4, 128, 1000, FP8, 8, A16, None, A16, need, None, None) == EUNSUP
    assert u(A16, A16, 4, 100, 1000, BF16, 8, A16, None, A16, need, None, None) == EUNSUP
    assert u(A16, MIS, 4, 128, 1000, BF16, 8, A16, None, A16, need, None, None) == EINVAL
    assert u(A16, A16, 4, 128, 0, BF16, 8, A16, None, A16, need, None, None) == EINVAL
    assert u(A16, A16, 0, 128, 1000, BF16, 8, None, None, None, 0, None, None) == OK


def test_unfused_and_next_sample_argument_errors(L):
    f = L.litetopk_unfused_score_select
    assert f(A16, None, A16, None, A16, A16, 4, 4, 64, 100, F32, 8, A16, None, A16, 10, None) == EWS
    assert f(A16, None, A16, None, A16, A16, 4, 4, 64, 100, FP8, 8, A16, None, A16, 1 << 20, None) == EINVAL
    assert f(A16, None, A16, None, A16, A16, 0, 4, 64, 100, F32, 8, A16, None, A16, 0, None) == OK
    assert f(None, None, A16, A16, None, None, 0, 4, 64, 100, FP8, 8, None, None, A16, 0, None) == OK
    ns = L.litetopk_next_sample
    ns.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, P, P, ctypes.c_size_t, P]
    assert ns(A16, 4, 8, 100, 101, A16, A16, 1 << 20, None) == EINVAL  # more samples than keys
    need = L.litetopk_workspace_bytes(3, 0, 0, 0, 100, 1, 0, 0, None)    # LTK_KIND_NEXT_SAMPLE
    assert need == 4 * (128 + 16384 + 64 + 1024)                          # counts, histogram, header, ties
    assert ns(A16, 4, 8, 100, 10, A16, A16, need - 1, None) == EWS
    assert ns(A16, 4, 8, 100, 0, A16, A16, 0, None) == OK
    assert L.litetopk_workspace_bytes(3, 0, 0, 0, 0, 1, 0, 0, None) == 0   # no keys
    assert L.litetopk_workspace_bytes(7, 1, 1, 1, 100, 1, 0, 0, None) == 0  # no such kind


def test_dsa_argument_errors(L):
    pk, ga = L.litetopk_dsa_pack, L.litetopk_dsa_gather
    I32, I64 = ctypes.c_int32, ctypes.c_int64
    pk.argtypes = [P, I32, I32, I64, I32, P, P, P, P]
    ga.argtypes = [P, I64, I64, P, P, I32, I32, P, P]
    assert pk(A16, 8, 2048, 1 << 20, 0, A16, A16, A16, None) == EINVAL      # group 0
    assert pk(A16, 8, 2048, 1 << 20, 33, A16, A16, A16, None) == EINVAL     # more than 32 rows per mask
    assert pk(A16, 8, 2048, 1 << 20, 17, A16, A16, A16, None) == EUNSUP     # 17 x 2048 > 32768 entries
    assert pk(A16, 8, 64, (1 << 26) + 1, 4, A16, A16, A16, None) == EUNSUP  # key << 5 | row needs L <= 2^26
    assert pk(A16, 8, 0, 100, 4, A16, A16, A16, None) == EINVAL
    assert pk(None, 8, 64, 100, 4, A16, A16, A16, None) == EINVAL
    assert pk(None, 0, 64, 100, 4, None, None, None, None) == OK            # no rows: nothing to do
    assert ga(A16, 100, 24, A16, A16, 4, 64, A16, None) == EINVAL           # rows not whole 16-byte vectors
    assert ga(MIS, 100, 32, A16, A16, 4, 64, A16, None) == EINVAL           # misaligned key/value rows
    assert ga(A16, 100, 32, A16, A16, 4, 0, A16, None) == EINVAL
    assert ga(None, 100, 32, None, None, 0, 64, None, None) == OK


# --------------------------------------------------------------------------- binding argument checks


def _cpu(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def _indexer_args(T=4, H=8, D=64, Lk=100, dtype="f32"):
    import torch
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[dtype]
    a = dict(q=_cpu((T, H, D), tdt), k=_cpu((Lk, D), tdt), w=_cpu((T, H), torch.float32),
             pos=_cpu((T,), torch.int32), q_scale=None, k_scale=None)
    if dtype == "fp8":
        a.update(q_scale=_cpu((T,), torch.float32), k_scale=_cpu((Lk,), torch.float32))
    return a


@pytest.mark.parametrize("change,match", [
    (dict(k=((100, 128), "f32")), "k rows have 128"),               # q with D = 64, k with D = 128
    (dict(w=((4, 7), "w")), r"w must be \[4, 8\]"),
    (dict(w=((3, 8), "w")), r"w must be \[4, 8\]"),
    (dict(pos=((5,), "pos")), r"pos must be \[4\]"),
    (dict(k=((100, 64), "bf16")), "share one dtype"),
    (dict(q=((4, 64), "f32")), r"q must be \[T, H, D\]"),
    (dict(q_scale=((4,), "w")), "float8_e4m3fn inputs only"),
])
def test_binding_rejects_mismatched_indexer_arguments(change, match):
    """Every size the kernels rely on is checked before the library is called
    (on CPU tensors the checks run before the device check)."""
    import torch
    a = _indexer_args()
    for name, (shape, kind) in change.items():
        a[name] = _cpu(shape, {"f32": torch.float32, "bf16": torch.bfloat16, "w": torch.float32,
                               "pos": torch.int32}[kind])
    with pytest.raises(ValueError, match=match):
        ltk.score_select(a["q"], a["k"], a["w"], a["pos"], 8, q_scale=a["q_scale"], k_scale=a["k_scale"])
    with pytest.raises(ValueError, match=match):
        ltk.unfused_score_select(a["q"], a["k"], a["w"], a["pos"], 8, q_scale=a["q_scale"], k_scale=a["k_scale"])


def test_binding_rejects_bad_fp8_scales_and_sample():
    import torch
    a = _indexer_args(dtype="fp8")
    with pytest.raises(ValueError, match=r"k_scale must be \[100\]"):
        ltk.score_select(a["q"], a["k"], a["w"], a["pos"], 8, q_scale=a["q_scale"], k_scale=_cpu((99,), torch.float32))
    with pytest.raises(ValueError, match=r"q_scale must be \[4\]"):
        ltk.score_select(a["q"], a["k"], a["w"], a["pos"], 8, q_scale=_cpu((3,), torch.float32), k_scale=a["k_scale"])
    with pytest.raises(ValueError, match="fp8 needs"):
        ltk.score_select(a["q"], a["k"], a["w"], a["pos"], 8)
    with pytest.raises(ValueError, match="sample must be int32"):
        ltk.score_select(a["q"], a["k"], a["w"], a["pos"], 8, q_scale=a["q_scale"], k_scale=a["k_scale"],
                         sample=_cpu((6,), torch.int64))
    # consistent shapes on the CPU: only the device check is left
    with pytest.raises(ValueError, match="device tensor"):
        ltk.score_select(a["q"], a["k"], a["w"], a["pos"], 8, q_scale=a["q_scale"], k_scale=a["k_scale"])


def test_binding_rejects_mismatched_retrieval_and_dsa_arguments():
    import torch
    q, db = _cpu((4, 128), torch.bfloat16), _cpu((1000, 64), torch.bfloat16)
    with pytest.raises(ValueError, match="db rows have 64"):
        ltk.retrieve(q, db, 8)
    with pytest.raises(ValueError, match="share one dtype"):
        ltk.retrieve(q, _cpu((1000, 128), torch.float32), 8)
    with pytest.raises(ValueError, match=r"idx must be \[T, k\]"):
        ltk.dsa_pack(_cpu((16,), torch.int32), 100, 4)
    with pytest.raises(ValueError, match="lens"):
        ltk.dsa_gather(_cpu((100, 16), torch.uint8), _cpu((3, 8), torch.int32), _cpu((2,), torch.int32))
    with pytest.raises(ValueError, match="n_sample must lie"):
        ltk.next_sample(_cpu((4, 8), torch.int32), 10, 11)


def test_prefill_workspace_covers_a_short_last_chunk(L):
    """A short last chunk gets more key splits, which switches on shared
    thresholds and a larger capacity: the driver's one workspace must cover it,
    and the first chunk's call without a sample."""
    full = ltk.workspace_bytes(0, 1024, 64, 128, 1 << 20, 2048, 6144, FP8)
    tail = ltk.workspace_bytes(0, 40, 64, 128, 1 << 20, 2048, 6144, FP8)
    assert tail > full
    need = ltk.prefill_workspace_bytes(1024 * 3 + 40, 1024, 64, 128, 1 << 20, 2048, 6144, FP8)
    assert need >= max(full, tail, ltk.workspace_bytes(0, 40, 64, 128, 1 << 20, 2048, 0, FP8))
    assert ltk.prefill_workspace_bytes(2048, 1024, 64, 128, 1 << 20, 2048, 6144, FP8) == max(
        full, ltk.workspace_bytes(0, 1024, 64, 128, 1 << 20, 2048, 0, FP8))


def test_split_ranges_at_the_key_limit(tmp_path):
    """The scans' split arithmetic (csrc/split.hpp) in 64 bits: at L near the
    2^31 - 256 key limit, with up to 4,096 splits of 32- to 512-key tiles, the
    ranges partition [0, L) into tile-aligned, ordered, non-negative pieces."""
    src = tmp_path / "split_check.cpp"
    src.write_text(r"""
#include <stdio.h>
#include "split.hpp"
int main() {
    const long long ends[] = {1, 511, 512, 513, 1048576, 2147483647LL - 256 - 511, 2147483647LL - 256};
    const int ns[] = {1, 2, 3, 7, 256, 4096};
    const int tiles[] = {32, 64, 128, 256, 512};
    long long bad = 0;
    for (long long end : ends) for (int n : ns) for (int tile : tiles) {
        long long next = 0;
        for (int s = 0; s < n; ++s) {
            const ltk::KeyRange r = ltk::split_range(end, n, s, tile);
            if (r.lo < 0 || r.hi < r.lo || r.hi > end || r.lo != next) ++bad;
            if (r.hi > r.lo && r.lo % tile != 0) ++bad;
            next = r.hi;
        }
        if (next != end) ++bad;
    }
    if (!ltk::tile_inside(2147483647LL - 256 - 512, 512, 2147483647LL - 256)) ++bad;
    if (ltk::tile_inside(2147483647LL - 256 - 100, 512, 2147483647LL - 256)) ++bad;
    printf("%lld\n", bad);
    return bad != 0;
}
""")
    exe = tmp_path / "split_check"
    csrc = os.path.join(os.path.dirname(B.INCLUDE), "indexer_topk_long_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", csrc, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "0", r.stdout
