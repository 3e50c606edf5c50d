"""Seeded input generators for the Indexer-TopK workloads.

The workloads stand in for the activations of a DSA-style sparse-attention
indexer in long-context prefill (LiteTopK pages, "Problem statement" and
"Experimental results": 1M-token context, 8,192-token chunks, k = 2,048) and
for a dense vector-retrieval workload (same pages, "Large-scale retrieval":
k from 1,024 up).  The pages print neither the data nor the generator; the
recipe below is synthetic and is stated in full in the design notes.

Score concentration, the property the method relies on (pages, "Methodology":
in high dimension, scores crowd into a narrow band with a long tail), is
built in: most keys are isotropic Gaussian noise and a minority of "hot" keys
carry a component along a shared direction that the queries also lean on.

The module holds no scoring, binning or selection arithmetic.  It returns raw
storage arrays (fp32 values, bf16 bit patterns as uint16, OCP fp8 e4m3fn bit
patterns as uint8 with fp32 per-token scales), exactly the bits handed to the
GPU, so that the oracle can decode the very same values.
"""
from __future__ import annotations

import math

import numpy as np

SEED_BASE = 20260713

# stream ids inside one workload's SeedSequence
_S_KEYS, _S_HOT, _S_QUERIES, _S_WEIGHTS, _S_SAMPLE, _S_PREV_QUERIES, _S_DB = 0, 1, 2, 3, 4, 5, 6
_S_DIR = 7

# The workloads, by name.  "tiny-4k-fp32" is small enough for the oracle to
# finish in seconds; the three prefill chunks sit at 64K / 256K / 1M context;
# the last one is the retrieval workload.  "tag" seeds the workload's streams.
WORKLOADS = {
    "tiny-4k-fp32": dict(kind="indexer", tag=0, T=64, L=4096, H=4, D=64, dtype="f32",
                         topk=256, n_hot=128, drift=False, w_range=(0.5, 1.0), n_sample=768),
    "prefill-64k-bf16": dict(kind="indexer", tag=1, T=2048, L=65536, H=64, D=128, dtype="bf16",
                             topk=2048, n_hot=4096, drift=True, w_range=(0.0, 1.0), n_sample=6144),
    "prefill-256k-bf16": dict(kind="indexer", tag=2, T=8192, L=262144, H=64, D=128, dtype="bf16",
                              topk=2048, n_hot=16384, drift=True, w_range=(0.0, 1.0), n_sample=6144),
    "prefill-1m-fp8": dict(kind="indexer", tag=3, T=8192, L=1048576, H=64, D=128, dtype="fp8",
                           topk=2048, n_hot=65536, drift=True, w_range=(0.0, 1.0), n_sample=6144),
    "retrieval-8m-d768-bf16": dict(kind="retrieval", tag=4, T=1024, N=8_000_000, D=768,
                                   dtype="bf16", topk=1024, n_centres=1000, sigma=0.3, n_sample=3072),
    # Decode over the 1M-context keys: T queries at the newest positions per
    # step (one new token, or one plus seven draft tokens verified together),
    # each step's sample being the previous step's result.
    "decode-1m-fp8": dict(kind="decode", keys="prefill-1m-fp8", T=1),
    "specdecode-1m-fp8": dict(kind="decode", keys="prefill-1m-fp8", T=8),
    # LiteDSA packing of the 1M-context chunk's selections in groups of 16
    # neighbouring queries; the key/value rows gathered are 576 bf16 values
    # (1,152 bytes, the latent key/value row width of DSA-style attention)
    "dsa-1m-fp8": dict(kind="dsa", keys="prefill-1m-fp8", group=16, kv_row_bytes=1152),
}
INDEXER_WORKLOADS = [n for n, c in WORKLOADS.items() if c["kind"] == "indexer"]

FP8_MAX = 448.0  # largest finite OCP e4m3fn value


def _rng(tag: int, stream: int, seed: int = SEED_BASE) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tag, stream]))


def _unit(v: np.ndarray, axis: int = -1) -> np.ndarray:
    return v / np.linalg.norm(v, axis=axis, keepdims=True)


def to_storage(x: np.ndarray, dtype: str, axes=None, inplace: bool = False):
    """Round fp32 values to the storage format ``dtype``.

    Returns ``(raw, scale)``: ``raw`` holds fp32 values, bf16 bit patterns
    (uint16) or e4m3fn bit patterns (uint8); ``scale`` is None except for fp8,
    where it is the fp32 per-token scale amax/448 over ``axes`` (so that no
    value saturates) and ``raw`` encodes ``x / scale``.  With ``inplace`` the
    fp8 path may overwrite ``x``.
    """
    import torch

    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x, None
    if dtype == "bf16":
        t = torch.from_numpy(x).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16), None
    if dtype == "fp8":
        # amax without an |x| temporary (large arrays are costly to allocate)
        amax = np.maximum(x.max(axis=axes, keepdims=True), -x.min(axis=axes, keepdims=True)).astype(np.float32)
        scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
        scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
        if not inplace:
            x = x.copy()
        np.divide(x, scale, out=x)
        t = torch.from_numpy(x).to(torch.float8_e4m3fn)
        raw = t.view(torch.uint8).numpy()
        return raw, scale.reshape(-1).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _direction(tag: int, D: int, seed: int):
    """Shared unit direction(s): u0 and an orthogonal u1 for the drifting case."""
    g = _rng(tag, _S_DIR, seed)
    u0 = _unit(g.standard_normal(D))
    v = g.standard_normal(D)
    v = v - (v @ u0) * u0
    u1 = _unit(v)
    return u0, u1


def _u_at(p: np.ndarray, L: int, u0: np.ndarray, u1: np.ndarray, drift: bool) -> np.ndarray:
    """Unit direction at positions p: a quarter turn from u0 to u1 over the context."""
    if not drift:
        return np.broadcast_to(u0, (len(p), len(u0)))
    phi = (math.pi / 2.0) * (np.asarray(p, dtype=np.float64) / float(L))
    v = np.cos(phi)[:, None] * u0[None, :] + np.sin(phi)[:, None] * u1[None, :]
    return _unit(v)


def indexer_inputs(T: int, L: int, H: int, D: int, dtype: str, topk: int, n_hot: int,
                   drift: bool = False, w_range=(0.0, 1.0), tag: int = 100,
                   seed: int = SEED_BASE, chunk: int = 0, pos=None, n_sample: int | None = None,
                   hot_gain: float = 3.0, q_gain: float = 0.5, keys=None):
    """Inputs for one indexer chunk.

    Keys: k[s] = N(0, I_D) + hot_gain * u(s) for s in a hot set of n_hot keys
    drawn without replacement.  Queries: q[t, h] = q_gain * u(pos[t]) +
    N(0, I_D) / sqrt(D).  Head weights: U(w_range).  Positions: the last T
    positions of the context for chunk 0, the T before them for chunk -1 (the
    previous chunk, whose queries come from their own stream), unless ``pos``
    is given.

    Returns a dict of raw storage arrays and sizes.  ``sample`` holds
    ``n_sample`` distinct seeded-random causal key indices (a bootstrap sample;
    the previous-chunk sample is built by the caller from a previous run).
    """
    u0, u1 = _direction(tag, D, seed)
    if keys is None:
        gk = _rng(tag, _S_KEYS, seed)
        k = gk.standard_normal((L, D), dtype=np.float32)
        gh = _rng(tag, _S_HOT, seed)
        n_hot = min(n_hot, L)
        hot = np.sort(gh.choice(L, size=n_hot, replace=False)) if n_hot > 0 else np.zeros(0, np.int64)
        if n_hot:
            for s0 in range(0, n_hot, 1 << 16):
                h = hot[s0 : s0 + (1 << 16)]
                k[h] += (hot_gain * _u_at(h, L, u0, u1, drift)).astype(np.float32)

    if pos is None:
        end = L + chunk * T
        pos = np.arange(end - T, end, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    assert pos.shape == (T,)
    gq = _rng(tag, _S_QUERIES if chunk == 0 else _S_PREV_QUERIES + 16 * (-chunk - 1), seed)
    q = gq.standard_normal((T, H, D), dtype=np.float32)
    q /= np.float32(math.sqrt(D))
    q += (q_gain * _u_at(np.clip(pos, 0, L - 1), L, u0, u1, drift)).astype(np.float32)[:, None, :]
    gw = _rng(tag, _S_WEIGHTS + 16 * (-chunk), seed)
    w = gw.uniform(w_range[0], w_range[1], size=(T, H)).astype(np.float32)

    q_raw, q_scale = to_storage(q, dtype, axes=(1, 2), inplace=True)
    del q
    if keys is None:
        k_raw, k_scale = to_storage(k, dtype, axes=(1,), inplace=True)
        del k
    else:  # the same (already rounded) keys as another chunk of this context
        k_raw, k_scale, hot = keys
    out = dict(kind="indexer", T=T, L=L, H=H, D=D, dtype=dtype, topk=topk,
               q=q_raw, k=k_raw, q_scale=q_scale, k_scale=k_scale, w=w,
               pos=pos.astype(np.int32), hot=hot.astype(np.int64))
    if n_sample is not None:
        out["sample"] = random_sample(n_sample, int(pos.max()) + 1 if T else L, tag, seed, stream=_S_SAMPLE + 16 * (-chunk))
    return out


def random_sample(n: int, upto: int, tag: int = 0, seed: int = SEED_BASE, stream: int = _S_SAMPLE) -> np.ndarray:
    """n distinct uniform indices in [0, upto), as int32 (fewer if upto < n)."""
    g = _rng(tag, stream, seed)
    n = min(n, upto)
    return np.sort(g.choice(upto, size=n, replace=False)).astype(np.int32)


def indexer_workload(name: str, chunk: int = 0, seed: int = SEED_BASE, with_prev: bool = False):
    """The seeded inputs of the named indexer workload; chunk -1 is the previous chunk.

    With ``with_prev``, the result also holds ``prev``: the previous chunk's
    queries, weights, positions and bootstrap sample over the same keys.
    """
    c = WORKLOADS[name]
    assert c["kind"] == "indexer"
    out = indexer_inputs(c["T"], c["L"], c["H"], c["D"], c["dtype"], c["topk"], c["n_hot"],
                         drift=c["drift"], w_range=c["w_range"], tag=c["tag"], seed=seed, chunk=chunk,
                         n_sample=c["n_sample"], keys=None)
    out["name"] = name
    if with_prev:
        p = indexer_inputs(c["T"], c["L"], c["H"], c["D"], c["dtype"], c["topk"], c["n_hot"],
                           drift=c["drift"], w_range=c["w_range"], tag=c["tag"], seed=seed, chunk=chunk - 1,
                           n_sample=c["n_sample"], keys=(out["k"], out["k_scale"], out["hot"]))
        out["prev"] = p
    return out


def indexer_keys(name: str, seed: int = SEED_BASE):
    """Keys of the named indexer workload alone (raw storage, per-key scales
    or None), the same as ``indexer_workload(name)["k"]``."""
    c = WORKLOADS[name]
    assert c["kind"] == "indexer"
    out = indexer_inputs(0, c["L"], c["H"], c["D"], c["dtype"], c["topk"], c["n_hot"], drift=c["drift"],
                         w_range=c["w_range"], tag=c["tag"], seed=seed)
    return out["k"], out["k_scale"]


_S_SELECT = 9    # stream id of the synthetic selection rows


def selection_rows(T: int, k: int, L: int, tag: int = 0, seed: int = SEED_BASE, spread: float = 1.5,
                   drift: int = 4, invalid: float = 0.0) -> np.ndarray:
    """Top-k-like selections of T neighbouring queries: row t holds k distinct
    keys drawn from a window of spread*k candidate keys that moves by `drift`
    candidates per row, so neighbouring rows overlap heavily.  A fraction
    `invalid` of the entries is replaced by -1.  int32 [T, k]."""
    g = _rng(tag, _S_SELECT, seed)
    w = max(int(spread * k), k)
    n = min(L, w + drift * T)
    cands = g.choice(L, size=n, replace=False).astype(np.int32)
    rows = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        win = cands[min(t * drift, max(n - w, 0)):][:w]
        m = min(k, len(win))
        rows[t, :m] = win[g.permutation(len(win))[:m]]
    if invalid > 0:
        rows[g.random(rows.shape) < invalid] = -1
    return rows


_S_PREFILL = 8   # stream id of the whole-prefill queries drawn on the device


def prefill_queries(name: str, device: str = "cuda", seed: int = SEED_BASE):
    """Queries and head weights of a whole prefill over the named indexer
    workload's keys, drawn with torch's generator on ``device``.

    Returns a function (c0, c1) -> (q, w, q_scale) for the queries at
    positions c0 .. c1-1: q[t, h] = q_gain * u(t) + N(0, I_D) / sqrt(D) and
    w ~ U(w_range), as in ``indexer_inputs``, rounded to the workload's storage
    format (fp8: per-token scale amax / 448).  Each chunk is drawn from its own
    generator state (seeded by its start position), so chunks can be drawn in
    any order.
    """
    import torch

    c = WORKLOADS[name]
    assert c["kind"] == "indexer"
    L, H, D, dt = c["L"], c["H"], c["D"], c["dtype"]
    u0, u1 = _direction(c["tag"], D, seed)
    dev = torch.device(device)
    tu0 = torch.from_numpy(u0.astype(np.float32)).to(dev)
    tu1 = torch.from_numpy(u1.astype(np.float32)).to(dev)
    base = int(np.random.SeedSequence([seed, c["tag"], _S_PREFILL]).generate_state(1, dtype=np.uint64)[0] >> 2)

    def chunk(c0: int, c1: int):
        g = torch.Generator(device=dev)
        g.manual_seed(base + c0)
        n = c1 - c0
        p = torch.arange(c0, c1, device=dev, dtype=torch.float64)
        if c["drift"]:
            phi = (math.pi / 2.0) * p / float(L)
            u = torch.cos(phi)[:, None].float() * tu0[None, :] + torch.sin(phi)[:, None].float() * tu1[None, :]
            u = u / torch.linalg.vector_norm(u, dim=1, keepdim=True)
        else:
            u = tu0[None, :].expand(n, D)
        q = torch.randn((n, H, D), generator=g, device=dev, dtype=torch.float32) / math.sqrt(D)
        q += 0.5 * u[:, None, :]
        w = torch.rand((n, H), generator=g, device=dev, dtype=torch.float32)
        w = c["w_range"][0] + (c["w_range"][1] - c["w_range"][0]) * w
        if dt == "f32":
            return q.contiguous(), w.contiguous(), None
        if dt == "bf16":
            return q.to(torch.bfloat16).contiguous(), w.contiguous(), None
        amax = q.abs().amax(dim=(1, 2))
        scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
        return (q / scale[:, None, None]).to(torch.float8_e4m3fn).contiguous(), w.contiguous(), scale.contiguous()

    return chunk


def _retrieval_centres(n_centres: int, D: int, tag: int, seed: int) -> np.ndarray:
    return _rng(tag, _S_HOT, seed).standard_normal((n_centres, D)).astype(np.float32)


def retrieval_queries(T: int, D: int, n_centres: int = 1000, sigma: float = 0.3, tag: int = 4,
                      seed: int = SEED_BASE, batch: int = 0, db_dtype: str = "bf16"):
    """Queries of the retrieval workload: unit(c_j + sigma * N(0, I_D)) with j
    uniform over the centres.  Batch 0 is the workload's own batch; batch -1,
    -2, ... are earlier batches of the same distribution (their own streams).
    Returns (raw storage bits, centre of each query)."""
    gq = _rng(tag, _S_QUERIES if batch == 0 else _S_PREV_QUERIES + 16 * (-batch - 1), seed)
    cq = gq.integers(0, n_centres, size=T)
    centres = _retrieval_centres(n_centres, D, tag, seed)
    q = _unit(centres[cq] + sigma * gq.standard_normal((T, D)).astype(np.float32)).astype(np.float32)
    q_raw, _ = to_storage(q, db_dtype)
    return q_raw, cq


def retrieval_inputs(T: int, N: int, D: int, topk: int, n_centres: int = 1000, sigma: float = 0.3,
                     n_sample: int = 3072, tag: int = 4, seed: int = SEED_BASE, device: str = "cpu",
                     block: int = 1 << 20, db_dtype: str = "bf16"):
    """Gaussian-mixture retrieval workload.

    Centres c_j ~ N(0, I_D); database row i = unit(c_{a_i} + sigma * N(0, I_D))
    with a_i uniform; query = unit(c_j + sigma * N(0, I_D)) with j uniform.
    The database is drawn with torch's generator on ``device`` (so that 8M
    rows of 768 dims can be drawn on the GPU in milliseconds) in blocks of
    ``block`` rows, then rounded to bf16; queries and the sample come from
    numpy.  Returns numpy queries (uint16 bf16 bits) and a torch bf16 database
    tensor on ``device``.
    """
    import torch

    centres = _retrieval_centres(n_centres, D, tag, seed)
    q_raw, cq = retrieval_queries(T, D, n_centres, sigma, tag=tag, seed=seed, db_dtype=db_dtype)

    dev = torch.device(device)
    seed_db = int(np.random.SeedSequence([seed, tag, _S_DB]).generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)
    g = torch.Generator(device=dev)
    g.manual_seed(seed_db)
    cen = torch.from_numpy(centres).to(dev)
    tdt = torch.bfloat16 if db_dtype == "bf16" else torch.float32
    db = torch.empty((N, D), dtype=tdt, device=dev)
    for s0 in range(0, N, block):
        n = min(block, N - s0)
        a = torch.randint(0, n_centres, (n,), generator=g, device=dev)
        x = cen[a] + sigma * torch.randn((n, D), generator=g, device=dev, dtype=torch.float32)
        x = x / torch.linalg.vector_norm(x, dim=1, keepdim=True)
        db[s0:s0 + n] = x.to(tdt)
        del a, x
    sample = random_sample(n_sample, N, tag, seed, stream=_S_SAMPLE)
    return dict(kind="retrieval", T=T, N=N, D=D, dtype=db_dtype, topk=topk, q=q_raw, db=db,
                sample=sample, centre_of_query=cq)


def retrieval_workload(name: str = "retrieval-8m-d768-bf16", device: str = "cpu", seed: int = SEED_BASE,
                       N: int | None = None, T: int | None = None):
    """The seeded inputs of the named retrieval workload (optionally with fewer rows or queries)."""
    c = WORKLOADS[name]
    assert c["kind"] == "retrieval"
    return retrieval_inputs(T or c["T"], N or c["N"], c["D"], c["topk"], c["n_centres"], c["sigma"],
                            c["n_sample"], tag=c["tag"], seed=seed, device=device)


def random_retrieval_sample_of(name: str, n: int, seed: int = SEED_BASE) -> np.ndarray:
    """n distinct seeded-random rows of the named retrieval workload's database."""
    c = WORKLOADS[name]
    return random_sample(n, c["N"], c["tag"], seed, stream=_S_SAMPLE)
