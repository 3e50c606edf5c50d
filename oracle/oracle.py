"""CPU oracle for the fused Indexer-TopK -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import or call anything in this package.  The GPU library never does, and
this package imports nothing from the GPU library.

What it computes is the plain definition that the LiteTopK method claims to
reach exactly (LiteTopK pages: arXiv abstract, "preserving exact top-k
correctness"; summary, "Selection": exact top-k).  No sampling, no bins:

  valid keys   V_t = { s : 0 <= s <= pos[t], s < L }           (causal, inclusive)
  indexer      I[t, s] = sum_h w[t, h] * max(0, q[t, h, :] . k[s, :])
  retrieval    I[t, s] = q[t, :] . x[s, :]                      (no heads, no ReLU)
  output       the first min(k, |V_t|) keys of V_t ordered by (I descending,
               index ascending), padded with -1 to length k.

The indexer score is the DSA-style indexer score (the pages call it the
relevance score of every candidate token, "Problem statement"); the
retrieval score is the inner product of the pages' vector-retrieval use.
LiteDSA packing (arXiv abstract) is written out as plain set operations on
the selected indices: per group of neighbouring queries, the sorted union of
their selections and a membership bitmask per union entry.

Inputs are the raw storage bits handed to the GPU (fp32 values, bf16 bit
patterns, OCP e4m3fn bit patterns with fp32 per-token scales) and are decoded
exactly to fp64; all arithmetic is fp64.  Ties are broken towards the lower
index by a full lexicographic sort; bit-identical keys (or database rows)
are scored once, at their first copy, so that they tie exactly.

Parity status: every function here is pinned by the tests in
tests/test_oracle.py (brute-force ranks, exhaustive subsets, hand-derived
golden values, algebraic identities, library special cases).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# exact decoding of the storage formats
# ---------------------------------------------------------------------------


def e4m3fn_table() -> np.ndarray:
    """fp64 value of each of the 256 OCP FP8 E4M3 ("fn") codes.

    From the OCP 8-bit floating point specification: 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
    (m/8) * 2^-6; S.1111.111 is NaN; there are no infinities, so the largest
    finite magnitude is 1.75 * 2^8 = 448.
    """
    vals = np.empty(256, dtype=np.float64)
    for b in range(256):
        sign = -1.0 if b & 0x80 else 1.0
        e = (b >> 3) & 0xF
        m = b & 0x7
        if e == 0xF and m == 0x7:
            vals[b] = np.nan
        elif e == 0:
            vals[b] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[b] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3fn_table()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64: a bf16 is the top half of an fp32."""
    b = np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode(raw: np.ndarray, dtype: str, scale: np.ndarray | None = None) -> np.ndarray:
    """Exact fp64 values of a storage array.

    For fp8, ``scale`` holds one fp32 factor per leading index (per token);
    the product of an e4m3fn value and an fp32 scale is exact in fp64.
    """
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(raw)
    if dtype == "fp8":
        v = _E4M3[np.asarray(raw, dtype=np.uint8)]
        if scale is not None:
            s = np.asarray(scale, dtype=np.float32).astype(np.float64)
            v = v * s.reshape((-1,) + (1,) * (v.ndim - 1))
        return v
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# scores
# ---------------------------------------------------------------------------


def indexer_scores(q: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Indexer scores of one query against a block of keys, in fp64.

    q: [H, D] decoded query heads; w: [H] head weights; keys: [n, D] decoded
    keys.  Returns [n] with I[s] = sum_h w[h] * max(0, q[h] . keys[s]).
    """
    x = keys @ q.T                      # [n, H]: per-head dot products
    return np.maximum(x, 0.0) @ w       # ReLU, then the weighted sum over heads


def retrieval_scores(q: np.ndarray, db: np.ndarray) -> np.ndarray:
    """Inner products q . x[s] of one query ([D]) against a block of rows, in
    fp64 ([n]); with queries as columns ([D, R]), one column per query ([n, R])."""
    return db @ q


def first_copy(raw: np.ndarray, scale: np.ndarray | None = None) -> np.ndarray:
    """For each stored row, the index of the first row with the same stored
    bits (and the same per-row scale, when given).

    A score is a function of the key's value, so bit-identical keys must get
    bit-identical scores for ties to reach the index order.  A blocked BLAS
    product does not guarantee that (rows in a block's tail or in another
    thread's share can take a different rounding path), so the scoring
    functions evaluate each distinct row once, at its first copy, and hand
    that value to every copy.  Rows are grouped by a 64-bit hash of their
    bytes and every grouping is then confirmed byte for byte; a row whose
    bytes differ from its group's first row keeps itself.
    """
    n = raw.shape[0]
    b = np.ascontiguousarray(raw).reshape(n, -1).view(np.uint8)
    if scale is not None:
        b = np.concatenate([b, np.ascontiguousarray(scale, dtype=np.float32).reshape(n, 1).view(np.uint8)], axis=1)
    if b.shape[1] % 8:
        b = np.concatenate([b, np.zeros((n, 8 - b.shape[1] % 8), np.uint8)], axis=1)
    words = np.ascontiguousarray(b).view(np.uint64)
    # hash: sum of the row's 64-bit words times fixed odd multipliers, mod
    # 2^64 (rows taken in blocks, so that large tables stream through memory
    # once); a collision only costs the byte comparison below
    mult = (np.arange(words.shape[1], dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)) | np.uint64(1)
    h = np.empty(n, np.uint64)
    with np.errstate(over="ignore"):
        for r0 in range(0, n, 1 << 14):
            h[r0 : r0 + (1 << 14)] = (words[r0 : r0 + (1 << 14)] * mult).sum(axis=1, dtype=np.uint64)
    _, first, inv = np.unique(h, return_index=True, return_inverse=True)
    rep = first[inv.ravel()].astype(np.int64)
    moved = np.nonzero(rep != np.arange(n))[0]
    if len(moved):
        same = np.all(words[moved] == words[rep[moved]], axis=1)
        rep[moved[~same]] = moved[~same]
    return rep


def key_table(inp: dict):
    """(decoded keys fp64 [L, D], first_copy of each key) of an indexer input."""
    return decode(inp["k"], inp["dtype"], inp.get("k_scale")), first_copy(inp["k"], inp.get("k_scale"))


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------


def topk_row(scores: np.ndarray, idx: np.ndarray, k: int):
    """The k best (score desc, index asc) of one row, padded with -1 / NaN."""
    order = np.lexsort((idx, -scores))[:k]
    out_i = np.full(k, -1, dtype=np.int32)
    out_s = np.full(k, np.nan, dtype=np.float64)
    out_i[: len(order)] = idx[order]
    out_s[: len(order)] = scores[order]
    return out_i, out_s


def valid_keys(pos_t: int, L: int) -> np.ndarray:
    """Causal key set of a query at position pos_t: 0..min(pos_t, L-1)."""
    hi = min(int(pos_t), L - 1)
    return np.arange(0, hi + 1, dtype=np.int64) if hi >= 0 else np.zeros(0, dtype=np.int64)


def indexer_row_scores(inp: dict, t: int, keys=None):
    """(valid key indices, fp64 scores) of query t of an indexer input dict.

    ``keys`` is ``key_table(inp)``, computed here when not given.  A key's
    score is the score of its first bit-identical copy (``first_copy``)."""
    dt = inp["dtype"]
    kd, rep = key_table(inp) if keys is None else keys
    qs = inp.get("q_scale")
    qd = decode(inp["q"][t : t + 1], dt, None if qs is None else qs[t : t + 1])[0]
    w = np.asarray(inp["w"][t], dtype=np.float32).astype(np.float64)
    v = valid_keys(inp["pos"][t], inp["L"])
    s = indexer_scores(qd, w, kd[: len(v)])           # V_t is the prefix 0..pos[t]
    return v, s[rep[: len(v)]]                         # a first copy never lies after its copies


def oracle_indexer(inp: dict, rows=None, with_scores: bool = True):
    """Exact top-k of the indexer input ``inp`` for the query rows ``rows``.

    Returns (idx int32 [R, k], scores fp64 [R, k]); padded entries are -1/NaN.
    """
    T, k = inp["T"], inp["topk"]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    keys = key_table(inp)
    out_i = np.full((len(rows), k), -1, dtype=np.int32)
    out_s = np.full((len(rows), k), np.nan, dtype=np.float64)
    for r, t in enumerate(rows):
        v, s = indexer_row_scores(inp, int(t), keys)
        out_i[r], out_s[r] = topk_row(s, v, k)
    return (out_i, out_s) if with_scores else out_i


def oracle_retrieval(q_raw: np.ndarray, db_raw: np.ndarray, k: int, rows=None, dtype: str = "bf16",
                     block: int = 1 << 18):
    """Exact top-k inner-product retrieval for the query rows ``rows``.

    db_raw is the raw [N, D] storage; it is decoded in blocks of ``block``
    rows so that an 8M x 768 database never exists in fp64 at once.
    """
    T = q_raw.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    qd = decode(q_raw[rows], dtype)                      # [R, D]
    N = db_raw.shape[0]
    scores = np.empty((len(rows), N), dtype=np.float64)
    for s0 in range(0, N, block):
        xd = decode(db_raw[s0 : s0 + block], dtype)      # [n, D]
        scores[:, s0 : s0 + len(xd)] = (xd @ qd.T).T
    scores = scores[:, first_copy(db_raw)]               # bit-identical rows score alike
    idx = np.arange(N, dtype=np.int64)
    out_i = np.full((len(rows), k), -1, dtype=np.int32)
    out_s = np.full((len(rows), k), np.nan, dtype=np.float64)
    for r in range(len(rows)):
        out_i[r], out_s[r] = topk_row(scores[r], idx, k)
    return out_i, out_s


def retrieval_row_scores(q_raw: np.ndarray, db_raw: np.ndarray, t, dtype: str = "bf16",
                         block: int = 1 << 18, rep: np.ndarray | None = None) -> np.ndarray:
    """fp64 scores of query t against every database row ([N]); for a
    sequence of query indices, one row of scores per query ([len(t), N]).
    ``rep`` is ``first_copy(db_raw)`` (computed here when not given): each row
    takes the score of its first bit-identical copy."""
    many = not np.isscalar(t)
    rows = np.atleast_1d(np.asarray(t, dtype=np.int64))
    qd = decode(q_raw[rows], dtype)                      # [R, D]
    N = db_raw.shape[0]
    out = np.empty((len(rows), N), dtype=np.float64)
    for s0 in range(0, N, block):
        xd = decode(db_raw[s0 : s0 + block], dtype)      # [n, D]
        out[:, s0 : s0 + len(xd)] = retrieval_scores(qd.T, xd).T   # [n, R] -> [R, n]
    out = out[:, first_copy(db_raw) if rep is None else rep]
    return out if many else out[0]


def next_sample(prev_idx: np.ndarray, L: int, n: int) -> np.ndarray:
    """Keys 0..L-1 ranked by how many entries of prev_idx name them (entries
    outside [0, L), such as -1 padding, are ignored; a top-k row names a key
    at most once, so this is the number of rows that selected it), ties to
    the lower index; the first n, in rank order.  This is the reading of the
    pages' "reuse the previous chunk's top-3k tokens as the sample"
    ("Sampling") for one shared sample per chunk."""
    p = np.asarray(prev_idx).ravel()
    counts = np.bincount(p[(p >= 0) & (p < L)], minlength=L)
    return np.lexsort((np.arange(L), -counts))[:n].astype(np.int32)


# ---------------------------------------------------------------------------
# LiteDSA packing (arXiv abstract: LiteDSA packs the overlapping candidates of
# neighbouring query tokens into one shared key/value list for joint
# attention, and per-query masks keep each token's own top-k membership)
# ---------------------------------------------------------------------------


def dsa_pack(idx: np.ndarray, group: int, L: int):
    """Shared lists and masks of groups of `group` consecutive query rows.

    Reading of the abstract's one sentence: group g holds rows
    [g*group, (g+1)*group); its shared list is the set union of the valid keys
    (0 <= s < L) those rows selected, in ascending key order; entry j of the
    list carries a mask whose bit i is set exactly when row g*group + i
    selected that key.  The list and masks are padded to group*k entries with
    -1 and 0.

    Returns (shared [G, group*k] int32, masks [G, group*k] uint32,
    lens [G] int32).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    ng = (T + group - 1) // group
    cap = group * k
    shared = np.full((ng, cap), -1, dtype=np.int32)
    masks = np.zeros((ng, cap), dtype=np.uint32)
    lens = np.zeros(ng, dtype=np.int32)
    for g in range(ng):
        rows = [set(int(s) for s in r if 0 <= s < L) for r in idx[g * group:(g + 1) * group]]
        union = sorted(set().union(*rows))
        lens[g] = len(union)
        for j, s in enumerate(union):
            shared[g, j] = s
            masks[g, j] = sum(1 << i for i, r in enumerate(rows) if s in r)
    return shared, masks, lens


def dsa_gather(kv: np.ndarray, shared: np.ndarray, lens: np.ndarray) -> list:
    """The key/value rows of each group's shared list: kv[shared[g, :lens[g]]]."""
    return [kv[shared[g, :lens[g]]] for g in range(len(lens))]
