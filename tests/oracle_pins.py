"""Pins of the CPU oracle against facts other than itself.

Each ``check_*`` takes the oracle module (so that the mutation tests can hand
in a copy with a planted mistake) and raises AssertionError on a mismatch.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _row_input(q, w, keys, pos, k):
    """A one-query fp32 indexer input dict around explicit values."""
    q = np.asarray(q, np.float32)[None]
    keys = np.asarray(keys, np.float32)
    return dict(kind="indexer", T=1, L=len(keys), H=q.shape[1], D=q.shape[2], dtype="f32", topk=k,
                q=q, k=keys, q_scale=None, k_scale=None, w=np.asarray(w, np.float32)[None],
                pos=np.array([pos], np.int32))


# --------------------------------------------------------------------------- scores


def check_hand_example(O):
    """Hand-derived scores and top-k sets (tests/golden/indexer_hand.json)."""
    g = _load("indexer_hand.json")
    q, w, keys = (np.array(g[x], np.float64) for x in ("q", "w", "keys"))
    s = O.indexer_scores(q, w, keys)
    assert np.array_equal(s, np.array(g["scores"])), (s, g["scores"])
    for c in g["cases"]:
        inp = _row_input(g["q"], g["w"], g["keys"], c["pos"], c["k"])
        idx, _ = O.oracle_indexer(inp)
        assert idx[0].tolist() == c["idx"], (c, idx[0].tolist())


def check_relu_identities(O, seed=1):
    """ReLU(x) - ReLU(-x) = x and ReLU(x) + ReLU(-x) = |x|, summed over heads.

    I(q) - I(-q) = (sum_h w_h q_h) . k is a single mat-vec that never applies a
    ReLU, and I(q) + I(-q) = sum_h w_h |q_h . k|; together they fix I(q).
    """
    g = np.random.default_rng(seed)
    H, D, n = 5, 7, 33
    q = g.standard_normal((H, D))
    w = g.uniform(0.1, 1.0, H)
    keys = g.standard_normal((n, D))
    a, b = O.indexer_scores(q, w, keys), O.indexer_scores(-q, w, keys)
    lin = keys @ (w @ q)
    absum = np.abs(np.einsum("nd,hd->nh", keys, q)) @ w
    assert np.allclose(a - b, lin, rtol=1e-12, atol=1e-12)
    assert np.allclose(a + b, absum, rtol=1e-12, atol=1e-12)
    assert np.all(a >= 0)


def check_homogeneity(O, seed=2):
    """Positive homogeneity in q and k, linearity in w, permutation of heads."""
    g = np.random.default_rng(seed)
    H, D, n = 4, 6, 20
    q, keys = g.standard_normal((H, D)), g.standard_normal((n, D))
    w1, w2 = g.uniform(0, 1, H), g.uniform(0, 1, H)
    s = O.indexer_scores(q, w1, keys)
    assert np.allclose(O.indexer_scores(2.5 * q, w1, keys), 2.5 * s, rtol=1e-12)
    assert np.allclose(O.indexer_scores(q, w1, 0.25 * keys), 0.25 * s, rtol=1e-12)
    assert np.allclose(O.indexer_scores(q, w1 + w2, keys), s + O.indexer_scores(q, w2, keys), rtol=1e-12)
    p = g.permutation(H)
    assert np.allclose(O.indexer_scores(q[p], w1[p], keys), s, rtol=1e-12)


def check_gemm_special_case(O, seed=3):
    """H = 1, w = 1 and non-negative q, k: the ReLU never fires and I = K q."""
    g = np.random.default_rng(seed)
    D, n = 16, 50
    q = np.abs(g.standard_normal((1, D)))
    keys = np.abs(g.standard_normal((n, D)))
    s = O.indexer_scores(q, np.ones(1), keys)
    assert np.allclose(s, np.matmul(keys, q[0]), rtol=1e-13)


def check_fp8_scale_factorisation(O, seed=4):
    """fp8 with per-token scales: I = sigma_q * sigma_k-weighted unscaled score.

    For one key, scaling that key by sigma_k scales its score by sigma_k (the
    decode of a scaled e4m3fn tensor must apply the scale per token, not per
    element or per tensor).
    """
    g = np.random.default_rng(seed)
    T, H, D, L = 3, 4, 8, 12
    q8 = g.integers(0, 0x7E, size=(T, H, D), dtype=np.uint8) | (g.integers(0, 2, size=(T, H, D), dtype=np.uint8) << 7)
    k8 = g.integers(0, 0x7E, size=(L, D), dtype=np.uint8) | (g.integers(0, 2, size=(L, D), dtype=np.uint8) << 7)
    sq = g.uniform(0.5, 2, T).astype(np.float32)
    sk = g.uniform(0.5, 2, L).astype(np.float32)
    w = g.uniform(0, 1, (T, H)).astype(np.float32)
    inp = dict(kind="indexer", T=T, L=L, H=H, D=D, dtype="fp8", topk=4, q=q8, k=k8, q_scale=sq, k_scale=sk,
               w=w, pos=np.full(T, L - 1, np.int32))
    tab = O.e4m3fn_table()
    for t in range(T):
        _, s = O.indexer_row_scores(inp, t)
        ref = np.array([float(sq[t]) * float(sk[j]) * O.indexer_scores(tab[q8[t]], w[t].astype(np.float64), tab[k8[j]][None])[0]
                        for j in range(L)])
        assert np.allclose(s, ref, rtol=1e-12), (s, ref)


# --------------------------------------------------------------------------- decoding


def check_e4m3fn_points(O):
    """Code points fixed by the OCP FP8 E4M3 definition (tests/golden/e4m3fn_points.json)."""
    tab = O.e4m3fn_table()
    for code, val in _load("e4m3fn_points.json")["points"].items():
        c = int(code, 16)
        if val is None:
            assert np.isnan(tab[c]), code
        else:
            assert tab[c] == float(val) and np.signbit(tab[c]) == (c >= 0x80), (code, tab[c], val)


def check_e4m3fn_vs_torch(O):
    """All 256 codes against torch's float8_e4m3fn -> float32 conversion."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    tab = O.e4m3fn_table()
    both_nan = np.isnan(ref) & np.isnan(tab)
    assert np.array_equal(tab[~both_nan], ref[~both_nan]) and np.array_equal(np.isnan(ref), np.isnan(tab))


def check_bf16_vs_torch(O, seed=5):
    import torch
    g = np.random.default_rng(seed)
    x = torch.from_numpy((g.standard_normal(1000) * 10 ** g.uniform(-30, 30, 1000)).astype(np.float32))
    b = x.to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_to_f64(bits), b.to(torch.float32).numpy().astype(np.float64))


# --------------------------------------------------------------------------- selection


def _brute_rank_select(scores, k):
    """Key i is selected iff fewer than k keys beat it under (score desc, index asc)."""
    n = len(scores)
    sel = []
    for i in range(n):
        beats = sum(1 for j in range(n) if scores[j] > scores[i] or (scores[j] == scores[i] and j < i))
        if beats < k:
            sel.append(i)
    return sel


def check_brute_force_ranks(O, seed=6, trials=60):
    g = np.random.default_rng(seed)
    for _ in range(trials):
        n = int(g.integers(1, 40))
        k = int(g.integers(1, 45))
        s = g.integers(-3, 4, n).astype(np.float64)           # many ties on purpose
        idx, sc = O.topk_row(s, np.arange(n), k)
        got = sorted(int(i) for i in idx if i >= 0)
        assert got == _brute_rank_select(s, k), (s, k, got)
        m = min(k, n)
        assert np.all(idx[m:] == -1) and np.all(idx[:m] >= 0)
        # returned in rank order
        assert list(idx[:m]) == sorted(idx[:m], key=lambda i: (-s[i], i))


def check_exhaustive_subsets(O, seed=7, trials=25):
    """For n <= 10, exactly one k-subset dominates its complement; it is the oracle's."""
    g = np.random.default_rng(seed)
    for _ in range(trials):
        n = int(g.integers(1, 11))
        k = int(g.integers(1, n + 1))
        s = g.integers(0, 3, n).astype(np.float64)
        winners = []
        for S in itertools.combinations(range(n), k):
            out = [j for j in range(n) if j not in S]
            if all(s[i] > s[j] or (s[i] == s[j] and i < j) for i in S for j in out):
                winners.append(set(S))
        assert len(winners) == 1
        idx, _ = O.topk_row(s, np.arange(n), k)
        assert set(int(i) for i in idx) == winners[0]


def check_selection_special_cases(O, seed=8):
    g = np.random.default_rng(seed)
    s = g.integers(0, 5, 100).astype(np.float64)
    idx, _ = O.topk_row(s, np.arange(100), 1)
    assert idx[0] == np.argmax(s)                             # argmax returns the first maximum
    idx, _ = O.topk_row(np.full(50, 7.0), np.arange(50), 10)
    assert idx.tolist() == list(range(10))                    # all equal -> lowest indices
    s = g.standard_normal(30)
    idx, _ = O.topk_row(s, np.arange(30), 40)
    assert sorted(idx[:30].tolist()) == list(range(30)) and np.all(idx[30:] == -1)
    s = g.standard_normal(200)                                # no ties: agrees with argpartition
    idx, _ = O.topk_row(s, np.arange(200), 17)
    assert set(idx.tolist()) == set(np.argpartition(-s, 17)[:17].tolist())


def check_invariant_on_workload(O, inp, rows):
    """Every selected score >= every unselected one; ties go to the lower index."""
    for t in rows:
        v, s = O.indexer_row_scores(inp, int(t))
        idx, sc = O.topk_row(s, v, inp["topk"])
        chosen = idx[idx >= 0]
        mask = np.zeros(len(v), bool)
        mask[chosen] = True
        if mask.all() or len(chosen) == 0:
            continue
        lo = s[mask].min()
        hi = s[~mask].max()
        assert lo >= hi
        if lo == hi:
            assert v[mask][s[mask] == lo].max() < v[~mask][s[~mask] == hi].min()


def check_causal(O, seed=9):
    """Keys after the query position never appear; positions clamp to the context."""
    g = np.random.default_rng(seed)
    H, D, L = 2, 4, 30
    q = g.standard_normal((H, D))
    keys = g.standard_normal((L, D))
    w = np.ones(H)
    for pos in (-1, 0, 5, 29, 100):
        inp = _row_input(q, w, keys, pos, 8)
        idx, _ = O.oracle_indexer(inp)
        nvalid = max(0, min(pos, L - 1) + 1)
        chosen = idx[0][idx[0] >= 0]
        assert len(chosen) == min(8, nvalid) and np.all(chosen <= min(pos, L - 1))


# --------------------------------------------------------------------------- retrieval


def check_retrieval_self_match(O, seed=10):
    """A database holding each query itself returns it first (Cauchy-Schwarz on unit rows)."""
    g = np.random.default_rng(seed)
    import torch
    N, D, T = 300, 24, 6
    x = g.standard_normal((N, D))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    bits = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rows = g.choice(N, T, replace=False)
    idx, sc = O.oracle_retrieval(bits[rows], bits, 5, block=37)
    assert idx[:, 0].tolist() == rows.tolist()
    xd = O.bf16_to_f64(bits)
    assert np.allclose(sc[:, 0], (xd[rows] ** 2).sum(1), rtol=1e-12)
    # block size does not change anything
    idx2, sc2 = O.oracle_retrieval(bits[rows], bits, 5, block=1 << 18)
    assert np.array_equal(idx, idx2) and np.array_equal(sc, sc2)


def check_retrieval_row_scores_closed_form(O):
    """Scores of one query against a database of scaled basis vectors: row s is
    c_s times unit vector e_{(7 s) mod D}, so its inner product with q is
    c_s * q[(7 s) mod D] exactly.  Every value is a small dyadic number, exact
    in bf16 and fp64.  The block size (5) does not divide N (23), so a block
    written at the wrong offset or a transposed operand changes the result."""
    import torch
    N, D = 23, 16
    c = np.array([(s % 9) - 4 + 0.5 * (s % 2) for s in range(N)], np.float32)
    x = np.zeros((N, D), np.float32)
    for s in range(N):
        x[s, (7 * s) % D] = c[s]
    q = np.array([[(d - 7) * 0.25 for d in range(D)], [1.0 + d for d in range(D)]], np.float32)

    def bits(a):
        return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    xb, qb = bits(x), bits(q)
    refs = [np.array([float(c[s]) * float(q[t, (7 * s) % D]) for s in range(N)]) for t in range(2)]
    for blk in (5, 1 << 18):
        for t in range(2):
            got = O.retrieval_row_scores(qb, xb, t, block=blk)
            assert got.shape == (N,) and np.array_equal(got, refs[t]), (t, blk, got, refs[t])
        # several queries in one call: one row of scores per query, in the order asked
        got = O.retrieval_row_scores(qb, xb, [1, 0, 0], block=blk)
        assert got.shape == (3, N), got.shape
        for i, t in enumerate([1, 0, 0]):
            assert np.array_equal(got[i], refs[t]), (i, t, blk)


def check_retrieval_row_scores_self_match(O, seed=13):
    """Unit rows, query = a database row: by Cauchy-Schwarz that row scores
    highest, with its squared norm; queries sit in every block of a block size
    that does not divide N."""
    import torch
    g = np.random.default_rng(seed)
    N, D, blk = 101, 12, 17
    x = g.standard_normal((N, D))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    bits = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xd = O.bf16_to_f64(bits)
    for r in (0, 16, 17, 50, 99, 100):
        s = O.retrieval_row_scores(bits[r:r + 1], bits, 0, block=blk)
        assert int(np.argmax(s)) == r
        assert np.isclose(s[r], (xd[r] ** 2).sum(), rtol=1e-12)


# --------------------------------------------------------------------------- sample carried to the next chunk


def check_next_sample_hand_example(O):
    """Hand-derived count ranking with ties, padding and entries that are not
    keys (tests/golden/next_sample_hand.json)."""
    g = _load("next_sample_hand.json")
    prev = np.array(g["prev_idx"], np.int32)
    for c in g["cases"]:
        got = O.next_sample(prev, g["L"], c["n"])
        assert got.tolist() == c["sample"], (c, got.tolist())


def _brute_next_sample(prev, L, n):
    """Key s is taken iff fewer than n keys beat it, where key a beats key b
    when it was selected more often, or as often with a lower index; counts
    ignore entries outside [0, L)."""
    counts = [0] * L
    for row in prev:
        for s in row:
            if 0 <= int(s) < L:
                counts[int(s)] += 1
    taken = []
    for s in range(L):
        beats = sum(1 for a in range(L) if counts[a] > counts[s] or (counts[a] == counts[s] and a < s))
        if beats < n:
            taken.append(s)
    return taken, counts


def check_next_sample_brute_force(O, seed=14, trials=40):
    """Brute-force ranks on small inputs full of ties, -1 padding and entries
    past the key range; the oracle returns the taken keys in rank order."""
    g = np.random.default_rng(seed)
    for _ in range(trials):
        L = int(g.integers(1, 30))
        T, k = int(g.integers(0, 8)), int(g.integers(1, 7))
        prev = g.integers(-2, L + 3, size=(T, k)).astype(np.int32)
        n = int(g.integers(1, L + 1))
        taken, counts = _brute_next_sample(prev, L, n)
        got = O.next_sample(prev, L, n)
        assert sorted(got.tolist()) == taken, (prev, L, n, got)
        assert got.tolist() == sorted(taken, key=lambda s: (-counts[s], s))


# --------------------------------------------------------------------------- identical keys


def check_first_copy_brute_force(O, seed=15):
    """first_copy against a dictionary from each row's bytes (and scale) to the
    first index holding them, on small arrays full of repeated rows."""
    g = np.random.default_rng(seed)
    for dt, D in ((np.uint8, 5), (np.uint8, 16), (np.uint16, 3), (np.float32, 4)):
        for with_scale in (False, True):
            n = int(g.integers(1, 60))
            src = g.integers(0, 7, size=(8, D)).astype(dt)
            raw = src[g.integers(0, 8, size=n)]
            sc = g.integers(1, 3, size=n).astype(np.float32) if with_scale else None
            first = {}
            want = []
            for r in range(n):
                key = raw[r].tobytes() + (sc[r].tobytes() if with_scale else b"")
                want.append(first.setdefault(key, r))
            got = O.first_copy(raw, sc)
            assert got.tolist() == want, (dt, D, with_scale, got, want)


def check_identical_keys_tie(O):
    """Bit-identical key rows score bit-identically, so a tie group cut by the
    k-th score gives its lowest key indices, whatever rounding path a blocked
    product would take for each copy."""
    from tests.tie_cases import tied_indexer_inputs
    inp = tied_indexer_inputs(16, 6000, 64, 128, "bf16", 200, 37, tag=4)
    k = inp["topk"]
    keys = O.key_table(inp)
    src = inp["src_of_key"]
    for t in range(inp["T"]):
        v, s = O.indexer_row_scores(inp, t, keys)
        for u in np.unique(src[: len(v)]):
            grp = s[src[: len(v)] == u]
            assert np.all(grp == grp[0]), (t, u)
        idx, _ = O.topk_row(s, v, k)
        vk = np.sort(s)[::-1][k - 1]
        need = k - int((s > vk).sum())
        want = set(v[s > vk].tolist()) | set(v[s == vk][:need].tolist())
        assert set(idx.tolist()) == want, t


# --------------------------------------------------------------------------- LiteDSA packing


def _topk_like_rows(rng, T, k, L, n_hot):
    """Rows of k distinct keys drawn mostly from a shared hot set (neighbouring
    queries overlap), with some -1 and out-of-range entries."""
    hot = rng.choice(L, size=min(n_hot, L), replace=False)
    rows = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        n = rng.integers(0, k + 1)
        pool = np.concatenate([hot, rng.choice(L, size=k, replace=False)])
        keys = np.unique(pool)[rng.permutation(len(np.unique(pool)))][:n]
        rows[t, :n] = keys
    flat = rows.ravel()
    bad = rng.random(flat.shape) < 0.02
    flat[bad] = L + rng.integers(0, 5, size=int(bad.sum()))   # not keys
    return rows


def check_dsa_hand_example(O):
    """Hand-derived union, masks and padding (tests/golden/dsa_pack_hand.json)."""
    g = _load("dsa_pack_hand.json")
    sh, m, n = O.dsa_pack(np.array(g["idx"], np.int32), g["group"], g["L"])
    assert np.array_equal(sh, np.array(g["shared"])), sh
    assert np.array_equal(m, np.array(g["masks"], np.uint32)), m
    assert np.array_equal(n, np.array(g["lens"])), n


def check_dsa_membership(O, seed=11):
    """Each query's own selection is exactly the list entries whose mask has its
    bit; lists are strictly ascending, padded, and between the largest row and
    the sum of the rows in size."""
    rng = np.random.default_rng(seed)
    for T, k, L, G in [(7, 5, 40, 3), (16, 8, 100, 8), (33, 6, 64, 32), (5, 4, 9, 1), (12, 16, 30, 5)]:
        idx = _topk_like_rows(rng, T, k, L, n_hot=2 * k)
        sh, m, n = O.dsa_pack(idx, G, L)
        assert sh.shape == (-(-T // G), G * k) and m.shape == sh.shape
        for g in range(len(n)):
            u = sh[g, :n[g]]
            assert np.all(np.diff(u) > 0) and np.all((u >= 0) & (u < L))
            assert np.all(sh[g, n[g]:] == -1) and np.all(m[g, n[g]:] == 0)
            rows = idx[g * G:(g + 1) * G]
            sets = [set(int(x) for x in r if 0 <= x < L) for r in rows]
            assert max(len(s) for s in sets) <= n[g] <= sum(len(s) for s in sets)
            for i, s in enumerate(sets):
                got = set(int(x) for x in u[(m[g, :n[g]] >> np.uint32(i)) & 1 == 1])
                assert got == s, (g, i)
            assert np.all(m[g, :n[g]] >> np.uint32(len(sets)) == 0)   # no bits for missing rows
            assert np.all(m[g, :n[g]] != 0)


def check_dsa_special_cases(O):
    """Group of one: the sorted row, every mask 1.  Identical rows: one copy,
    every row's bit.  No keys: empty lists."""
    row = np.array([[9, 2, 5, -1, 7]], np.int32)
    sh, m, n = O.dsa_pack(row, 1, 10)
    assert n[0] == 4 and list(sh[0, :4]) == [2, 5, 7, 9] and np.all(m[0, :4] == 1)
    same = np.tile(np.array([[4, 0, 3]], np.int32), (5, 1))
    sh, m, n = O.dsa_pack(same, 5, 6)
    assert n[0] == 3 and list(sh[0, :3]) == [0, 3, 4] and np.all(m[0, :3] == 0b11111)
    sh, m, n = O.dsa_pack(np.full((4, 3), -1, np.int32), 2, 6)
    assert np.all(n == 0) and np.all(sh == -1) and np.all(m == 0)


def check_dsa_joint_attention(O, seed=12):
    """What the packing is for: attention of each query over its group's shared
    list, restricted by its mask, equals attention over its own selection
    (softmax of q.k over the selected keys, weighted sum of their values)."""
    rng = np.random.default_rng(seed)
    T, k, L, G, D = 10, 6, 50, 4, 8
    idx = _topk_like_rows(rng, T, k, L, n_hot=8)
    K, V, Q = rng.standard_normal((L, D)), rng.standard_normal((L, D)), rng.standard_normal((T, D))
    sh, m, n = O.dsa_pack(idx, G, L)
    kv = O.dsa_gather(np.concatenate([K, V], axis=1), sh, n)
    for t in range(T):
        own = np.array(sorted(set(int(x) for x in idx[t] if 0 <= x < L)), dtype=np.int64)
        if len(own) == 0:
            continue
        s = K[own] @ Q[t]
        ref = np.exp(s - s.max()) @ V[own] / np.exp(s - s.max()).sum()
        g, i = divmod(t, G)
        keep = (m[g, :n[g]] >> np.uint32(i)) & 1 == 1
        Kg, Vg = kv[g][:, :D], kv[g][:, D:]
        s2 = np.where(keep, Kg @ Q[t], -np.inf)
        e = np.exp(s2 - s2[keep].max())
        got = e @ Vg / e.sum()
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), t
        assert np.array_equal(kv[g], np.concatenate([K, V], axis=1)[sh[g, :n[g]]])


ALL_CHECKS = [
    check_dsa_hand_example,
    check_dsa_membership,
    check_dsa_special_cases,
    check_dsa_joint_attention,
    check_hand_example, check_relu_identities, check_homogeneity, check_gemm_special_case,
    check_fp8_scale_factorisation, check_e4m3fn_points, check_e4m3fn_vs_torch, check_bf16_vs_torch,
    check_brute_force_ranks, check_exhaustive_subsets, check_selection_special_cases, check_causal,
    check_retrieval_self_match, check_retrieval_row_scores_closed_form, check_retrieval_row_scores_self_match,
    check_next_sample_hand_example, check_next_sample_brute_force,
    check_first_copy_brute_force, check_identical_keys_tie,
]
