"""LiteDSA packing on the GPU (LiteTopK pages, arXiv abstract: neighbouring
queries' candidates packed into one shared key/value list, per-query masks
keeping each query's own top-k membership): lists, masks and lengths
bit-identical to the oracle's, and the gathered key/value rows equal to the
oracle's gather."""
import numpy as np
import pytest

from tests.gpu_util import say
from workloads import indexer_inputs, selection_rows

pytestmark = pytest.mark.gpu


def _check_pack(lib, idx_np, L, G, groups=None):
    import torch
    from oracle import dsa_pack
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).cuda()
    sh, m, n = (x.cpu().numpy() for x in lib.dsa_pack(idx, L, G))
    ng = -(-idx_np.shape[0] // G)
    assert sh.shape == (ng, G * idx_np.shape[1]) and m.shape == sh.shape and n.shape == (ng,)
    groups = range(ng) if groups is None else groups
    for g in groups:
        rsh, rm, rn = dsa_pack(idx_np[g * G:(g + 1) * G], G, L)
        assert n[g] == rn[0], (g, n[g], rn[0])
        assert np.array_equal(sh[g], rsh[0]), g
        assert np.array_equal(m[g].view(np.uint32), rm[0]), g
    return sh, m, n


CASES = [
    # (T, k, L, G, invalid fraction)
    (7, 5, 40, 3, 0.1),
    (5, 300, 1 << 26, 7, 0.0),          # the largest key range
    (64, 256, 5000, 16, 0.02),
    (33, 1024, 100000, 32, 0.0),        # 32 rows per mask, ragged last group
    (10, 2048, 1 << 20, 16, 0.0),       # 32,768 entries: the largest group
    (9, 100, 700, 1, 0.05),             # one row per group
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c[0]}_k{c[1]}_L{c[2]}_G{c[3]}")
def test_dsa_pack_vs_oracle(lib, case):
    T, k, L, G, bad = case
    say("dsa", case)
    rows = selection_rows(T, k, L, tag=71, invalid=bad)
    if bad:   # entries past the key range are not keys either
        rows[np.random.default_rng(3).random(rows.shape) < bad / 2] = L + 5
    _check_pack(lib, rows, L, G)


def test_dsa_pack_of_exact_topk(lib):
    """The oracle's own top-k of a small indexer chunk, packed in groups of 8."""
    from oracle import oracle_indexer
    inp = indexer_inputs(40, 3000, 64, 128, "bf16", 128, 200, drift=True, tag=72)
    idx, _ = oracle_indexer(inp)
    sh, m, n = _check_pack(lib, idx, inp["L"], 8)
    say("  union sizes", n.tolist(), "of", 8 * 128)


def test_dsa_pack_duplicates_and_empty_rows(lib):
    rows = np.full((6, 8), -1, np.int32)
    rows[0] = [3, 3, 3, 1, 1, -1, 7, 3]        # repeated keys within a row
    rows[2] = [5, 6, 7, 8, 9, 10, 11, 12]
    rows[5] = [0, 0, 0, 0, 0, 0, 0, 0]
    _check_pack(lib, rows, 20, 4)


def test_dsa_pack_union_past_hash_table(lib):
    """Groups with more distinct keys than half the LDS hash table's 16,384
    slots are packed by sorting every selection: uniformly drawn rows give
    about 32,000 distinct keys per group of 16, beside groups of heavily
    shared rows, and a group just below and just above the switch.  The last
    group's keys crowd one key-range bucket (3,000 keys near 0 and one near
    2^26), which sends its distinct keys to the bitonic sort."""
    rng = np.random.default_rng(75)
    k, G = 2048, 16
    rows = rng.integers(0, 1 << 26, (6 * G, k), dtype=np.int64).astype(np.int32)
    rows[G:2 * G] = rng.integers(0, 3000, (G, k))                    # about 3,000 distinct
    rows[5 * G:] = rng.integers(0, 3000, (G, k))
    rows[5 * G + 7, 100] = (1 << 26) - 1
    for g, n_distinct in ((2, 8100), (3, 8200)):                      # either side of 8,192
        pool = rng.choice(1 << 24, n_distinct, replace=False)
        blk = rng.choice(pool, (G, k))
        blk.reshape(-1)[:n_distinct] = pool                           # every pool key appears
        rows[g * G:(g + 1) * G] = blk
    sh, m, n = _check_pack(lib, rows, 1 << 26, G)
    say("  union sizes", n.tolist())
    assert n[2] == 8100 and n[3] == 8200 and n[5] == len(np.unique(rows[5 * G:]))


def test_dsa_full_size_sampled_groups(lib):
    """A 1M-context chunk of 8,192 queries with k = 2,048 in groups of 16:
    32 groups checked against the oracle, spread over the chunk."""
    T, k, L, G = 8192, 2048, 1 << 20, 16
    rows = selection_rows(T, k, L, tag=73)
    ng = T // G
    _check_pack(lib, rows, L, G, groups=list(range(0, ng, ng // 31))[:31] + [ng - 1])


def test_dsa_gather_vs_oracle(lib):
    import torch
    from oracle import dsa_gather, dsa_pack
    T, k, L, G = 24, 64, 5000, 8
    rows = selection_rows(T, k, L, tag=74, invalid=0.05)
    kv = torch.randint(-2 ** 31, 2 ** 31 - 1, (L, 288), dtype=torch.int32, device="cuda")   # 1,152-byte rows
    sh, m, n = lib.dsa_pack(torch.from_numpy(rows).cuda(), L, G)
    out = lib.dsa_gather(kv, sh, n)
    rsh, _, rn = dsa_pack(rows, G, L)
    ref = dsa_gather(kv.cpu().numpy(), rsh, rn)
    got = out.cpu().numpy()
    for g in range(len(rn)):
        assert np.array_equal(got[g, :rn[g]], ref[g]), g
