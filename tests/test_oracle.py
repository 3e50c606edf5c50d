"""The CPU oracle against facts other than itself, plus planted-mistake checks."""
import importlib.util
import os

import numpy as np
import pytest

import oracle as O
from tests import oracle_pins as P
from workloads import indexer_inputs, indexer_workload


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(O)


def test_invariant_tiny_workload():
    inp = indexer_workload("tiny-4k-fp32")
    P.check_invariant_on_workload(O, inp, range(inp["T"]))


def test_invariant_small_bf16_fp8():
    for dt in ("bf16", "fp8"):
        inp = indexer_inputs(16, 700, 8, 32, dt, 50, 40, drift=True, tag=11)
        P.check_invariant_on_workload(O, inp, range(16))


def test_oracle_rows_subset_consistent():
    inp = indexer_workload("tiny-4k-fp32")
    full, _ = O.oracle_indexer(inp)
    rows = [3, 17, 63]
    part, _ = O.oracle_indexer(inp, rows=rows)
    assert np.array_equal(full[rows], part)


# --------------------------------------------------------------------------- planted mistakes

ORACLE_PY = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.py")


def _fresh_oracle():
    spec = importlib.util.spec_from_file_location("oracle_mutant", ORACLE_PY)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _no_relu(m):
    m.indexer_scores = lambda q, w, keys: (keys @ q.T) @ w


def _ties_high(m):
    orig = m.topk_row

    def topk_row(scores, idx, k):
        order = np.lexsort((-np.asarray(idx), -scores))[:k]
        oi = np.full(k, -1, np.int32)
        os_ = np.full(k, np.nan)
        oi[: len(order)] = np.asarray(idx)[order]
        os_[: len(order)] = scores[order]
        return oi, os_
    m.topk_row = topk_row
    assert orig is not topk_row


def _causal_exclusive(m):
    m.valid_keys = lambda pos_t, L: np.arange(0, max(0, min(int(pos_t), L)), dtype=np.int64)


def _fp8_bias8(m):
    orig = m.e4m3fn_table

    def tab():
        t = orig()
        return t / 2.0
    m.e4m3fn_table = tab


def _fp8_scale_per_tensor(m):
    orig = m.decode

    def decode(raw, dtype, scale=None):
        if dtype == "fp8" and scale is not None:
            return orig(raw, dtype, None) * float(np.asarray(scale).reshape(-1)[0])
        return orig(raw, dtype, scale)
    m.decode = decode


def _weights_reversed(m):
    m.indexer_scores = lambda q, w, keys: np.maximum(keys @ q.T, 0.0) @ w[::-1]


def _bf16_shift15(m):
    m.bf16_to_f64 = lambda bits: (np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)


def _transposed_keys(m):
    m.retrieval_scores = lambda q, db: db[:, ::-1] @ q
    m.oracle_retrieval.__globals__["retrieval_scores"] = m.retrieval_scores

    def oracle_retrieval(q_raw, db_raw, k, rows=None, dtype="bf16", block=1 << 18):
        T = q_raw.shape[0]
        rows = np.arange(T) if rows is None else np.asarray(rows)
        qd = m.decode(q_raw[rows], dtype)
        xd = m.decode(db_raw, dtype)
        scores = (xd[:, ::-1] @ qd.T).T
        idx = np.arange(len(xd))
        oi = np.full((len(rows), k), -1, np.int32)
        os_ = np.full((len(rows), k), np.nan)
        for r in range(len(rows)):
            oi[r], os_[r] = m.topk_row(scores[r], idx, k)
        return oi, os_
    m.oracle_retrieval = oracle_retrieval


def _dsa_bits_reversed(m):
    orig = m.dsa_pack

    def dsa_pack(idx, group, L):
        sh, mk, n = orig(idx, group, L)
        rev = np.zeros_like(mk)
        for i in range(group):
            rev |= ((mk >> np.uint32(i)) & np.uint32(1)) << np.uint32(group - 1 - i)
        return sh, rev, n
    m.dsa_pack = dsa_pack


def _dsa_descending(m):
    orig = m.dsa_pack

    def dsa_pack(idx, group, L):
        sh, mk, n = orig(idx, group, L)
        for g in range(len(n)):
            sh[g, :n[g]] = sh[g, :n[g]][::-1].copy()
            mk[g, :n[g]] = mk[g, :n[g]][::-1].copy()
        return sh, mk, n
    m.dsa_pack = dsa_pack


def _ns_ties_high(m):
    def next_sample(prev_idx, L, n):
        p = np.asarray(prev_idx).ravel()
        counts = np.bincount(p[(p >= 0) & (p < L)], minlength=L)
        return np.lexsort((-np.arange(L), -counts))[:n].astype(np.int32)
    m.next_sample = next_sample


def _ns_counts_invalid(m):
    # -1 padding wraps to the last key and entries past the range are clipped onto it
    def next_sample(prev_idx, L, n):
        p = np.asarray(prev_idx).ravel()
        counts = np.bincount(np.clip(p % max(L, 1), 0, L - 1), minlength=L)
        return np.lexsort((np.arange(L), -counts))[:n].astype(np.int32)
    m.next_sample = next_sample


def _rrs_block_offset(m):
    orig = m.retrieval_row_scores

    def retrieval_row_scores(q_raw, db_raw, t, dtype="bf16", block=1 << 18, rep=None):
        out = orig(q_raw, db_raw, t, dtype, block, rep)
        for s0 in range(0, out.shape[-1], block):
            out[..., s0:s0 + block] = np.roll(out[..., s0:s0 + block], 1, axis=-1)
        return out
    m.retrieval_row_scores = retrieval_row_scores


def _rrs_transposed(m):
    def retrieval_row_scores(q_raw, db_raw, t, dtype="bf16", block=1 << 18, rep=None):
        qd = m.decode(q_raw[np.atleast_1d(t)], dtype)
        out = (m.decode(db_raw, dtype)[:, ::-1] @ qd.T).T
        return out if not np.isscalar(t) else out[0]
    m.retrieval_row_scores = retrieval_row_scores


def _rrs_rows_swapped(m):
    # several queries at once: the score rows come back in the wrong order
    orig = m.retrieval_row_scores

    def retrieval_row_scores(q_raw, db_raw, t, dtype="bf16", block=1 << 18, rep=None):
        out = orig(q_raw, db_raw, t, dtype, block, rep)
        return out[::-1].copy() if not np.isscalar(t) else out
    m.retrieval_row_scores = retrieval_row_scores


def _no_first_copy(m):
    m.first_copy = lambda raw, scale=None: np.arange(raw.shape[0], dtype=np.int64)


MUTANTS = {
    "dsa_mask_bits_reversed": (_dsa_bits_reversed, [P.check_dsa_hand_example, P.check_dsa_membership]),
    "dsa_list_descending": (_dsa_descending, [P.check_dsa_hand_example, P.check_dsa_membership]),
    "no_relu": (_no_relu, [P.check_hand_example, P.check_relu_identities]),
    "ties_to_higher_index": (_ties_high, [P.check_brute_force_ranks, P.check_hand_example,
                                           P.check_selection_special_cases]),
    "causal_exclusive": (_causal_exclusive, [P.check_hand_example, P.check_causal]),
    "fp8_wrong_bias": (_fp8_bias8, [P.check_e4m3fn_points, P.check_e4m3fn_vs_torch]),
    "fp8_scale_per_tensor": (_fp8_scale_per_tensor, [P.check_fp8_scale_factorisation]),
    "head_weights_reversed": (_weights_reversed, [P.check_hand_example, P.check_relu_identities]),
    "bf16_wrong_shift": (_bf16_shift15, [P.check_bf16_vs_torch, P.check_retrieval_self_match]),
    "retrieval_transposed": (_transposed_keys, [P.check_retrieval_self_match]),
    "next_sample_ties_to_higher_index": (_ns_ties_high, [P.check_next_sample_hand_example,
                                                         P.check_next_sample_brute_force]),
    "next_sample_counts_invalid_entries": (_ns_counts_invalid, [P.check_next_sample_hand_example,
                                                                P.check_next_sample_brute_force]),
    "retrieval_row_scores_block_offset": (_rrs_block_offset, [P.check_retrieval_row_scores_closed_form,
                                                              P.check_retrieval_row_scores_self_match]),
    "retrieval_row_scores_transposed": (_rrs_transposed, [P.check_retrieval_row_scores_closed_form,
                                                          P.check_retrieval_row_scores_self_match]),
    "retrieval_row_scores_rows_swapped": (_rrs_rows_swapped, [P.check_retrieval_row_scores_closed_form]),
    "identical_keys_scored_apart": (_no_first_copy, [P.check_first_copy_brute_force]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    plant, checks = MUTANTS[name]
    for check in checks:
        m = _fresh_oracle()
        plant(m)
        with pytest.raises(AssertionError):
            check(m)
