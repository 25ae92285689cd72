"""Pins for the oracle's attention (CPU only).

Closed forms, a library routine on an equivalent problem, invariants and a
pure-Python brute force, so that a dropped term, a wrong sign or index, or
a transposed operand in the oracle fails at least one of them.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.brute import attention_brute
from tests.oracle_cases import call, make_problem, rope_fn


def _brute(common, row):
    return np.array(attention_brute(
        common["q"].tolist(), row["k_nope"].tolist(), row["v"].tolist(), rope_fn(common),
        [int(x) for x in common["cache_lengths"]], [int(x) for x in common["valid_length"]],
        [int(x) for x in row["cache_row_offsets"]],
        None if row["cache_offsets"] is None else [int(x) for x in row["cache_offsets"]],
        common["scale"]))


BRUTE_CASES = [
    dict(n=[5], p=[0]),
    dict(n=[3, 1, 4], p=[2, 0, 5]),
    dict(n=[0, 6], p=[3, 1]),
    dict(n=[7, 2], p=[0, 9], cap=5),      # several buffer rows, keys split across rows
    dict(n=[1], p=[0]),
]


@pytest.mark.parametrize("case", range(len(BRUTE_CASES)))
def test_oracle_matches_brute_force(case):
    kw = dict(BRUTE_CASES[case])
    rng = np.random.default_rng(case)
    common, rows, _ = make_problem(rng, heads=2, **kw)
    for row in rows:
        got = call(oracle, common, row)
        ref = _brute(common, row)
        assert np.abs(got - ref).max() <= 1e-12


def _causal_mean(common, meta):
    """Mean of V over each query's visible keys (single buffer row), via cumulative sums."""
    outs = []
    for b in range(len(meta["n"])):
        V = meta["v_seq"][b]                     # [L, H, 128] by cache position
        csum = np.cumsum(V, axis=0)
        for i in range(int(meta["n"][b])):
            qpos = int(meta["p"][b]) + i
            outs.append(csum[qpos] / (qpos + 1))
    return np.stack(outs) if outs else np.zeros((0,) + meta["v_seq"][0].shape[1:])


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(11)
    n, p = [6, 3, 5], [0, 4, 2]
    q = np.zeros((14, 3, 192))
    common, rows, meta = make_problem(rng, n, p, heads=3, q=q)
    got = call(oracle, common, rows[0])
    assert np.abs(got - _causal_mean(common, meta)).max() <= 1e-12


def test_zero_scale_gives_mean_of_visible_values():
    rng = np.random.default_rng(12)
    common, rows, meta = make_problem(rng, [4, 5], [3, 0], heads=2)
    common["scale"] = 0.0
    got = call(oracle, common, rows[0])
    assert np.abs(got - _causal_mean(common, meta)).max() <= 1e-12


def test_first_new_token_without_prefix_returns_first_value():
    rng = np.random.default_rng(13)
    common, rows, meta = make_problem(rng, [5, 1, 3], [0, 0, 0], heads=2)
    got = call(oracle, common, rows[0])
    vl = common["valid_length"]
    for b in range(3):
        assert np.array_equal(got[vl[b]], meta["v_seq"][b][0])


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(14)
    common, rows, _ = make_problem(rng, [4, 6], [2, 1], heads=2)
    row = dict(rows[0])
    row["v"] = np.full_like(row["v"], 0.375)
    got = call(oracle, common, row)
    assert np.abs(got - 0.375).max() <= 1e-15


def test_two_token_closed_form():
    """One head, two new tokens, scores chosen so softmax weights are e^0 : e^2."""
    rng = np.random.default_rng(15)
    q = np.zeros((2, 1, 192))
    common, rows, meta = make_problem(rng, [2], [0], heads=1, q=q, width=64, rope_col=0, page_size=2, perm=False)
    row = dict(rows[0])
    kn = np.zeros_like(row["k_nope"])
    common["cache"][...] = 0.0
    common["cache"][0, 0, 1, 0, 5] = 1.0      # K_rope of position 1 = e_5
    common["q"][1, 0, 128 + 5] = 2.0 / common["scale"]   # q_rope . K_rope(1) * scale = 2
    row["k_nope"] = kn
    got = call(oracle, common, row)
    w1 = np.exp(2.0) / (1.0 + np.exp(2.0))
    V = row["v"][:, 0, :]
    assert np.abs(got[0, 0] - V[0]).max() == 0.0
    assert np.abs(got[1, 0] - ((1 - w1) * V[0] + w1 * V[1])).max() <= 1e-14


def test_concatenated_rope_equals_standard_attention():
    """Appending the shared K_rope to every head's K_nope gives ordinary 192-dim
    attention; torch's scaled_dot_product_attention computes that here."""
    rng = np.random.default_rng(16)
    n, p = [7, 4, 9], [3, 0, 6]
    common, rows, meta = make_problem(rng, n, p, heads=3)
    got = call(oracle, common, rows[0])
    vl = common["valid_length"]
    rope = rope_fn(common)
    for b in range(3):
        L = int(meta["L"][b])
        kr = np.array([rope(b, pos) for pos in range(L)])                      # [L, 64]
        kfull = np.concatenate([meta["kn_seq"][b], np.broadcast_to(kr[:, None, :], (L, 3, 64))], axis=2)
        qb = common["q"][vl[b]:vl[b + 1]]                                      # [n, H, 192]
        qpos = p[b] + np.arange(n[b])
        mask = torch.from_numpy(np.arange(L)[None, :] <= qpos[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qb).permute(1, 0, 2), torch.from_numpy(kfull).permute(1, 0, 2).contiguous(),
            torch.from_numpy(meta["v_seq"][b]).permute(1, 0, 2).contiguous(), attn_mask=mask,
            scale=float(common["scale"])).permute(1, 0, 2).numpy()
        assert np.abs(got[vl[b]:vl[b + 1]] - ref).max() <= 1e-12


def test_prefix_consistency():
    """P cached + N new tokens == the last N rows of P+N new tokens with no prefix."""
    rng = np.random.default_rng(17)
    P, N = 6, 5
    common_a, rows_a, meta_a = make_problem(rng, [P + N], [0], heads=2, perm=False)
    common_b = dict(common_a)
    common_b["q"] = common_a["q"][P:]
    common_b["cache_lengths"] = np.array([P], dtype=np.uint32)
    common_b["valid_length"] = np.array([0, N], dtype=np.uint32)
    a = call(oracle, common_a, rows_a[0])
    b = call(oracle, common_b, rows_a[0])
    assert np.abs(a[P:] - b).max() <= 1e-14


def test_page_permutation_invariance():
    n, p = [5, 3], [6, 2]
    a_common, a_rows, _ = make_problem(np.random.default_rng(18), n, p, heads=2, perm=False)
    b_common, b_rows, _ = make_problem(np.random.default_rng(18), n, p, heads=2, perm=False)
    # move every physical page to a new slot and fix the page table accordingly
    npages = a_common["cache"].shape[1]
    perm = np.random.default_rng(99).permutation(npages)
    b_common["cache"] = np.empty_like(a_common["cache"])
    b_common["cache"][:, perm] = a_common["cache"]
    b_common["page_table"] = perm[a_common["page_table"]].astype(np.uint32)
    a = call(oracle, a_common, a_rows[0])
    b = call(oracle, b_common, b_rows[0])
    assert np.array_equal(a, b)


def test_head_and_batch_independence():
    rng = np.random.default_rng(19)
    n, p = [4, 5], [2, 3]
    common, rows, meta = make_problem(rng, n, p, heads=3)
    full = call(oracle, common, rows[0])
    # one head at a time
    for h in range(3):
        c1 = dict(common, q=common["q"][:, h:h + 1])
        r1 = dict(rows[0], k_nope=rows[0]["k_nope"][:, h:h + 1], v=rows[0]["v"][:, h:h + 1])
        assert np.array_equal(call(oracle, c1, r1)[:, 0], full[:, h])
    # the second sequence alone
    vl = common["valid_length"]
    bro = rows[0]["cache_row_offsets"]
    c2 = dict(common, q=common["q"][vl[1]:], valid_length=np.array([0, n[1]], dtype=np.uint32),
              cache_lengths=common["cache_lengths"][1:], page_table=common["page_table"][1:])
    r2 = dict(rows[0], k_nope=rows[0]["k_nope"][bro[1]:], v=rows[0]["v"][bro[1]:],
              cache_row_offsets=np.array([0, bro[2] - bro[1]], dtype=np.uint32), cache_offsets=None)
    assert np.abs(call(oracle, c2, r2) - full[vl[1]:]).max() <= 1e-14


def test_query_with_no_visible_key_is_zero():
    """With several buffer rows, a row may hold only keys later than a query."""
    rng = np.random.default_rng(20)
    common, rows, _ = make_problem(rng, [6], [0], heads=1, cap=3)
    second = call(oracle, common, rows[1])      # keys at positions 3..5
    assert np.array_equal(second[:3], np.zeros((3, 1, 128)))
    assert np.abs(second[3:]).max() > 0


def test_sampled_rows_match_full_output():
    rng = np.random.default_rng(21)
    common, rows, _ = make_problem(rng, [5, 0, 7], [1, 2, 3], heads=2, cap=6)
    for row in rows:
        full = call(oracle, common, row)
        picks = [(0, 1), (4, 0), (5, 1), (11, 0)]
        got = oracle.mla_prefill_rows(picks, common["q"], row["k_nope"], row["v"], common["cache"], 0,
                                      common["page_table"], common["page_size"], common["rope_col"],
                                      common["cache_lengths"], common["valid_length"],
                                      row["cache_row_offsets"], row["cache_offsets"], common["scale"])
        for k, (t, h) in enumerate(picks):
            assert np.abs(got[k] - full[t, h]).max() <= 1e-14
