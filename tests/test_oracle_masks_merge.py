"""Pins for the oracle's null mask, log-sum-exp output and merge of partial
attentions (CPU only).

The mask predicate is chosen per call, causal or null among others
("mla_prefill_v2_ragged", Args: mask_t and mask_functor).  With several
buffer rows ("generic_flare_mla_prefill_ragged_paged_plan", description and
Args) each row holds part of the keys; the log-sum-exp of a row's scores and
the combine of partials must give back the attention over every key.  Pinned
by a pure-Python brute force, closed forms, invariants, and the identity
"rows merged = one row holding every key", whose right-hand side is the
attention's definition and shares no code with the merge.
"""
import math

import numpy as np
import pytest

import oracle
from tests.brute import attention_brute
from tests.oracle_cases import make_problem, rope_fn


def _call(common, row, mask="causal", lse=False):
    return oracle.mla_prefill_ragged(
        common["q"], row["k_nope"], row["v"], common["cache"], common["layer_idx"], common["page_table"],
        common["page_size"], common["rope_col"], common["cache_lengths"], common["valid_length"],
        row["cache_row_offsets"], row["cache_offsets"], common["scale"], mask=mask, return_lse=lse)


def _brute(common, row, causal):
    out, lse = attention_brute(
        common["q"].tolist(), row["k_nope"].tolist(), row["v"].tolist(), rope_fn(common),
        [int(x) for x in common["cache_lengths"]], [int(x) for x in common["valid_length"]],
        [int(x) for x in row["cache_row_offsets"]],
        None if row["cache_offsets"] is None else [int(x) for x in row["cache_offsets"]],
        common["scale"], causal=causal, with_lse=True)
    return np.array(out), np.array(lse)


def _same_lse(a, b, tol):
    """Equal where finite, -inf at the same places."""
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb)
    assert np.array_equal(a[~fa], b[~fb])
    if fa.any():
        assert np.abs(a[fa] - b[fb]).max() <= tol


NULL_CASES = [
    dict(n=[5], p=[0]),
    dict(n=[3, 1, 4], p=[2, 0, 5]),
    dict(n=[0, 6], p=[3, 1]),
    dict(n=[7, 2], p=[0, 9], cap=5),      # several rows: a query also sees keys after it
]


@pytest.mark.parametrize("case", range(len(NULL_CASES)))
def test_null_mask_matches_brute_force(case):
    rng = np.random.default_rng(100 + case)
    common, rows, _ = make_problem(rng, heads=2, **NULL_CASES[case])
    for row in rows:
        out, lse = _call(common, row, "null", True)
        ref, ref_lse = _brute(common, row, causal=False)
        assert np.abs(out - ref).max() <= 1e-12
        _same_lse(lse, ref_lse, 1e-12)


LSE_CASES = [
    dict(n=[5], p=[0]),
    dict(n=[3, 1, 4], p=[2, 0, 5]),
    dict(n=[6], p=[0], cap=3),            # the second row is hidden from the first three queries
    dict(n=[7, 2], p=[0, 9], cap=5),
]


@pytest.mark.parametrize("case", range(len(LSE_CASES)))
def test_lse_matches_brute_force(case):
    rng = np.random.default_rng(200 + case)
    common, rows, _ = make_problem(rng, heads=2, **LSE_CASES[case])
    saw_empty = False
    for row in rows:
        out, lse = _call(common, row, "causal", True)
        ref, ref_lse = _brute(common, row, causal=True)
        assert np.abs(out - ref).max() <= 1e-12
        _same_lse(lse, ref_lse, 1e-12)
        saw_empty |= bool(np.isneginf(lse).any())
    if "cap" in LSE_CASES[case]:
        assert saw_empty                   # the case exercises a query with no visible key


def test_null_mask_zero_query_gives_mean_of_all_values():
    rng = np.random.default_rng(300)
    n, p = [4, 3, 5], [2, 0, 6]
    common, rows, meta = make_problem(rng, n, p, heads=2, q=np.zeros((12, 2, 192)))
    out, lse = _call(common, rows[0], "null", True)
    vl = common["valid_length"]
    for b in range(3):
        mean = meta["v_seq"][b].mean(axis=0)                 # [H, 128] over all L_b keys
        assert np.abs(out[vl[b]:vl[b + 1]] - mean[None]).max() <= 1e-12
        assert np.abs(lse[vl[b]:vl[b + 1]] - math.log(int(meta["L"][b]))).max() <= 1e-12


def test_null_mask_last_token_equals_causal():
    """The last new token sees every key under both masks; earlier tokens do not."""
    rng = np.random.default_rng(301)
    n, p = [5, 4], [3, 0]
    common, rows, _ = make_problem(rng, n, p, heads=2)
    nul = _call(common, rows[0], "null")
    cau = _call(common, rows[0], "causal")
    last = [int(x) - 1 for x in common["valid_length"][1:]]
    assert np.abs(nul[last] - cau[last]).max() <= 1e-14
    others = [t for t in range(int(sum(n))) if t not in last]
    assert np.abs(nul[others] - cau[others]).max(axis=(1, 2)).min() > 1e-6


def test_lse_single_key_is_the_scaled_score():
    """One query, one key: the log-sum-exp is that key's score."""
    rng = np.random.default_rng(302)
    q = np.zeros((1, 1, 192))
    common, rows, _ = make_problem(rng, [1], [0], heads=1, q=q, width=64, rope_col=0, page_size=2, perm=False)
    row = dict(rows[0])
    common["cache"][...] = 0.0
    common["cache"][0, 0, 0, 0, 3] = 2.0             # K_rope of position 0 = 2 e_3
    row["k_nope"] = np.zeros_like(row["k_nope"])
    row["k_nope"][0, 0, 7] = -1.5                    # K_nope of position 0 = -1.5 e_7
    common["q"][0, 0, 7] = 4.0                       # q_nope . k_nope = -6
    common["q"][0, 0, 128 + 3] = 0.25                # q_rope . k_rope = 0.5
    common["scale"] = 0.5
    _, lse = _call(common, row, "causal", True)
    assert lse[0, 0] == 0.5 * (-6.0 + 0.5)


def test_lse_of_zero_query_is_log_of_key_count():
    rng = np.random.default_rng(303)
    n, p = [4, 6], [3, 0]
    common, rows, _ = make_problem(rng, n, p, heads=3, q=np.zeros((10, 3, 192)))
    _, lse = _call(common, rows[0], "causal", True)
    vl = common["valid_length"]
    for b in range(2):
        for i in range(n[b]):
            assert np.abs(lse[vl[b] + i] - math.log(p[b] + i + 1)).max() <= 1e-13


def test_lse_shift_by_constant_score():
    """A term shared by every key's score shifts the log-sum-exp by that term
    and leaves the output unchanged: all K_rope rows equal r, q_rope = a r."""
    rng = np.random.default_rng(304)
    n, p = [5, 3], [2, 4]
    common, rows, _ = make_problem(rng, n, p, heads=2)
    r = rng.standard_normal(64)
    common["cache"][..., common["rope_col"]:common["rope_col"] + 64] = r
    q0 = common["q"].copy()
    q0[..., 128:] = 0.0
    common0 = dict(common, q=q0)
    o0, l0 = _call(common0, rows[0], "causal", True)
    a = 3.0
    q1 = q0.copy()
    q1[..., 128:] = a * r
    o1, l1 = _call(dict(common, q=q1), rows[0], "causal", True)
    shift = common["scale"] * a * float(r @ r)
    assert np.abs(o1 - o0).max() <= 1e-12
    assert np.abs((l1 - l0) - shift).max() <= 1e-11


def test_merge_two_single_key_partials_closed_form():
    """Two partials of one key each, scores 0 and 2: softmax weights 1 : e^2."""
    va = np.array([[1.0, -2.0, 0.5]])
    vb = np.array([[3.0, 4.0, -1.0]])
    o, lse = oracle.merge_partials(va, np.array([0.0]), vb, np.array([2.0]))
    w = math.exp(2.0) / (1.0 + math.exp(2.0))
    assert np.abs(o - ((1 - w) * va + w * vb)).max() <= 1e-15
    assert abs(lse[0] - math.log(1.0 + math.exp(2.0))) <= 1e-15


def test_merge_with_empty_side_is_identity():
    rng = np.random.default_rng(305)
    o_a = rng.standard_normal((4, 3, 8))
    l_a = rng.standard_normal((4, 3)) * 5
    empty_o = np.zeros_like(o_a)
    empty_l = np.full((4, 3), -np.inf)
    o, lse = oracle.merge_partials(o_a, l_a, empty_o, empty_l)
    assert np.array_equal(o, o_a) and np.array_equal(lse, l_a)
    o, lse = oracle.merge_partials(empty_o, empty_l, o_a, l_a)
    assert np.array_equal(o, o_a) and np.array_equal(lse, l_a)
    o, lse = oracle.merge_partials(empty_o, empty_l, empty_o, empty_l)
    assert np.array_equal(o, empty_o) and np.all(np.isneginf(lse))


def test_merge_is_symmetric_and_associative():
    rng = np.random.default_rng(306)
    parts = [(rng.standard_normal((5, 8)), rng.standard_normal(5) * 4) for _ in range(3)]
    ab = oracle.merge_partials(*parts[0], *parts[1])
    ba = oracle.merge_partials(*parts[1], *parts[0])
    assert np.abs(ab[0] - ba[0]).max() <= 1e-14 and np.abs(ab[1] - ba[1]).max() <= 1e-14
    left = oracle.merge_partials(*ab, *parts[2])
    right = oracle.merge_partials(*parts[0], *oracle.merge_partials(*parts[1], *parts[2]))
    assert np.abs(left[0] - right[0]).max() <= 1e-13 and np.abs(left[1] - right[1]).max() <= 1e-13


MULTI_ROW_CASES = [
    dict(n=[7, 2], p=[0, 9], cap=5, mask="causal"),
    dict(n=[5, 0, 7], p=[1, 2, 3], cap=6, mask="causal"),
    dict(n=[3, 4, 1], p=[10, 0, 2], cap=4, mask="causal"),
    dict(n=[6], p=[20], cap=7, mask="causal"),
    dict(n=[7, 2], p=[0, 9], cap=5, mask="null"),
    dict(n=[3, 4, 1], p=[10, 0, 2], cap=4, mask="null"),
]


@pytest.mark.parametrize("case", range(len(MULTI_ROW_CASES)))
def test_rows_merged_equal_single_row(case):
    """Partials of every buffer row, merged, equal one row holding every key."""
    kw = dict(MULTI_ROW_CASES[case])
    mask, cap = kw.pop("mask"), kw.pop("cap")
    full_common, full_rows, _ = make_problem(np.random.default_rng(400 + case), heads=2, **kw)
    common, rows, _ = make_problem(np.random.default_rng(400 + case), heads=2, cap=cap, **kw)
    assert len(full_rows) == 1 and len(rows) > 1
    ref, ref_lse = _call(full_common, full_rows[0], mask, True)
    o, lse = _call(common, rows[0], mask, True)
    for row in rows[1:]:
        o, lse = oracle.merge_partials(o, lse, *_call(common, row, mask, True))
    assert np.abs(o - ref).max() <= 1e-12
    _same_lse(lse, ref_lse, 1e-12)


def test_sampled_rows_with_mask_and_lse_match_full_output():
    rng = np.random.default_rng(500)
    common, rows, _ = make_problem(rng, [5, 0, 7], [1, 2, 3], heads=2, cap=6)
    picks = [(0, 1), (4, 0), (5, 1), (11, 0)]
    for mask in ("causal", "null"):
        for row in rows:
            full, full_lse = _call(common, row, mask, True)
            got, got_lse = oracle.mla_prefill_rows(
                picks, common["q"], row["k_nope"], row["v"], common["cache"], 0, common["page_table"],
                common["page_size"], common["rope_col"], common["cache_lengths"], common["valid_length"],
                row["cache_row_offsets"], row["cache_offsets"], common["scale"], mask=mask, return_lse=True)
            for k, (t, h) in enumerate(picks):
                assert np.abs(got[k] - full[t, h]).max() <= 1e-13
                _same_lse(np.array([got_lse[k]]), np.array([full_lse[t, h]]), 1e-13)
