"""Pins for the oracle's split-Q attention (CPU only).

"flare_mla_prefill" has overloads whose query arrives as q_nope (with q_scale
when fp8) and q_rope, whose K carries k_scales, and whose K_rope is paged or
contiguous.  Pinned by the pure-Python brute force on the decoded values (torch's
own fp8 decoder), by the identity "two halves of one query = that query" against
the pinned non-split oracle, and by where each scale and each rope row goes.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.brute import attention_brute
from tests.oracle_cases import call, make_problem, rope_fn


def _q8(x):
    s = float(np.float32(np.abs(x).max() / 448.0))
    return torch.from_numpy(x / s).to(torch.float8_e4m3fn), s


def _deq(c, s):
    return c.to(torch.float64).numpy() * s          # torch's own decoder


def _split(common, row, **kw):
    return oracle.mla_prefill_ragged_split(
        kw.get("q_nope", common["q"][..., :128]), kw.get("q_rope", common["q"][..., 128:]),
        kw.get("k_nope", row["k_nope"]), kw.get("v", row["v"]), common["cache_lengths"], common["valid_length"],
        row["cache_row_offsets"], row["cache_offsets"], common["scale"], k_rope_rows=kw.get("k_rope_rows"),
        cache=kw.get("cache", common["cache"]), layer_idx=0, page_table=common["page_table"],
        page_size=common["page_size"], rope_col=common["rope_col"], scales=kw.get("scales"),
        mask=kw.get("mask", "causal"), return_lse=kw.get("return_lse", False))


def _contiguous_rope(common, row, meta):
    """K_rope rows laid out like K / V: buffer row g holds the rope of the cache
    position the row's plan puts there (zeros in unused slots)."""
    rope = rope_fn(common)
    bro = [int(x) for x in row["cache_row_offsets"]]
    co = [0] * (len(bro) - 1) if row["cache_offsets"] is None else [int(x) for x in row["cache_offsets"]]
    rows = np.zeros((row["k_nope"].shape[0], 1, 64))
    for b in range(len(bro) - 1):
        for j in range(bro[b + 1] - bro[b]):
            rows[bro[b] + j, 0] = rope(b, co[b] + j)
    return rows


SPLIT_CASES = [
    dict(n=[5], p=[0]),
    dict(n=[3, 1, 4], p=[2, 0, 5]),
    dict(n=[7, 2], p=[0, 9], cap=5),
]


@pytest.mark.parametrize("contig", [False, True])
@pytest.mark.parametrize("case", range(len(SPLIT_CASES)))
def test_split_fp8_matches_brute_force(case, contig):
    """fp8 q_nope / K / V with four distinct scales, bf16-valued q_rope, paged fp8
    or contiguous float K_rope, against the brute force on the decoded values."""
    rng = np.random.default_rng(700 + case)
    common, rows, meta = make_problem(rng, heads=2, **SPLIT_CASES[case])
    qn_c, sq = _q8(common["q"][..., :128])
    qr = torch.from_numpy(common["q"][..., 128:]).to(torch.bfloat16).to(torch.float64).numpy()
    cache_c, skr = _q8(common["cache"] * 0.5)
    for row in rows:
        kn_c, skn = _q8(row["k_nope"] * 2.0)
        v_c, sv = _q8(row["v"] * 3.0)
        scales = {"q": sq, "k_nope": skn, "v": sv, "k_rope": skr}
        assert len(set(scales.values())) == 4
        kw = dict(q_nope=qn_c, q_rope=qr, k_nope=kn_c, v=v_c, scales=scales, return_lse=True)
        deq_common = dict(common, cache=_deq(cache_c, skr))
        if contig:
            kw["k_rope_rows"] = _contiguous_rope(deq_common, row, meta)
        else:
            kw["cache"] = cache_c
        got, got_lse = _split(common, row, **kw)
        q_full = np.concatenate([_deq(qn_c, sq), qr], axis=2)
        rope = rope_fn(deq_common)
        ref, ref_lse = attention_brute(
            q_full.tolist(), _deq(kn_c, skn).tolist(), _deq(v_c, sv).tolist(), rope,
            [int(x) for x in common["cache_lengths"]], [int(x) for x in common["valid_length"]],
            [int(x) for x in row["cache_row_offsets"]],
            None if row["cache_offsets"] is None else [int(x) for x in row["cache_offsets"]],
            common["scale"], with_lse=True)
        assert np.abs(got - np.array(ref)).max() <= 1e-12
        ref_lse = np.array(ref_lse)
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(got_lse))
        assert np.abs(got_lse[fin] - ref_lse[fin]).max() <= 1e-12


@pytest.mark.parametrize("mask", ["causal", "null"])
def test_halves_of_one_query_equal_that_query(mask):
    """Unquantised q split at column 128 gives the non-split attention exactly."""
    rng = np.random.default_rng(710)
    common, rows, _ = make_problem(rng, [6, 3, 5], [2, 0, 7], heads=3, cap=9)
    for row in rows:
        got = _split(common, row, mask=mask)
        ref = oracle.mla_prefill_ragged(common["q"], row["k_nope"], row["v"], common["cache"], 0,
                                        common["page_table"], common["page_size"], common["rope_col"],
                                        common["cache_lengths"], common["valid_length"], row["cache_row_offsets"],
                                        row["cache_offsets"], common["scale"], mask=mask)
        assert np.array_equal(got, ref)


def test_q_scale_scales_q_nope_only():
    """Doubling q_scale equals doubling the nope half of the query, not the rope half."""
    rng = np.random.default_rng(711)
    common, rows, _ = make_problem(rng, [5, 4], [3, 1], heads=2)
    row = rows[0]
    qn_c, sq = _q8(common["q"][..., :128])
    qr = common["q"][..., 128:]
    one = {"q": 2.0 * sq, "k_nope": 1.0, "v": 1.0, "k_rope": 1.0}
    kn = torch.from_numpy(row["k_nope"]).to(torch.float8_e4m3fn)
    v = torch.from_numpy(row["v"]).to(torch.float8_e4m3fn)
    cache = torch.from_numpy(common["cache"]).to(torch.float8_e4m3fn)
    got = _split(common, row, q_nope=qn_c, q_rope=qr, k_nope=kn, v=v, cache=cache, scales=one)
    q2 = np.concatenate([2.0 * _deq(qn_c, sq), qr], axis=2)
    ref = call(oracle, dict(common, q=q2, cache=_deq(cache, 1.0)),
               dict(row, k_nope=_deq(kn, 1.0), v=_deq(v, 1.0)))
    assert np.abs(got - ref).max() <= 1e-12


def test_contiguous_rope_equals_paged_rope():
    """Contiguous K_rope rows holding what the page table points at give the paged result
    bit for bit, over several buffer rows (cache_offsets non-zero)."""
    rng = np.random.default_rng(712)
    common, rows, meta = make_problem(rng, [7, 2, 4], [3, 9, 0], heads=2, cap=6)
    assert len(rows) > 1
    for row in rows:
        paged = _split(common, row)
        contig = _split(common, row, k_rope_rows=_contiguous_rope(common, row, meta), cache=None)
        assert np.array_equal(paged, contig)


def test_contiguous_rope_is_indexed_by_buffer_row():
    """Moving a sequence's K_nope / V / K_rope rows to other buffer rows (and its
    cache_row_offsets with them) leaves its output unchanged."""
    rng = np.random.default_rng(713)
    common, rows, meta = make_problem(rng, [4, 3], [2, 5], heads=2)
    row = rows[0]
    kr = _contiguous_rope(common, row, meta)
    a = _split(common, row, k_rope_rows=kr, cache=None)
    bro = [int(x) for x in row["cache_row_offsets"]]
    gap = 3                                            # 3 unused rows in front of the batch's rows
    idx = [bro[2] - 1] * gap + list(range(bro[2]))
    moved = dict(row, k_nope=row["k_nope"][idx], v=row["v"][idx],
                 cache_row_offsets=np.array([gap, bro[1] + gap, bro[2] + gap], dtype=np.uint32))
    b = _split(common, moved, k_rope_rows=kr[idx], cache=None)
    assert np.array_equal(a, b)


def test_sampled_split_rows_match_full_output():
    rng = np.random.default_rng(714)
    common, rows, meta = make_problem(rng, [5, 0, 7], [1, 2, 3], heads=2, cap=6)
    qn_c, sq = _q8(common["q"][..., :128])
    qr = common["q"][..., 128:]
    cache_c, skr = _q8(common["cache"])
    picks = [(0, 1), (4, 0), (5, 1), (11, 0)]
    for row in rows:
        kn_c, skn = _q8(row["k_nope"])
        v_c, sv = _q8(row["v"])
        scales = {"q": sq, "k_nope": skn, "v": sv, "k_rope": skr}
        for contig in (False, True):
            kw = dict(q_nope=qn_c, q_rope=qr, k_nope=kn_c, v=v_c, scales=scales, mask="null" if contig else "causal")
            if contig:
                kw["k_rope_rows"] = _contiguous_rope(common, row, meta)
            else:
                kw["cache"] = cache_c
            full = _split(common, row, **kw)
            got = oracle.mla_prefill_rows_split(
                picks, qn_c, qr, kn_c, v_c, common["cache_lengths"], common["valid_length"],
                row["cache_row_offsets"], row["cache_offsets"], common["scale"], k_rope_rows=kw.get("k_rope_rows"),
                cache=kw.get("cache"), page_table=common["page_table"], page_size=common["page_size"],
                rope_col=common["rope_col"], scales=scales, mask=kw["mask"])
            for k, (t, h) in enumerate(picks):
                assert np.abs(got[k] - full[t, h]).max() <= 1e-13
