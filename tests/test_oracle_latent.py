"""Pins for the oracle's latent up-projection (CPU only).

K_nope and V of a buffer row are linear in the latent part of the cache rows
the plan row places there (reading R-y).  Pinned by a pure-Python brute force,
one-hot weights that select latent columns, linearity in the weights, the
place of the key and value halves of each head's weight rows, and untouched
unused slots.
"""
import numpy as np
import pytest

import oracle
from tests.brute import latent_up_brute
from tests.oracle_cases import make_problem


def _problem(seed, n, p, cap=None, heads=2, latent_dim=16, width=96, latent_col=8, page_size=4):
    rng = np.random.default_rng(seed)
    common, rows, meta = make_problem(rng, n, p, heads=heads, width=width, rope_col=width - 64 if width >= 64 else 0,
                                      page_size=page_size, cap=cap)
    w = rng.standard_normal((heads * 256, latent_dim))
    return common, rows, w, dict(latent_col=latent_col, latent_dim=latent_dim, heads=heads)


def _call(common, row, w, latent_col, latent_dim, heads, cap):
    return oracle.latent_up(common["cache"], 0, common["page_table"], common["page_size"], row["cache_row_offsets"],
                            np.zeros(len(row["cache_row_offsets"]) - 1, dtype=np.uint32)
                            if row["cache_offsets"] is None else row["cache_offsets"],
                            latent_col, latent_dim, w, heads, cap)


def _cache_rows(common, latent_col, latent_dim):
    cache, pt, ps = common["cache"], common["page_table"], common["page_size"]

    def rows(b, pos):
        return list(cache[0, int(pt[b][pos // ps]), pos % ps, 0, latent_col:latent_col + latent_dim])
    return rows


CASES = [
    dict(n=[3], p=[2]),
    dict(n=[2, 1, 3], p=[0, 4, 1]),
    dict(n=[4, 2], p=[3, 5], cap=5),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_latent_up_matches_brute_force(case):
    kw = dict(CASES[case])
    common, rows, w, geo = _problem(900 + case, **kw)
    for row in rows:
        cap = row["k_nope"].shape[0]
        k, v = _call(common, row, w, geo["latent_col"], geo["latent_dim"], geo["heads"], cap)
        co = [0] * (len(row["cache_row_offsets"]) - 1) if row["cache_offsets"] is None \
            else [int(x) for x in row["cache_offsets"]]
        kb, vb = latent_up_brute(_cache_rows(common, geo["latent_col"], geo["latent_dim"]),
                                 [int(x) for x in row["cache_row_offsets"]], co, w.tolist(), geo["heads"], cap,
                                 geo["latent_dim"])
        assert np.abs(k - np.array(kb)).max() <= 1e-12
        assert np.abs(v - np.array(vb)).max() <= 1e-12


def test_one_hot_weights_select_latent_columns():
    common, rows, _, geo = _problem(910, [5, 2], [1, 3], heads=3, latent_dim=64)
    row = rows[0]
    H, D = 3, 64
    w = np.zeros((H * 256, D))
    sel = np.zeros((H, 2, 128), dtype=np.int64)
    for h in range(H):
        for part in range(2):
            for d in range(128):
                sel[h, part, d] = (h * 37 + part * 11 + d * 5) % D
                w[h * 256 + part * 128 + d, sel[h, part, d]] = 1.0
    cap = row["k_nope"].shape[0]
    k, v = _call(common, row, w, geo["latent_col"], D, H, cap)
    rows_fn = _cache_rows(common, geo["latent_col"], D)
    bro = [int(x) for x in row["cache_row_offsets"]]
    for b in range(2):
        for j in range(bro[b + 1] - bro[b]):
            lat = np.array(rows_fn(b, j))
            assert np.array_equal(k[bro[b] + j], lat[sel[:, 0, :]])
            assert np.array_equal(v[bro[b] + j], lat[sel[:, 1, :]])


def test_linear_in_the_weights_and_halves_in_place():
    common, rows, w1, geo = _problem(911, [4, 3], [2, 1], heads=2)
    w2 = np.random.default_rng(912).standard_normal(w1.shape)
    row = rows[0]
    cap = row["k_nope"].shape[0]
    args = (geo["latent_col"], geo["latent_dim"], geo["heads"], cap)
    k1, v1 = _call(common, row, w1, *args)
    k2, v2 = _call(common, row, w2, *args)
    k12, v12 = _call(common, row, w1 + w2, *args)
    assert np.abs(k12 - (k1 + k2)).max() <= 1e-12 and np.abs(v12 - (v1 + v2)).max() <= 1e-12
    # swapping each head's key and value weight rows swaps the outputs
    sw = w1.reshape(2, 2, 128, -1)[:, ::-1].reshape(w1.shape)
    ks, vs = _call(common, row, sw, *args)
    assert np.array_equal(ks, v1) and np.array_equal(vs, k1)
    # heads are independent: head 1's weights only move head 1's outputs
    w3 = w1.copy()
    w3[256:] *= 2.0
    k3, v3 = _call(common, row, w3, *args)
    assert np.array_equal(k3[:, 0], k1[:, 0]) and np.abs(k3[:, 1] - 2 * k1[:, 1]).max() <= 1e-12


def test_unused_slots_are_zero_and_rows_follow_the_plan():
    common, rows, w, geo = _problem(913, [4, 2], [3, 5], cap=5)
    assert len(rows) >= 2
    for row in rows:
        cap = row["k_nope"].shape[0]
        k, v = _call(common, row, w, geo["latent_col"], geo["latent_dim"], geo["heads"], cap)
        used = int(row["cache_row_offsets"][-1])
        assert not k[used:].any() and not v[used:].any()


def test_selected_slots_match_full_output():
    common, rows, w, geo = _problem(914, [4, 2], [3, 5], cap=5)
    for row in rows:
        cap = row["k_nope"].shape[0]
        k, v = _call(common, row, w, geo["latent_col"], geo["latent_dim"], geo["heads"], cap)
        picks = [cap - 1, 0, 2]
        ks, vs = oracle.latent_up(common["cache"], 0, common["page_table"], common["page_size"],
                                  row["cache_row_offsets"], row["cache_offsets"], geo["latent_col"],
                                  geo["latent_dim"], w, geo["heads"], cap, slots=picks)
        assert np.array_equal(ks, k[picks]) and np.array_equal(vs, v[picks])
