"""Pins for the oracle's plan and gather (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests.brute import plan_by_enumeration

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_worked_examples.json")


def _examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _examples(), ids=lambda e: e["name"])
def test_plan_hand_worked_examples(ex):
    bro, co, bl, st = oracle.plan(ex["input_row_offsets"], ex["cache_lengths"], ex["buffer_token_size"],
                                  ex["num_buffer_rows"])
    assert bro.tolist() == ex["buffer_row_offsets"]
    assert co.tolist() == ex["cache_offsets"]
    assert bl.tolist() == ex["buffer_lengths"]
    assert st == ex["status"]
    assert bro.dtype == np.uint32 and co.dtype == np.uint32 and bl.dtype == np.int32


def _random_case(rng, B, max_n, max_p):
    n = rng.integers(0, max_n + 1, size=B)
    p = rng.integers(0, max_p + 1, size=B)
    iro = np.concatenate([[0], np.cumsum(n)])
    return iro, p


@pytest.mark.parametrize("seed", range(40))
def test_plan_matches_enumeration(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 7))
    iro, p = _random_case(rng, B, 9, 12)
    cap = int(rng.integers(1, 20))
    total = int(p.sum() + iro[-1])
    rows = int(rng.integers(0, total // cap + 3))
    bro, co, bl, st = oracle.plan(iro, p, cap, rows)
    ebro, eco, ebl, est = plan_by_enumeration(iro.tolist(), p.tolist(), cap, rows)
    assert bro.tolist() == ebro
    assert co.tolist() == eco
    assert bl.tolist() == ebl
    assert st == est


@pytest.mark.parametrize("seed", range(20))
def test_plan_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 9))
    iro, p = _random_case(rng, B, 30, 50)
    L = p + np.diff(iro)
    C = int(L.sum())
    cap = int(rng.integers(1, 64))
    R = -(-C // cap) + 1
    bro, co, bl, st = oracle.plan(iro, p, cap, R)
    assert st == 0
    # every (sequence, position) lands in exactly one (row, slot)
    seen = np.zeros(C, dtype=np.int64)
    start = np.concatenate([[0], np.cumsum(L)])
    for r in range(R):
        if bl[r] < 0:
            continue
        for b in range(B):
            ln = int(bro[r, b + 1]) - int(bro[r, b])
            assert ln >= 0
            for j in range(ln):
                seen[start[b] + int(co[r, b]) + j] += 1
    assert (seen == 1).all()
    assert int(np.maximum(bl, 0).sum()) == C
    # a single row of enough capacity: exclusive prefix sum, zero offsets
    bro1, co1, bl1, st1 = oracle.plan(iro, p, max(C, 1), 2)
    assert bro1[0].tolist() == start.tolist()
    assert co1[0].tolist() == [0] * B
    assert bl1.tolist() == [C, -1]


def test_plan_empty_batch_and_zero_rows():
    bro, co, bl, st = oracle.plan([0, 0, 0], [0, 0], 8, 2)
    assert bl.tolist() == [-1, -1] and st == 0
    bro, co, bl, st = oracle.plan([0, 5], [0], 8, 0)
    assert bro.shape == (0, 2) and st == 1


# ---- gather -------------------------------------------------------------
def _paged_cache(rng, L, ps, width, perm):
    pages_per = [(x + ps - 1) // ps for x in L]
    npages = max(1, sum(pages_per))
    logical = rng.standard_normal((sum(L), width))  # rows by (b, pos) in batch order
    cache = np.zeros((1, npages, ps, 1, width))
    pt = np.zeros((len(L), max(pages_per + [1])), dtype=np.uint32)
    k, s = 0, 0
    for b, l in enumerate(L):
        for j in range(pages_per[b]):
            pt[b, j] = perm[k]
            k += 1
        for pos in range(l):
            cache[0, pt[b, pos // ps], pos % ps, 0, :] = logical[s + pos]
        s += l
    return logical, cache, pt, npages


@pytest.mark.parametrize("seed", range(6))
def test_gather_is_a_contiguous_slice_and_permutation_invariant(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 5))
    n = rng.integers(0, 20, size=B)
    p = rng.integers(0, 30, size=B)
    L = (n + p).tolist()
    ps, width = int(rng.choice([1, 4, 16])), 24
    iro = np.concatenate([[0], np.cumsum(n)])
    pages = sum((x + ps - 1) // ps for x in L) or 1
    logical, cache_id, pt_id, _ = _paged_cache(np.random.default_rng(seed), L, ps, width, np.arange(pages))
    _, cache_pm, pt_pm, _ = _paged_cache(np.random.default_rng(seed), L, ps, width, rng.permutation(pages))
    cap = int(rng.integers(1, 40))
    C = sum(L)
    R = -(-C // cap) if C else 1
    bro, co, bl, _ = oracle.plan(iro, p, cap, R)
    col0, ncol = 3, 17
    for r in range(R):
        init = np.full((cap, ncol), -7.0)
        a = oracle.gather(cache_id, 0, pt_id, ps, bro[r], co[r], col0, ncol, init)
        b_ = oracle.gather(cache_pm, 0, pt_pm, ps, bro[r], co[r], col0, ncol, init)
        assert np.array_equal(a, b_)
        used = max(int(bl[r]), 0)
        # the used part of the row is the stream slice [r*cap, r*cap+used)
        assert np.array_equal(a[:used], logical[r * cap:r * cap + used, col0:col0 + ncol])
        assert (a[used:] == -7.0).all()


def test_gather_accepts_torch_bf16():
    rng = np.random.default_rng(0)
    cache = torch.randn(1, 3, 4, 1, 8).to(torch.bfloat16)
    pt = np.array([[2, 0, 1]], dtype=np.uint32)
    out = oracle.gather(cache, 0, pt, 4, np.array([0, 9]), np.array([1]), 0, 8, np.zeros((9, 8)))
    c = cache.to(torch.float64).numpy()
    ref = np.stack([c[0, pt[0, pos // 4], pos % 4, 0] for pos in range(1, 10)])
    assert np.array_equal(out, ref)
    del rng
