"""Property-based pins of the oracle's plan and gather (CPU only).

Random batches drawn by hypothesis: sequence count, new tokens n_b, cached
prefixes p_b, buffer-row capacity and row count, page size and a random
physical page permutation ("generic_flare_mla_prefill_ragged_paged_plan",
Args: input_row_offsets, buffer_token_size, and the rows it fills).

* plan: equals the enumeration brute force of tests/brute.py (every
  (sequence, position) placed at its stream index and read back), and the
  rows together cover each position exactly once;
* gather: every slot a row fills holds the cache row the page table names for
  that (sequence, position), computed here by a per-slot walk that shares no
  code with the oracle; slots past the row's fill keep their old contents;
  a different physical page permutation of the same logical cache gives the
  same buffer.
"""
import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from tests.brute import plan_by_enumeration


@st.composite
def batches(draw, max_b=6, max_n=20, max_p=24):
    B = draw(st.integers(1, max_b))
    n = draw(st.lists(st.integers(0, max_n), min_size=B, max_size=B))
    p = draw(st.lists(st.integers(0, max_p), min_size=B, max_size=B))
    return n, p


@settings(max_examples=150, deadline=None)
@given(batches(), st.integers(1, 40), st.integers(0, 6))
def test_plan_matches_enumeration_property(np_pair, cap, extra_rows):
    n, p = np_pair
    iro = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    total = int(sum(n) + sum(p))
    rows = max(0, -(-total // cap) - 1 + extra_rows)   # sometimes one row short
    bro, co, bl, status = oracle.plan(iro, p, cap, rows)
    ebro, eco, ebl, est = plan_by_enumeration(iro.tolist(), list(p), cap, rows)
    assert bro.tolist() == ebro
    assert co.tolist() == eco
    assert bl.tolist() == ebl
    assert status == est
    # coverage: when the rows suffice, every (b, pos) is in exactly one row slice
    if status == 0:
        seen = {}
        for r in range(rows):
            for b in range(len(n)):
                for j in range(int(bro[r, b + 1]) - int(bro[r, b])):
                    key = (b, int(co[r, b]) + j)
                    seen[key] = seen.get(key, 0) + 1
        want = {(b, pos) for b in range(len(n)) for pos in range(n[b] + p[b])}
        assert set(seen) == want and all(c == 1 for c in seen.values())


def _paged_cache(rng, L, page_size, width, perm):
    """A logical cache (one row of `width` values per (b, pos)) stored in pages
    whose physical ids follow `perm`; returns (cache, page_table, logical)."""
    pages = [-(-int(x) // page_size) for x in L]
    num_pages = max(1, sum(pages))
    cache = np.full((1, num_pages, page_size, 1, width), -1.0)
    table = np.zeros((len(L), max([1] + pages)), dtype=np.uint32)
    logical = {}
    k = 0
    for b, cnt in enumerate(pages):
        for j in range(cnt):
            table[b, j] = perm[k]
            k += 1
        for pos in range(int(L[b])):
            row = rng.standard_normal(width)
            logical[(b, pos)] = row
    for (b, pos), row in logical.items():
        cache[0, table[b, pos // page_size], pos % page_size, 0, :] = row
    return cache, table, logical


@settings(max_examples=120, deadline=None)
@given(batches(max_b=5, max_n=12, max_p=20), st.integers(1, 30), st.sampled_from([1, 2, 4, 16]),
       st.integers(0, 2 ** 32 - 1), st.integers(0, 5), st.integers(1, 5))
def test_gather_property(np_pair, cap, page_size, seed, col_begin, col_count):
    n, p = np_pair
    L = np.asarray(n) + np.asarray(p)
    total = int(L.sum())
    width = 10
    rng = np.random.default_rng(seed)
    num_pages = max(1, sum(-(-int(x) // page_size) for x in L))
    perm_a = rng.permutation(num_pages)
    perm_b = rng.permutation(num_pages)
    cache_a, table_a, logical = _paged_cache(np.random.default_rng(seed), L, page_size, width, perm_a)
    cache_b, table_b, _ = _paged_cache(np.random.default_rng(seed), L, page_size, width, perm_b)
    iro = np.concatenate([[0], np.cumsum(n)])
    rows = max(1, -(-total // cap))
    bro, co, bl, status = oracle.plan(iro, p, cap, rows)
    assert status == 0
    cols = slice(col_begin, col_begin + col_count)
    for r in range(rows):
        before = np.full((cap, col_count), 7.0)
        got_a = oracle.gather(cache_a, 0, table_a, page_size, bro[r], co[r], col_begin, col_count, before)
        got_b = oracle.gather(cache_b, 0, table_b, page_size, bro[r], co[r], col_begin, col_count, before)
        assert np.array_equal(got_a, got_b)                      # page permutation invariance
        fill = max(int(bl[r]), 0)                              # -1: a row the batch does not reach
        slot = 0
        for b in range(len(n)):                                  # per-slot walk of the row
            for j in range(int(bro[r, b + 1]) - int(bro[r, b])):
                assert int(bro[r, b]) + j == slot
                assert np.array_equal(got_a[slot], logical[(b, int(co[r, b]) + j)][cols])
                slot += 1
        assert slot == fill
        assert np.all(got_a[fill:] == 7.0)                       # slots past the fill untouched
