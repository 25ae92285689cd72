"""Helpers for the GPU parity tests (test side only)."""
import functools
import sys

import numpy as np
import torch

import oracle
from mla_ragged_paged_amd import workloads
from mla_ragged_paged_amd.pipeline import PrefillStep


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host_u32(t):
    return t.cpu().numpy().astype(np.int64).astype(np.uint32)


def check_plan(step, w):
    bro, co, bl, st = oracle.plan(w.input_row_offsets, w.cache_lengths, step.cap, step.rows)
    assert np.array_equal(host_u32(step.buffer_row_offsets), bro)
    assert np.array_equal(host_u32(step.cache_offsets), co)
    assert np.array_equal(step.buffer_lengths.cpu().numpy(), bl)
    assert int(step.status.cpu()[0]) == st
    return bro, co, bl


def oracle_full(w, bro_r, co_r, k_nope=None, v=None, mask="causal", return_lse=False):
    return oracle.mla_prefill_ragged(w.q, w.k_nope if k_nope is None else k_nope, w.v if v is None else v, w.cache,
                                     w.spec.layer_idx, w.page_table, w.spec.page_size, w.spec.rope_col,
                                     w.cache_lengths, w.input_row_offsets, bro_r, co_r, w.softmax_scale,
                                     scales=w.scales, mask=mask, return_lse=return_lse)


def oracle_rows(w, rows, bro_r, co_r, mask="causal", return_lse=False):
    return oracle.mla_prefill_rows(rows, w.q, w.k_nope, w.v, w.cache, w.spec.layer_idx, w.page_table,
                                   w.spec.page_size, w.spec.rope_col, w.cache_lengths, w.input_row_offsets,
                                   bro_r, co_r, w.softmax_scale, scales=w.scales, mask=mask, return_lse=return_lse)


def report_lse(got, ref, bar, label):
    """Compare log-sum-exps: -inf exactly where the oracle has -inf, else max abs error <= bar."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"[{label}] -inf pattern differs"
    fin = np.isfinite(ref)
    assert np.isfinite(got[fin]).all(), f"[{label}] non-finite lse where the oracle is finite"
    worst = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
    say(f"[{label}] max|lse gpu-oracle| = {worst:.3e} (bar {bar:g}); finite = {int(fin.sum())}, "
        f"-inf = {int((~fin).sum())}")
    return worst


def sample_rows(w, count, seed):
    """(token, head) pairs: every sequence's first and last token, tile edges, and random ones."""
    rng = np.random.default_rng(seed)
    vl = w.input_row_offsets.astype(np.int64)
    picks = []
    for b in range(w.batch):
        n = int(vl[b + 1] - vl[b])
        if n == 0:
            continue
        for i in {0, n - 1, min(n - 1, 127), min(n - 1, 128), min(n - 1, 31), min(n - 1, 32), n // 2}:
            picks.append((int(vl[b] + i), int(rng.integers(0, w.heads))))
    while len(picks) < count:
        t = int(rng.integers(0, w.total_q))
        picks.append((t, int(rng.integers(0, w.heads))))
    return picks


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def report(got, ref, bar, label):
    """Print the max error and the part of it beyond the bf16 rounding of the output itself."""
    err = np.abs(got - ref)
    worst = float(err.max()) if err.size else 0.0
    excess = float(np.max(err - 0.5 * bf16_ulp(ref))) if err.size else 0.0
    say(f"[{label}] max|gpu-oracle| = {worst:.3e} (bar {bar:g}); max error beyond half a bf16 ulp of the "
        f"oracle = {excess:.3e}; outputs compared = {err.size}")
    return worst


@functools.lru_cache(maxsize=None)
def get_workload(name):
    say(f"building workload {name}: {workloads.SPECS[name].description}")
    return workloads.build(workloads.SPECS[name])
