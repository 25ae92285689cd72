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


def visible_keys(w, bro_r, co_r, mask="causal"):
    """Keys each new token sees in one buffer row: p_b + i - co_b + 1 clamped to the row's
    [0, len_b] under the causal mask, len_b under the null mask (int64 [T])."""
    vl = w.input_row_offsets.astype(np.int64)
    bro = np.asarray(bro_r, dtype=np.int64)
    co = np.zeros(w.batch, dtype=np.int64) if co_r is None else np.asarray(co_r, dtype=np.int64)
    out = np.zeros(w.total_q, dtype=np.int64)
    for b in range(w.batch):
        n = int(vl[b + 1] - vl[b])
        ln = int(bro[b + 1] - bro[b])
        i = np.arange(n)
        k = np.clip(int(w.p[b]) + i - int(co[b]) + 1, 0, ln) if mask == "causal" else np.full(n, ln)
        out[vl[b]:vl[b + 1]] = k
    return out


def report_keys(got, ref, keys, bar, label, few=5, few_excess=5e-3):
    """The bf16 bar as the flat tests read it: max |gpu - oracle| <= bar on tokens that see
    more than `few` keys; a token seeing 1..few keys averages only a few value rows, so its
    output can reach |o| of 4..8, where the bf16 rounding of the output alone is up to
    1.6e-2 -- there the error beyond half a bf16 ulp of the oracle must stay <= few_excess.
    got / ref are [T, H, 128]; returns the literal maximum."""
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    many = keys > few
    worst = float(err.max()) if err.size else 0.0
    worst_many = float(err[many].max()) if many.any() else 0.0
    excess = float((err[~many] - 0.5 * bf16_ulp(ref[~many])).max()) if (~many).any() else 0.0
    say(f"[{label}] max|gpu-oracle| = {worst:.3e}; on tokens with > {few} keys {worst_many:.3e} (bar {bar:g}); "
        f"beyond half a bf16 ulp on tokens with <= {few} keys {excess:.3e} (bar {few_excess:g})")
    assert worst_many <= bar, f"[{label}] {worst_many} > {bar}"
    assert excess <= few_excess, f"[{label}] {excess} > {few_excess}"
    return worst
