"""Device-side precondition check (mla_prefill_check) and debug mode on the GPU.

The check reads only inside the documented extents of its arrays and compares
values, so it runs on corrupted copies of valid inputs; each corruption must
set exactly the bit the header documents for it, and valid inputs none.

Debug mode runs the check inside the entry points and returns
MLA_ERR_PRECONDITION without launching.  Its corrupted calls are built so that
they would stay inside every allocation even if they ran: the cache descriptor
claims one page fewer than the tensor holds and a page id points at that last
page (>= num_pages for the check, real memory for the kernels).
"""
import numpy as np
import pytest
import torch

import mla_ragged_paged_amd as m
from mla_ragged_paged_amd import workloads
from mla_ragged_paged_amd.pipeline import PrefillStep
from tests.gpu_util import get_workload, say

pytestmark = pytest.mark.gpu

Q, ROW, POS, PAGE = (m.MLA_VIOLATION_Q_OFFSETS, m.MLA_VIOLATION_ROW_OFFSETS, m.MLA_VIOLATION_POSITIONS,
                     m.MLA_VIOLATION_PAGE_IDS)

CASES = [
    dict(n=[130, 1, 257, 0, 64], p=[0, 300, 77, 5, 0], heads=4, ps=16),
    dict(n=[150, 70], p=[33, 0], heads=2, ps=48),
    dict(n=[0, 300, 0, 7], p=[900, 0, 0, 1500], heads=8, ps=128),
]


def _workload(case):
    kw = CASES[case]
    spec = workloads.Spec("chk", len(kw["n"]), (0, 0), (0, 0), kw["heads"], kw["ps"], True, "bf16",
                          row_width=576, rope_col=512, seed=900 + case)
    return workloads.build(spec, n=kw["n"], p=kw["p"])


def _bits(kv, **kw):
    v = torch.zeros(1, dtype=torch.int32, device="cuda")
    m.mla_prefill_check(kv, v, **kw)
    torch.cuda.synchronize()
    return int(v.item())


def _kv(step, page_table=None, cache_lengths=None, data=None):
    return m.PagedCache(step.cache_data if data is None else data,
                        step.page_table if page_table is None else page_table,
                        step.cache_lengths if cache_lengths is None else cache_lengths, step.w.spec.rope_col)


def _full_args(step):
    w = step.w
    return dict(valid_length=step.input_row_offsets, total_q_tokens=w.total_q, q_max_seq_len=w.max_q,
                row_offsets=step.buffer_row_offsets[0], row_positions=step.cache_offsets[0])


@pytest.mark.parametrize("case", range(len(CASES)))
def test_valid_inputs_set_no_bit(case):
    w = _workload(case)
    step = PrefillStep(w, "cuda", cap=max(1, w.total_ctx // 3))
    step.plan()
    kv = _kv(step)
    assert _bits(kv, valid_length=step.input_row_offsets, total_q_tokens=w.total_q) == 0
    for r in range(step.rows):
        assert _bits(kv, row_offsets=step.buffer_row_offsets[r], row_positions=step.cache_offsets[r],
                     row_capacity=step.cap) == 0
        assert _bits(kv, valid_length=step.input_row_offsets, total_q_tokens=w.total_q, q_max_seq_len=w.max_q,
                     row_offsets=step.buffer_row_offsets[r], row_positions=step.cache_offsets[r]) == 0


def test_full_size_workload_sets_no_bit():
    w = get_workload("prefix")
    step = PrefillStep(w, "cuda")
    step.plan()
    assert _bits(_kv(step), **_full_args(step), row_capacity=step.cap) == 0


def test_each_corruption_sets_its_bit():
    w = _workload(0)
    step = PrefillStep(w, "cuda")
    step.plan()
    torch.cuda.synchronize()
    kv = _kv(step)
    base = _full_args(step)
    vl = step.input_row_offsets

    def with_(**kw):
        args = dict(base)
        args.update(kw)
        return args

    # new-token offsets: a decreasing step, a nonzero start, the wrong total, n_b above q_max
    bad = vl.clone()
    bad[2] = bad[1] - 1
    assert _bits(kv, **with_(valid_length=bad)) & Q
    bad = vl.clone()
    bad[0] = 1
    assert _bits(kv, **with_(valid_length=bad)) & Q
    assert _bits(kv, **with_(total_q_tokens=w.total_q + 1)) == Q
    assert _bits(kv, **with_(total_q_tokens=None)) == 0
    assert _bits(kv, **with_(q_max_seq_len=w.max_q - 1)) == Q
    # row offsets: a decreasing step, past the capacity
    bro = step.buffer_row_offsets[0].clone()
    bro[3] = bro[2] - 1
    assert _bits(kv, **with_(row_offsets=bro)) & ROW
    assert _bits(kv, **with_(row_capacity=w.total_ctx - 1)) == ROW
    assert _bits(kv, **with_(row_capacity=w.total_ctx)) == 0
    # positions: a row starting one position late runs past the context p_b + n_b
    co = step.cache_offsets[0].clone()
    co[0] = 1
    assert _bits(kv, **with_(row_positions=co)) == POS
    # positions past the sequence's page-table row (a prefix longer than its pages)
    cl = step.cache_lengths.clone()
    ps, mp = w.spec.page_size, step.page_table.shape[1]
    cl[0] = mp * ps
    assert _bits(_kv(step, cache_lengths=cl), valid_length=vl, total_q_tokens=w.total_q) & POS
    # page ids: one out of range inside a sequence's pages, one only in an unread slot
    pt = step.page_table.clone()
    pt[2, 0] = int(w.cache.shape[1])
    assert _bits(_kv(step, page_table=pt), **base) == PAGE
    pt = step.page_table.clone()
    used = -(-int(w.n[4] + w.p[4]) // ps)
    assert used < mp
    pt[4, used] = 10 ** 6
    assert _bits(_kv(step, page_table=pt), **base) == 0


def test_debug_mode_refuses_violating_calls_and_runs_valid_ones():
    w = _workload(0)
    step = PrefillStep(w, "cuda")
    step.run()
    torch.cuda.synchronize()
    expected = step.out.clone()
    # the descriptor claims one page fewer than the tensor holds; sequence 2's first page is moved
    # to that last page (a valid id for the memory, >= num_pages for the check)
    last = int(w.cache.shape[1]) - 1
    kv_short = _kv(step, data=step.cache_data[:, :last])
    pt_bad = step.page_table.clone()
    pt_bad[2, 0] = last
    kv_bad = _kv(step, page_table=pt_bad, data=step.cache_data[:, :last])
    prev = m.mla_prefill_set_debug(True)
    try:
        say("debug mode: valid step")
        step.out.fill_(float("nan"))
        step.run()
        torch.cuda.synchronize()
        assert torch.equal(step.out, expected)
        say("debug mode: attention with an out-of-range page id")
        out = torch.full_like(step.out, float("nan"))
        with pytest.raises(m.MlaError) as e:
            m.mla_prefill_ragged(out, step.q, step.k_nope, step.v, kv_bad, 0, step.input_row_offsets,
                                 step.buffer_row_offsets[0], step.cache_offsets[0], w.softmax_scale,
                                 q_max_seq_len=w.max_q)
        assert e.value.status == m.MLA_ERR_PRECONDITION
        torch.cuda.synchronize()
        assert bool(torch.isnan(out.float()).all())            # nothing was launched
        say("debug mode: gather with an out-of-range page id")
        gathered = torch.full_like(step.gathered, 7)
        with pytest.raises(m.MlaError) as e:
            m.mla_prefill_gather(kv_bad, 0, step.buffer_row_offsets[0], step.cache_offsets[0], 0,
                                 step.gathered.shape[1], gathered)
        assert e.value.status == m.MLA_ERR_PRECONDITION
        torch.cuda.synchronize()
        assert bool((gathered == 7).all())
        say("debug mode: plan with a decreasing new-token offset")
        bad = step.input_row_offsets.clone()
        bad[2] = bad[1] - 1
        bro = torch.full_like(step.buffer_row_offsets, -5)
        with pytest.raises(m.MlaError) as e:
            m.mla_prefill_plan(bad, kv_short, 0, step.cap, bro, step.cache_offsets.clone(),
                               step.buffer_lengths.clone(), None)
        assert e.value.status == m.MLA_ERR_PRECONDITION
        torch.cuda.synchronize()
        assert bool((bro == -5).all())
    finally:
        m.mla_prefill_set_debug(prev)
    assert m.mla_prefill_set_debug(prev) == prev
