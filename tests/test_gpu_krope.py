"""Attention with K_rope given as rows laid out like K (mla_prefill_ragged_krope, and
mla_prefill_ragged_row_krope for the rows of a multi-row plan) on the GPU against the
float64 oracle.

Bars: max |gpu - oracle| <= 1e-2 (bf16; on tokens that see 1..5 keys the error
beyond half a bf16 ulp of the output, <= 5e-3, as in the other bf16 tests) and
<= 6e-2 (float8_e4m3fn inputs, bf16 output).  Rows holding exactly the cache's
K_rope window must give the paged call's output bit for bit (the same
arithmetic on the same values).
"""
import numpy as np
import pytest
import torch

import oracle
import mla_ragged_paged_amd as m
from mla_ragged_paged_amd import workloads
from mla_ragged_paged_amd.pipeline import PrefillStep
from tests.gpu_util import check_plan, report, report_keys, say, visible_keys

pytestmark = pytest.mark.gpu

BAR = {"bf16": 1e-2, "fp8": 6e-2}

CASES = [
    dict(n=[130, 1, 257, 0, 64], p=[0, 300, 77, 5, 0], heads=8, ps=16),
    dict(n=[200], p=[1000], heads=3, ps=128),                  # one queue (H not a multiple of 8)
    dict(n=[150, 70], p=[33, 0], heads=16, ps=48),
    dict(n=[513, 40, 0, 200], p=[0, 0, 5, 64], heads=24, ps=16),
    dict(n=[300, 129, 1], p=[20, 0, 7], heads=128, ps=128),    # the DeepSeek-V3 head count
]


def _workload(kw, dtype, seed):
    spec = workloads.Spec("krope", len(kw["n"]), (0, 0), (0, 0), kw["heads"], kw["ps"], True, dtype,
                          row_width=576, rope_col=512, seed=seed)
    return workloads.build(spec, n=kw["n"], p=kw["p"])


def _host_rows(w, bro, co):
    """K_rope rows laid out like K for one plan row, read off the paged cache on the host."""
    rows = torch.zeros((max(1, int(bro[-1])), 1, 64), dtype=w.cache.dtype)
    for b in range(w.batch):
        for j in range(int(bro[b + 1]) - int(bro[b])):
            pos = int(co[b]) + j
            page = int(w.page_table[b][pos // w.spec.page_size])
            rows[int(bro[b]) + j, 0] = w.cache[0, page, pos % w.spec.page_size, 0, 512:576]
    return rows


def _call(step, out, rows, rows_scale=None, mask="causal", cache_offsets="plan", cro=None):
    w = step.w
    sc = step.scales or {}
    co = step.cache_offsets[0] if isinstance(cache_offsets, str) else cache_offsets
    m.mla_prefill_ragged_krope(out, step.q, step.k_nope, step.v, rows, step.cache_lengths, step.input_row_offsets,
                               step.buffer_row_offsets[0] if cro is None else cro, co, w.softmax_scale,
                               k_rope_scale=rows_scale, q_scale=sc.get("q"), k_nope_scale=sc.get("k_nope"),
                               v_scale=sc.get("v"), q_max_seq_len=w.max_q, mask=mask)
    torch.cuda.synchronize()


def _oracle_rows(w, bro, co, rows_f64, mask="causal"):
    """The definition with K_rope taken from the given rows (float64 values), via the
    split-query oracle: q's columns 0..127 as q_nope (codes with q_scale when fp8) and
    its columns 128..191, dequantised, as q_rope."""
    q_nope = w.q[..., :128].contiguous()
    if w.spec.dtype == "fp8":
        q_rope = oracle.dequantize_e4m3fn(w.q[..., 128:].contiguous().view(torch.uint8).numpy(), w.scales["q"])
    else:
        q_rope = w.q[..., 128:].contiguous()
    return oracle.mla_prefill_ragged_split(q_nope, q_rope, w.k_nope, w.v, w.cache_lengths, w.input_row_offsets, bro,
                                           co, w.softmax_scale, k_rope_rows=rows_f64, scales=w.scales, mask=mask)


@pytest.mark.parametrize("mask", ["causal", "null"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_cache_window_rows(case, dtype, mask):
    """Rows holding the cache's K_rope window: the oracle's paged definition, and the paged
    call's output bit for bit."""
    kw = CASES[case]
    say(f"krope case {kw} {dtype} {mask}")
    w = _workload(kw, dtype, 900 + case)
    step = PrefillStep(w, "cuda", mask=mask)
    step.plan()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    rows = _host_rows(w, bro[0], co[0]).cuda()
    rs = step.scales["k_rope"] if dtype == "fp8" else None
    ref = oracle.mla_prefill_ragged(w.q, w.k_nope, w.v, w.cache, 0, w.page_table, w.spec.page_size, w.spec.rope_col,
                                    w.cache_lengths, w.input_row_offsets, bro[0], co[0], w.softmax_scale,
                                    scales=w.scales, mask=mask)
    out = torch.full_like(step.out, float("nan"))
    _call(step, out, rows, rs, mask=mask)
    if dtype == "bf16":
        report_keys(out.float().cpu().numpy(), ref, visible_keys(w, bro[0], co[0], mask), BAR[dtype], "krope")
    else:
        assert report(out.float().cpu().numpy(), ref, BAR[dtype], "krope") <= BAR[dtype]
    paged = torch.full_like(step.out, float("nan"))
    sc = step.scales or {}
    m.mla_prefill_ragged(paged, step.q, step.k_nope, step.v, step.kv, 0, step.input_row_offsets,
                         step.buffer_row_offsets[0], step.cache_offsets[0], w.softmax_scale, sc.get("q"),
                         sc.get("k_nope"), sc.get("v"), w.max_q, mask=mask)
    torch.cuda.synchronize()
    assert torch.equal(out, paged)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_independent_rows(dtype):
    """Rows that are not the cache's (drawn on their own): the kernel reads the rows argument."""
    kw = CASES[0]
    w = _workload(kw, dtype, 950)
    step = PrefillStep(w, "cuda")
    step.plan()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    raw = workloads.draw_rope_rows(w.total_ctx, seed=951).float()
    if dtype == "fp8":
        scale = float(raw.abs().max()) / 448.0
        codes = (raw / scale).to(torch.float8_e4m3fn)
        rows_f64 = oracle.dequantize_e4m3fn(codes.view(torch.uint8).numpy(), np.float32(scale))
        rows = codes.cuda()
        rs = torch.tensor([scale], dtype=torch.float32, device="cuda")
    else:
        rows16 = raw.to(torch.bfloat16)
        rows_f64 = rows16.to(torch.float64).numpy()
        rows = rows16.cuda()
        rs = None
    ref = _oracle_rows(w, bro[0], co[0], rows_f64)
    out = torch.full_like(step.out, float("nan"))
    _call(step, out, rows, rs)
    if dtype == "bf16":
        report_keys(out.float().cpu().numpy(), ref, visible_keys(w, bro[0], co[0]), BAR[dtype], "independent rows bf16")
    else:
        assert report(out.float().cpu().numpy(), ref, BAR[dtype], "independent rows fp8") <= BAR[dtype]


def test_units_without_visible_keys():
    """A buffer row holding only positions 200..299 of a 300-token sequence: the first query
    tile sees no key (zeros), the others part of the row."""
    spec = workloads.Spec("late", 1, (0, 0), (0, 0), 8, 16, True, "bf16", row_width=576, rope_col=512, seed=960)
    w = workloads.build(spec, n=[300], p=[0])
    step = PrefillStep(w, "cuda")
    step.plan()
    torch.cuda.synchronize()
    cro = torch.tensor([0, 100], dtype=torch.int32, device="cuda")
    co = torch.tensor([200], dtype=torch.int32, device="cuda")
    bro_h, co_h = np.array([0, 100], dtype=np.uint32), np.array([200], dtype=np.uint32)
    kn, v = w.k_nope[:100].contiguous(), w.v[:100].contiguous()
    step.k_nope, step.v = kn.cuda(), v.cuda()
    rows = _host_rows(w, bro_h, co_h).cuda()
    ref = oracle.mla_prefill_ragged(w.q, kn, v, w.cache, 0, w.page_table, w.spec.page_size, w.spec.rope_col,
                                    w.cache_lengths, w.input_row_offsets, bro_h, co_h, w.softmax_scale)
    assert np.all(ref[:128] == 0.0) and np.any(ref[128:] != 0.0)
    out = torch.full_like(step.out, float("nan"))
    _call(step, out, rows, cache_offsets=co, cro=cro)
    report_keys(out.float().cpu().numpy(), ref, visible_keys(w, bro_h, co_h), BAR["bf16"], "late keys")


def test_step_gather_feeds_the_attention():
    """The step's default gather is the K_rope window of the plan row, bit-exact, and the
    one-row attention reads it: the step output equals the paged call bit for bit."""
    kw = CASES[4]
    w = _workload(kw, "bf16", 990)
    step = PrefillStep(w, "cuda")
    step.run()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    assert step.gather_cols == (512, 64)
    want = _host_rows(w, bro[0], co[0]).view(torch.int16)[:, 0]
    got = step.gathered.view(torch.int16).cpu()[:want.shape[0]]
    assert torch.equal(got, want)
    paged = torch.full_like(step.out, float("nan"))
    step.attention(0, out=paged, rope="paged")
    torch.cuda.synchronize()
    assert torch.equal(paged, step.out)


@pytest.mark.parametrize("mask", ["causal", "null"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_rows_read_their_gathered_window(dtype, mask):
    """A plan of several buffer rows: each row's attention reads that row's gathered K_rope
    window (mla_prefill_ragged_row_krope).  The output equals the same rows read through the
    page table bit for bit (the same arithmetic on the same values) and the oracle over every
    key (one row holding all of them)."""
    kw = CASES[0]
    say(f"rows gathered {kw} {dtype} {mask}")
    w = _workload(kw, dtype, 970)
    step = PrefillStep(w, "cuda", cap=150, mask=mask)
    assert step.rows >= 2
    step.out.fill_(float("nan"))
    step.acc.fill_(float("nan"))
    step.lse.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    check_plan(step, w)
    gathered = step.out.clone()
    step.out.fill_(float("nan"))
    step.acc.fill_(float("nan"))
    for r in range(step.rows):
        step.attention_row_merged(r, rope="paged")
    torch.cuda.synchronize()
    assert torch.equal(gathered, step.out)
    bro1, co1, _, st = oracle.plan(w.input_row_offsets, w.cache_lengths, max(1, w.total_ctx), 1)
    assert st == 0
    ref = oracle.mla_prefill_ragged(w.q, w.k_nope, w.v, w.cache, 0, w.page_table, w.spec.page_size, w.spec.rope_col,
                                    w.cache_lengths, w.input_row_offsets, bro1[0], co1[0], w.softmax_scale,
                                    scales=w.scales, mask=mask)
    if dtype == "bf16":
        report_keys(gathered.float().cpu().numpy(), ref, visible_keys(w, bro1[0], co1[0], mask), BAR[dtype],
                    "rows gathered")
    else:
        assert report(gathered.float().cpu().numpy(), ref, BAR[dtype], "rows gathered fp8") <= BAR[dtype]
