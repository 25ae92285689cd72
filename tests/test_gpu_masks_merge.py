"""Null mask, log-sum-exp output and the merge of buffer rows on the GPU,
against the float64 oracle.

Bars (the accuracy bars of the output, written here): max |gpu - oracle|
<= 1e-2 with bf16 inputs and <= 6e-2 with float8_e4m3fn inputs.

Log-sum-exp bars, derived from the arithmetic: scores are exact up to fp32
rounding, and the row sum is taken over the weights p as the kernel rounds
them (bf16: relative error <= 2^-9 per weight; e4m3 on tiles every query of
the wave fully sees: <= 2^-4), so the relative error of the sum is at most
that and the error of its log at most -ln(1 - 2^-9) = 2.0e-3 (bf16) and
-ln(1 - 2^-4) = 0.0645 (fp8).  Bars: 1e-2 and 6.5e-2.

The standalone merge kernel combines fp32 partials; its result is compared
with the oracle's merge of the very same fp32 values, bar 1e-5 (fp32
arithmetic with the hardware exp2 / log2, relative error ~1e-7 on values of
magnitude <= 4).
"""
import numpy as np
import pytest
import torch

import oracle
import mla_ragged_paged_amd as m
from mla_ragged_paged_amd import workloads
from mla_ragged_paged_amd.pipeline import PrefillStep
from tests.gpu_util import (check_plan, get_workload, host_u32, oracle_full, oracle_rows, report, report_lse,
                            sample_rows, say)

pytestmark = pytest.mark.gpu

BAR = {"bf16": 1e-2, "fp8": 6e-2}
LSE_BAR = {"bf16": 1e-2, "fp8": 6.5e-2}
MERGE_BAR = 1e-5

CASES = [
    dict(n=[130, 1, 257, 0, 64], p=[0, 300, 77, 5, 0], heads=4, ps=16),
    dict(n=[200], p=[1000], heads=3, ps=128),
    dict(n=[150, 70], p=[33, 0], heads=2, ps=48),           # page size not a power of two
    dict(n=[513], p=[0], heads=2, ps=128),                  # 4 full query tiles + 1 row
    dict(n=[130, 40, 0, 200], p=[10, 0, 5, 64], heads=16, ps=16),
    dict(n=[0, 300, 0, 7], p=[900, 0, 0, 1500], heads=8, ps=128),     # contexts without new tokens, empty ones
]


def _workload(case, dtype, seed_base):
    kw = CASES[case]
    spec = workloads.Spec("mm", len(kw["n"]), (0, 0), (0, 0), kw["heads"], kw["ps"], True, dtype,
                          row_width=576, rope_col=512, seed=seed_base + case)
    return workloads.build(spec, n=kw["n"], p=kw["p"])


def _one_row_plan(w):
    bro, co, _, st = oracle.plan(w.input_row_offsets, w.cache_lengths, max(1, w.total_ctx), 1)
    assert st == 0
    return bro[0], co[0]


def _partial(step, row, mask, out_dtype=torch.float32):
    """One plan row's attention with its lse, no earlier partial."""
    w = step.w
    kn, v = step.row_buffers(row)
    out = torch.full((w.total_q, w.heads, 128), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((w.total_q, w.heads), float("nan"), dtype=torch.float32, device="cuda")
    sc = step.scales or {}
    m.mla_prefill_ragged_lse(out, lse, step.q, kn, v, step.kv, 0, step.input_row_offsets,
                             step.buffer_row_offsets[row], step.cache_offsets[row], w.softmax_scale,
                             q_scale=sc.get("q"), k_nope_scale=sc.get("k_nope"), v_scale=sc.get("v"),
                             q_max_seq_len=w.max_q, mask=mask)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_null_mask_every_output(case, dtype):
    w = _workload(case, dtype, 600)
    say(f"null mask {dtype} case {CASES[case]}")
    step = PrefillStep(w, "cuda", mask="null")
    step.out.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    ref = oracle_full(w, bro[0], co[0], mask="null")
    assert report(step.out.float().cpu().numpy(), ref, BAR[dtype], f"null-{dtype}{case}") <= BAR[dtype]


@pytest.mark.parametrize("mask", ["causal", "null"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("case", [0, 1, 4])
def test_lse_and_fp32_output_every_output(case, dtype, mask):
    w = _workload(case, dtype, 620)
    say(f"lse {dtype} {mask} case {CASES[case]}")
    step = PrefillStep(w, "cuda", mask=mask)
    step.run()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    out32, lse = _partial(step, 0, mask)
    ref, ref_lse = oracle_full(w, bro[0], co[0], mask=mask, return_lse=True)
    assert report(out32.cpu().numpy(), ref, BAR[dtype], f"fp32out-{dtype}-{mask}{case}") <= BAR[dtype]
    assert report_lse(lse.cpu().numpy(), ref_lse, LSE_BAR[dtype], f"lse-{dtype}-{mask}{case}") <= LSE_BAR[dtype]
    # the bf16 output of the lse entry point is the plain entry point's, bit for bit
    out16, _ = _partial(step, 0, mask, torch.bfloat16)
    assert torch.equal(out16, step.out)
    # and the fp32 output rounds to it
    assert torch.equal(out32.to(torch.bfloat16), step.out)


MULTI = [
    dict(case=0, cap=300), dict(case=0, cap=97), dict(case=1, cap=512), dict(case=2, cap=64),
    dict(case=3, cap=200), dict(case=4, cap=128), dict(case=5, cap=700),
]


@pytest.mark.parametrize("mask", ["causal", "null"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("mc", range(len(MULTI)))
def test_rows_merged_every_output(mc, dtype, mask):
    """Capacity below the context: the per-row partials, merged in the attention's
    epilogue, equal the attention over every key."""
    case, cap = MULTI[mc]["case"], MULTI[mc]["cap"]
    w = _workload(case, dtype, 640)
    say(f"rows merged {dtype} {mask} case {CASES[case]} cap {cap}")
    step = PrefillStep(w, "cuda", cap=cap, mask=mask)
    assert step.rows >= 2
    # no initial contents are needed: every value read is written by an earlier row
    step.out.fill_(float("nan"))
    step.acc.fill_(float("nan"))
    step.lse.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    check_plan(step, w)
    bro1, co1 = _one_row_plan(w)
    ref = oracle_full(w, bro1, co1, mask=mask)
    got = step.out.float().cpu().numpy()
    assert report(got, ref, BAR[dtype], f"merged-{dtype}-{mask}-{mc}") <= BAR[dtype]
    # rerun: bit-identical
    first = step.out.clone()
    step.run()
    torch.cuda.synchronize()
    assert torch.equal(first, step.out)


@pytest.mark.parametrize("mask", ["causal", "null"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("mc", [0, 1, 3, 5])
def test_rows_chained_through_the_lse_entry_point(mc, dtype, mask):
    """The general entry point: row 0 writes an fp32 partial and lse, each later
    row merges into them in place (prev = output), the last writes bf16."""
    case, cap = MULTI[mc]["case"], MULTI[mc]["cap"]
    w = _workload(case, dtype, 680)
    step = PrefillStep(w, "cuda", cap=cap, mask=mask)
    step.plan()
    torch.cuda.synchronize()
    check_plan(step, w)
    acc = torch.full((w.total_q, w.heads, 128), float("nan"), device="cuda")
    lse = torch.full((w.total_q, w.heads), float("nan"), device="cuda")
    out = torch.full_like(step.out, float("nan"))
    final_lse = torch.full_like(lse, float("nan"))
    sc = step.scales or {}
    for r in range(step.rows):
        kn, v = step.row_buffers(r)
        last = r == step.rows - 1
        m.mla_prefill_ragged_lse(out if last else acc, final_lse if last else lse, step.q, kn, v, step.kv, 0,
                                 step.input_row_offsets, step.buffer_row_offsets[r], step.cache_offsets[r],
                                 w.softmax_scale, prev_output=None if r == 0 else acc,
                                 prev_lse=None if r == 0 else lse, q_scale=sc.get("q"),
                                 k_nope_scale=sc.get("k_nope"), v_scale=sc.get("v"), q_max_seq_len=w.max_q,
                                 mask=mask)
    torch.cuda.synchronize()
    bro1, co1 = _one_row_plan(w)
    ref, ref_lse = oracle_full(w, bro1, co1, mask=mask, return_lse=True)
    assert report(out.float().cpu().numpy(), ref, BAR[dtype], f"chain-{dtype}-{mask}-{mc}") <= BAR[dtype]
    assert report_lse(final_lse.cpu().numpy(), ref_lse, LSE_BAR[dtype], f"chain-lse-{dtype}-{mask}-{mc}") \
        <= LSE_BAR[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_row_mode_final_lse_and_fp32_output(dtype):
    """Row mode with the final log-sum-exp and an fp32 output."""
    w = _workload(0, dtype, 690)
    step = PrefillStep(w, "cuda", cap=120)
    step.plan()
    torch.cuda.synchronize()
    check_plan(step, w)
    out = torch.full((w.total_q, w.heads, 128), float("nan"), device="cuda")
    lse = torch.full((w.total_q, w.heads), float("nan"), device="cuda")
    sc = step.scales or {}
    for r in range(step.rows):
        kn, v = step.row_buffers(r)
        m.mla_prefill_ragged_row(out, step.acc, step.lse, step.q, kn, v, step.kv, 0, step.input_row_offsets,
                                 step.buffer_row_offsets[r], step.cache_offsets[r], w.softmax_scale, lse=lse,
                                 q_scale=sc.get("q"), k_nope_scale=sc.get("k_nope"), v_scale=sc.get("v"),
                                 q_max_seq_len=w.max_q)
    torch.cuda.synchronize()
    bro1, co1 = _one_row_plan(w)
    ref, ref_lse = oracle_full(w, bro1, co1, return_lse=True)
    assert report(out.cpu().numpy(), ref, BAR[dtype], f"rowmode-fp32-{dtype}") <= BAR[dtype]
    assert report_lse(lse.cpu().numpy(), ref_lse, LSE_BAR[dtype], f"rowmode-lse-{dtype}") <= LSE_BAR[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_row_partials_and_final_lse(dtype):
    """Each row's partial (fp32 output + lse, -inf where a query sees no key of
    the row) against the oracle on that row, and the merged lse against the
    oracle's lse over every key."""
    w = _workload(0, dtype, 660)
    step = PrefillStep(w, "cuda", cap=150)
    step.plan()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    saw_empty = False
    acc = lse_acc = None
    for r in range(step.rows):
        kn, v = step.row_buffers(r)
        o, lse = _partial(step, r, "causal")
        ref, ref_lse = oracle.mla_prefill_ragged(
            w.q, kn.cpu()[:max(1, int(bro[r][-1]))], v.cpu()[:max(1, int(bro[r][-1]))], w.cache, 0, w.page_table,
            w.spec.page_size, w.spec.rope_col, w.cache_lengths, w.input_row_offsets, bro[r], co[r],
            w.softmax_scale, scales=w.scales, return_lse=True)
        assert report(o.cpu().numpy(), ref, BAR[dtype], f"row{r}-{dtype}") <= BAR[dtype]
        assert report_lse(lse.cpu().numpy(), ref_lse, LSE_BAR[dtype], f"row{r}-lse-{dtype}") <= LSE_BAR[dtype]
        empty = np.isneginf(ref_lse)
        saw_empty |= bool(empty.any())
        assert np.array_equal(o.cpu().numpy()[empty], np.zeros((int(empty.sum()), 128)))
        if acc is None:
            acc, lse_acc = o, lse
        else:
            m.mla_prefill_merge(acc, lse_acc, acc, lse_acc, o, lse)     # in place into the accumulator
    torch.cuda.synchronize()
    assert saw_empty
    bro1, co1 = _one_row_plan(w)
    ref, ref_lse = oracle_full(w, bro1, co1, return_lse=True)
    assert report(acc.cpu().numpy(), ref, BAR[dtype], f"merged-standalone-{dtype}") <= BAR[dtype]
    assert report_lse(lse_acc.cpu().numpy(), ref_lse, LSE_BAR[dtype], f"merged-lse-{dtype}") <= LSE_BAR[dtype]


def test_standalone_merge_matches_oracle_merge():
    g = torch.Generator().manual_seed(5)
    T, H = 300, 7
    o_a = torch.randn((T, H, 128), generator=g) * 2
    o_b = torch.randn((T, H, 128), generator=g)
    l_a = torch.randn((T, H), generator=g) * 6
    l_b = torch.randn((T, H), generator=g) * 6
    # empty sides: -inf lse, NaN output that must not be read
    l_a[:20] = float("-inf")
    o_a[:20] = float("nan")
    l_b[10:40] = float("-inf")
    o_b[10:40] = float("nan")
    l_b[50:60] = l_a[50:60]                                   # equal weights
    l_b[60:70] = l_a[60:70] + 80.0                            # one side dominates
    ref_o, ref_l = oracle.merge_partials(
        np.nan_to_num(o_a.double().numpy()), l_a.double().numpy(), np.nan_to_num(o_b.double().numpy()),
        l_b.double().numpy())
    da, db, dla, dlb = (x.cuda() for x in (o_a, o_b, l_a, l_b))
    out = torch.full((T, H, 128), float("nan"), device="cuda")
    lse = torch.full((T, H), float("nan"), device="cuda")
    m.mla_prefill_merge(out, lse, da, dla, db, dlb)
    out16 = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    m.mla_prefill_merge(out16, None, da, dla, db, dlb)
    torch.cuda.synchronize()
    got_o, got_l = out.cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.isfinite(got_o).all()
    assert report(got_o, ref_o, MERGE_BAR, "merge-fp32") <= MERGE_BAR
    assert report_lse(got_l, ref_l, MERGE_BAR, "merge-lse") <= MERGE_BAR
    # one side empty: the other side passes through exactly; both empty: zeros, -inf
    assert torch.equal(out[:10].cpu(), o_b[:10]) and torch.equal(lse[:10].cpu(), l_b[:10])
    assert torch.equal(out[20:40].cpu(), o_a[20:40]) and torch.equal(lse[20:40].cpu(), l_a[20:40])
    assert torch.equal(out[10:20].cpu(), torch.zeros(10, H, 128)) and bool(torch.isneginf(lse[10:20]).all())
    # the bf16 output is the fp32 result rounded
    assert torch.equal(out16, out.to(torch.bfloat16))


@pytest.mark.parametrize("name,cap", [("dsv3", 2000), ("prefix", 16384), ("fp8", 12288)])
def test_full_size_rows_merged_sampled(name, cap):
    w = get_workload(name)
    say(f"{name} in rows of {cap}: B={w.batch} T={w.total_q} C={w.total_ctx} H={w.heads}")
    step = PrefillStep(w, "cuda", cap=cap)
    assert step.rows >= 2
    step.out.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    check_plan(step, w)
    out = step.out.float()
    assert bool(torch.isfinite(out).all())
    bro1, co1 = _one_row_plan(w)
    rows = sample_rows(w, 160, seed=9)
    ref = oracle_rows(w, rows, bro1, co1)
    got = np.stack([out[t, h].cpu().numpy() for t, h in rows])
    bar = BAR[w.spec.dtype]
    assert report(got, ref, bar, f"{name}-rows{step.rows}") <= bar


@pytest.mark.parametrize("name", ["dsv3", "fp8"])
def test_full_size_null_mask_sampled(name):
    w = get_workload(name)
    step = PrefillStep(w, "cuda", mask="null")
    step.out.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    out = step.out.float()
    assert bool(torch.isfinite(out).all())
    rows = sample_rows(w, 160, seed=10)
    ref = oracle_rows(w, rows, bro[0], co[0], mask="null")
    got = np.stack([out[t, h].cpu().numpy() for t, h in rows])
    bar = BAR[w.spec.dtype]
    assert report(got, ref, bar, f"{name}-null") <= bar
