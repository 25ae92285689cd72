"""Split-query attention on the GPU (q_nope + q_rope, K_rope paged or
contiguous) against the float64 oracle.

Bars (the accuracy bars of the output): max |gpu - oracle| <= 1e-2 for bf16 inputs and
<= 6e-2 for float8_e4m3fn q_nope / K / V.  The split bf16 query runs the same
arithmetic as the one-tensor query, so those outputs must also match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import mla_ragged_paged_amd as m
from mla_ragged_paged_amd import workloads
from mla_ragged_paged_amd.pipeline import PrefillStep
from tests.gpu_util import check_plan, get_workload, report, report_lse, sample_rows, say

pytestmark = pytest.mark.gpu

BAR = {"bf16": 1e-2, "fp8": 6e-2}
LSE_BAR = {"bf16": 1e-2, "fp8": 6.5e-2}

CASES = [
    dict(n=[130, 1, 257, 0, 64], p=[0, 300, 77, 5, 0], heads=4, ps=16),
    dict(n=[200], p=[1000], heads=3, ps=128),
    dict(n=[150, 70], p=[33, 0], heads=2, ps=48),
    dict(n=[130, 40, 0, 200], p=[10, 0, 5, 64], heads=16, ps=16),
]


def _workload(case, dtype, seed_base=800):
    kw = CASES[case]
    spec = workloads.Spec("split", len(kw["n"]), (0, 0), (0, 0), kw["heads"], kw["ps"], True, dtype,
                          row_width=576, rope_col=512, seed=seed_base + case)
    return workloads.build(spec, n=kw["n"], p=kw["p"])


def _gathered_rope(w, bro, co):
    """K_rope rows laid out like K / V (one-row plan), read off the paged cache on the host."""
    rows = torch.zeros((max(1, int(bro[-1])), 1, 64), dtype=w.cache.dtype)
    for b in range(w.batch):
        for j in range(int(bro[b + 1]) - int(bro[b])):
            pos = int(co[b]) + j
            page = int(w.page_table[b][pos // w.spec.page_size])
            rows[int(bro[b]) + j, 0] = w.cache[0, page, pos % w.spec.page_size, 0, 512:576]
    return rows


def _split_call(step, q_nope, q_rope, out, rope_rows=None, lse=None, mask="causal"):
    w = step.w
    sc = step.scales or {}
    m.mla_prefill_ragged_split(out, q_nope, q_rope, step.k_nope, step.v, step.kv, 0, step.input_row_offsets,
                               step.buffer_row_offsets[0], step.cache_offsets[0], w.softmax_scale,
                               q_scale=sc.get("q"), k_scales=sc.get("k_nope"), v_scale=sc.get("v"),
                               k_rope_rows=rope_rows, lse=lse, q_max_seq_len=w.max_q, mask=mask)
    torch.cuda.synchronize()


def _oracle(w, bro, co, q_nope, q_rope, rope_rows=None, mask="causal", lse=False):
    return oracle.mla_prefill_ragged_split(
        q_nope, q_rope, w.k_nope, w.v, w.cache_lengths, w.input_row_offsets, bro, co, w.softmax_scale,
        k_rope_rows=rope_rows, cache=w.cache, layer_idx=0, page_table=w.page_table, page_size=w.spec.page_size,
        rope_col=w.spec.rope_col, scales=w.scales, mask=mask, return_lse=lse)


@pytest.mark.parametrize("mask", ["causal", "null"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_bf16_split_equals_one_tensor_query(case, mask):
    """bf16: the split call (paged and contiguous K_rope) gives the one-tensor call's output bit for bit."""
    w = _workload(case, "bf16")
    say(f"bf16 split {mask} case {CASES[case]}")
    step = PrefillStep(w, "cuda", mask=mask)
    step.run()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    q_nope, q_rope = workloads.split_query(w)
    out = torch.full_like(step.out, float("nan"))
    _split_call(step, q_nope.cuda(), q_rope.cuda(), out, mask=mask)
    assert torch.equal(out, step.out)
    out.fill_(float("nan"))
    _split_call(step, q_nope.cuda(), q_rope.cuda(), out, rope_rows=_gathered_rope(w, bro[0], co[0]).cuda(),
                mask=mask)
    assert torch.equal(out, step.out)
    ref = _oracle(w, bro[0], co[0], q_nope, q_rope, mask=mask)
    assert report(out.float().cpu().numpy(), ref, BAR["bf16"], f"split-bf16-{mask}{case}") <= BAR["bf16"]


@pytest.mark.parametrize("mask", ["causal", "null"])
@pytest.mark.parametrize("rope", ["paged-fp8", "contiguous-bf16", "paged-bf16"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_fp8_split_every_output(case, rope, mask):
    """e4m3 q_nope / K / V with their scales, bf16 q_rope; K_rope from the e4m3 cache
    (converted to bf16 in the kernel), from contiguous bf16 rows, or from a bf16 cache."""
    w = _workload(case, "fp8")
    say(f"fp8 split {rope} {mask} case {CASES[case]}")
    step = PrefillStep(w, "cuda", mask=mask)
    step.plan()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    q_nope, q_rope = workloads.split_query(w)
    rope_rows = None
    w_ref = w
    if rope == "contiguous-bf16":
        rope_rows = workloads.draw_rope_rows(max(1, w.total_ctx), seed=w.spec.seed)
    elif rope == "paged-bf16":
        # the same shapes, seed and page table with a bf16 cache
        wb = workloads.build(workloads.Spec("split", w.batch, (0, 0), (0, 0), w.heads, w.spec.page_size, True,
                                            "bf16", row_width=576, rope_col=512, seed=w.spec.seed),
                             n=w.n.tolist(), p=w.p.tolist())
        assert np.array_equal(wb.page_table, w.page_table)
        step.kv = m.PagedCache(wb.cache.cuda(), step.page_table, step.cache_lengths, 512)
        w_ref = workloads.Workload(**{**w.__dict__, "cache": wb.cache,
                                      "scales": dict(w.scales, k_rope=1.0)})
    out = torch.full((w.total_q, w.heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.total_q, w.heads), float("nan"), dtype=torch.float32, device="cuda")
    _split_call(step, q_nope.cuda(), q_rope.cuda(), out, rope_rows=None if rope_rows is None else rope_rows.cuda(),
                lse=lse, mask=mask)
    if rope == "paged-bf16":
        # the oracle decodes e4m3 codes only for fp8 operands: hand it the bf16 cache values
        ref, ref_lse = oracle.mla_prefill_ragged_split(
            q_nope, q_rope, w.k_nope, w.v, w.cache_lengths, w.input_row_offsets, bro[0], co[0], w.softmax_scale,
            k_rope_rows=_gathered_rope(w_ref, bro[0], co[0]).to(torch.float64).numpy(), scales=w.scales,
            mask=mask, return_lse=True)
    else:
        ref, ref_lse = _oracle(w, bro[0], co[0], q_nope, q_rope, rope_rows=rope_rows, mask=mask, lse=True)
    label = f"split-fp8-{rope}-{mask}{case}"
    assert report(out.float().cpu().numpy(), ref, BAR["fp8"], label) <= BAR["fp8"]
    assert report_lse(lse.cpu().numpy(), ref_lse, LSE_BAR["fp8"], label + "-lse") <= LSE_BAR["fp8"]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("scale", [-0.0721687836, 0.0])
def test_split_scale_sign_and_zero(dtype, scale):
    w = _workload(0, dtype, seed_base=820)
    w.softmax_scale = scale
    step = PrefillStep(w, "cuda")
    step.plan()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    q_nope, q_rope = workloads.split_query(w)
    out = torch.full((w.total_q, w.heads, 128), float("nan"), dtype=torch.float32, device="cuda")
    _split_call(step, q_nope.cuda(), q_rope.cuda(), out)
    ref = _oracle(w, bro[0], co[0], q_nope, q_rope)
    assert report(out.cpu().numpy(), ref, BAR[dtype], f"split-{dtype}-scale{scale}") <= BAR[dtype]


@pytest.mark.parametrize("name,rope", [("fp8", "paged-fp8"), ("fp8", "contiguous-bf16"), ("dsv3", "paged")])
def test_full_size_split_sampled(name, rope):
    w = get_workload(name)
    say(f"{name} split ({rope}): B={w.batch} T={w.total_q} C={w.total_ctx}")
    step = PrefillStep(w, "cuda")
    step.plan()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    q_nope, q_rope = workloads.split_query(w)
    rope_rows = workloads.draw_rope_rows(w.total_ctx, seed=w.spec.seed) if rope.startswith("contiguous") else None
    out = torch.full((w.total_q, w.heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    _split_call(step, q_nope.cuda(), q_rope.cuda(), out, rope_rows=None if rope_rows is None else rope_rows.cuda())
    got_all = out.float()
    assert bool(torch.isfinite(got_all).all())
    rows = sample_rows(w, 120, seed=12)
    ref = oracle.mla_prefill_rows_split(
        rows, q_nope, q_rope, w.k_nope, w.v, w.cache_lengths, w.input_row_offsets, bro[0], co[0], w.softmax_scale,
        k_rope_rows=rope_rows, cache=w.cache, layer_idx=0, page_table=w.page_table, page_size=w.spec.page_size,
        rope_col=w.spec.rope_col, scales=w.scales)
    got = np.stack([got_all[t, h].cpu().numpy() for t, h in rows])
    bar = BAR[w.spec.dtype]
    assert report(got, ref, bar, f"{name}-split-{rope}") <= bar


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("heads", [8, 24])
def test_split_one_plan_row_of_several(dtype, heads):
    """A later row of a multi-row plan (cache_offsets non-zero, keys after some
    queries) with 8 and 24 heads, paged K_rope, against the oracle on that row."""
    spec = workloads.Spec("splitrow", 3, (0, 0), (0, 0), heads, 16, True, dtype, row_width=576, rope_col=512,
                          seed=840 + heads)
    w = workloads.build(spec, n=[90, 20, 150], p=[60, 0, 200])
    step = PrefillStep(w, "cuda", cap=160)
    step.plan()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    q_nope, q_rope = workloads.split_query(w)
    sc = step.scales or {}
    for r in (1, step.rows - 1):
        kn, v = step.row_buffers(r)
        out = torch.full((w.total_q, w.heads, 128), float("nan"), dtype=torch.float32, device="cuda")
        m.mla_prefill_ragged_split(out, q_nope.cuda(), q_rope.cuda(), kn, v, step.kv, 0, step.input_row_offsets,
                                   step.buffer_row_offsets[r], step.cache_offsets[r], w.softmax_scale,
                                   q_scale=sc.get("q"), k_scales=sc.get("k_nope"), v_scale=sc.get("v"),
                                   q_max_seq_len=w.max_q)
        torch.cuda.synchronize()
        used = max(1, int(bro[r][-1]))
        ref = oracle.mla_prefill_ragged_split(
            q_nope, q_rope, kn[:used].cpu(), v[:used].cpu(), w.cache_lengths, w.input_row_offsets, bro[r], co[r],
            w.softmax_scale, cache=w.cache, layer_idx=0, page_table=w.page_table, page_size=w.spec.page_size,
            rope_col=w.spec.rope_col, scales=w.scales)
        assert report(out.cpu().numpy(), ref, BAR[dtype], f"splitrow-{dtype}-h{heads}-r{r}") <= BAR[dtype]
