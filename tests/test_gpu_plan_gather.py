"""Plan and gather on the GPU, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from mla_ragged_paged_amd import workloads
from mla_ragged_paged_amd.pipeline import PrefillStep
from tests.gpu_util import check_plan, get_workload, host_u32, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "dsv3", "prefix", "long", "fp8"])
def test_plan_and_gather_on_workloads(name):
    spec = workloads.SPECS[name]
    say(f"plan+gather {name}: {spec.description}")
    w = get_workload(name)
    step = PrefillStep(w, "cuda", gather_cols=(0, w.cache.shape[4]))   # whole cache rows
    step.plan()
    step.gather(0)
    torch.cuda.synchronize()
    bro, co, bl = check_plan(step, w)
    got = step.gathered.view(torch.uint8) if w.spec.dtype == "fp8" else step.gathered.view(torch.int16)
    init = np.zeros(tuple(got.shape), dtype=np.int64)
    cache_bits = (w.cache.view(torch.uint8) if w.spec.dtype == "fp8" else w.cache.view(torch.int16)).numpy()
    ref = oracle.gather(cache_bits.astype(np.int64), 0, w.page_table, w.spec.page_size, bro[0], co[0], 0,
                        w.cache.shape[4], init)
    assert np.array_equal(got.cpu().numpy().astype(np.int64), ref)


# narrow copies (a thread per 16-byte unit) and wide ones (>= 32 units: a wave per slot)
ADVERSARIAL = [
    dict(n=[5, 0, 9, 1], p=[3, 7, 0, 0], cap=4),       # many rows, an empty sequence, straddling rows
    dict(n=[1, 1, 1], p=[0, 0, 0], cap=1),             # capacity one
    dict(n=[40, 3], p=[100, 17], cap=37),              # prefix split over rows
    dict(n=[0, 0], p=[0, 0], cap=8),                   # nothing at all
    dict(n=[5, 0, 9, 1], p=[3, 7, 0, 0], cap=4, width=576, cols=(0, 576), ps=16),     # wide rows, 16-byte units
    dict(n=[40, 0, 3, 70], p=[100, 0, 17, 5], cap=37, width=576, cols=(4, 300), ps=8),  # wide, 8-byte units
    dict(n=[130, 1], p=[0, 200], cap=331, width=320, cols=(0, 320), ps=3),            # wide, one row, odd pages
]


@pytest.mark.parametrize("case", range(len(ADVERSARIAL)))
def test_plan_and_gather_adversarial(case):
    kw = ADVERSARIAL[case]
    say(f"plan+gather adversarial {kw}")
    width = kw.get("width", 96)
    cols = kw.get("cols", (8, 40))
    spec = workloads.Spec("adv", len(kw["n"]), (0, 0), (0, 0), 2, kw.get("ps", 4), True, "bf16", row_width=width,
                          rope_col=width - 64, seed=50 + case)
    w = workloads.build(spec, n=kw["n"], p=kw["p"])
    step = PrefillStep(w, "cuda", cap=kw["cap"], gather_cols=cols)
    step.plan()
    torch.cuda.synchronize()
    bro, co, bl = check_plan(step, w)
    bits = w.cache.view(torch.int16).numpy().astype(np.int64)
    for r in range(step.rows):
        step.gathered.fill_(-3)
        step.gather(r)
        torch.cuda.synchronize()
        init = np.full((step.cap, cols[1]), -3, dtype=np.int64)
        # -3 as bf16 bits: compare raw 16-bit patterns
        fill_bits = int(torch.tensor([-3.0]).to(torch.bfloat16).view(torch.int16)[0])
        init[:] = fill_bits
        ref = oracle.gather(bits, 0, w.page_table, w.spec.page_size, bro[r], co[r], cols[0], cols[1], init)
        got = step.gathered.view(torch.int16).cpu().numpy().astype(np.int64)
        assert np.array_equal(got, ref), f"row {r}"


def test_plan_status_flag_when_rows_are_too_few():
    spec = workloads.Spec("flag", 2, (0, 0), (0, 0), 2, 4, False, "bf16", row_width=64, rope_col=0, seed=60)
    w = workloads.build(spec, n=[6, 6], p=[2, 2])
    step = PrefillStep(w, "cuda", cap=4)
    # hand the plan fewer rows than the 4 it needs
    import mla_ragged_paged_amd as m
    bro = torch.zeros((2, 3), dtype=torch.int32, device="cuda")
    co = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    bl = torch.zeros((2,), dtype=torch.int32, device="cuda")
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    m.mla_prefill_plan(step.input_row_offsets, step.kv, 0, 4, bro, co, bl, st)
    torch.cuda.synchronize()
    ebro, eco, ebl, est = oracle.plan(w.input_row_offsets, w.cache_lengths, 4, 2)
    assert est == 1 and int(st.cpu()[0]) == 1
    assert np.array_equal(host_u32(bro), ebro) and np.array_equal(host_u32(co), eco)
    assert np.array_equal(bl.cpu().numpy(), ebl)
