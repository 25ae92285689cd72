"""float8_e4m3fn attention on the GPU against the float64 oracle.

Inputs are e4m3 codes with one fp32 scale per tensor; the oracle evaluates the
definition on the exactly dequantised values.  Bar: max |gpu - oracle| <= 6e-2
(fp8 inputs, bf16 output) on N(0, 1)-derived inputs.
"""
import numpy as np
import pytest
import torch

from mla_ragged_paged_amd import workloads
from mla_ragged_paged_amd.pipeline import PrefillStep
from tests.gpu_util import check_plan, get_workload, oracle_full, oracle_rows, report, sample_rows, say

pytestmark = pytest.mark.gpu

BAR_FP8 = 6e-2

SMALL_FP8 = [
    dict(n=[130, 1, 257, 0, 64], p=[0, 300, 77, 5, 0], heads=4, ps=16, width=576, rope=512),
    dict(n=[200], p=[1000], heads=3, ps=128, width=576, rope=512),
    dict(n=[150, 70], p=[33, 0], heads=2, ps=48, width=576, rope=512),
    dict(n=[40, 7], p=[10, 3], heads=2, ps=1, width=64, rope=0),
    dict(n=[513], p=[0], heads=2, ps=128, width=576, rope=512),
    dict(n=[130, 40, 0, 200], p=[10, 0, 5, 64], heads=16, ps=16, width=576, rope=512),
    dict(n=[300], p=[20], heads=8, ps=64, width=576, rope=512),
]


def _run(w, cap=None):
    step = PrefillStep(w, "cuda", cap=cap)
    step.run()
    torch.cuda.synchronize()
    return step


@pytest.mark.parametrize("case", range(len(SMALL_FP8)))
def test_fp8_small_ragged_every_output(case):
    kw = SMALL_FP8[case]
    say(f"fp8 small ragged case {kw}")
    spec = workloads.Spec("small8", len(kw["n"]), (0, 0), (0, 0), kw["heads"], kw["ps"], True, "fp8",
                          row_width=kw["width"], rope_col=kw["rope"], seed=170 + case)
    w = workloads.build(spec, n=kw["n"], p=kw["p"])
    step = _run(w)
    bro, co, _ = check_plan(step, w)
    ref = oracle_full(w, bro[0], co[0])
    assert report(step.out.float().cpu().numpy(), ref, BAR_FP8, f"fp8small{case}") <= BAR_FP8


@pytest.mark.parametrize("scale", [-0.0721687836, 0.0])
def test_fp8_scale_sign_and_zero(scale):
    spec = workloads.Spec("scale8", 2, (0, 0), (0, 0), 3, 16, True, "fp8", row_width=576, rope_col=512, seed=190)
    w = workloads.build(spec, n=[150, 33], p=[20, 0])
    w.softmax_scale = scale
    step = _run(w)
    bro, co, _ = check_plan(step, w)
    ref = oracle_full(w, bro[0], co[0])
    assert report(step.out.float().cpu().numpy(), ref, BAR_FP8, f"fp8scale{scale}") <= BAR_FP8


def test_fp8_workload_sampled():
    w = get_workload("fp8")
    say(f"fp8: B={w.batch} T={w.total_q} C={w.total_ctx} H={w.heads} scales={w.scales}")
    step = _run(w)
    bro, co, _ = check_plan(step, w)
    step.out.fill_(float("nan"))        # every output must be written by this launch
    step.attention(0)
    torch.cuda.synchronize()
    out = step.out.float()
    assert bool(torch.isfinite(out).all())
    rows = sample_rows(w, 160, seed=11)
    ref = oracle_rows(w, rows, bro[0], co[0])
    got = np.stack([out[t, h].cpu().numpy() for t, h in rows])
    assert report(got, ref, BAR_FP8, "fp8") <= BAR_FP8


def test_fp8_bit_identical_reruns():
    w = get_workload("fp8")
    step = _run(w)
    first = step.out.clone()
    step.run()
    torch.cuda.synchronize()
    assert torch.equal(first, step.out)
