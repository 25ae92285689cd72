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
    # query tiles past the first straddle the diagonal with every row seeing >= 128
    # keys (e4m3 P.V there); the first tile's rows see fewer (bf16 P.V)
    dict(n=[513], p=[0], heads=2, ps=128, width=576, rope=512),
    dict(n=[130, 40, 0, 200], p=[10, 0, 5, 64], heads=16, ps=16, width=576, rope=512),
    dict(n=[300], p=[20], heads=8, ps=64, width=576, rope=512),
    dict(n=[90, 200, 17], p=[0, 64, 300], heads=40, ps=64, width=576, rope=512),  # 5 heads per XCD
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


@pytest.mark.parametrize("p", [95, 96, 127])
def test_fp8_straddling_tiles_either_side_of_the_key_count_threshold(p):
    """A straddling tile takes e4m3 weights and P.V when every row of its wave
    sees at least 128 keys, else bf16 ones.  With a prefix of 95 keys the first
    wave's first row sees 96 keys (bf16) and the second wave's first row exactly
    128 (e4m3); with 96 the second wave's first row sees 129; with 127 the first
    wave's first row sees exactly 128, so every wave takes e4m3.  Every output
    against the oracle."""
    spec = workloads.Spec("thr8", 1, (0, 0), (0, 0), 2, 32, True, "fp8", row_width=576, rope_col=512, seed=200 + p)
    w = workloads.build(spec, n=[300], p=[p])
    step = _run(w)
    bro, co, _ = check_plan(step, w)
    ref = oracle_full(w, bro[0], co[0])
    assert report(step.out.float().cpu().numpy(), ref, BAR_FP8, f"fp8thr{p}") <= BAR_FP8


@pytest.mark.parametrize("scale", [-0.0721687836, 0.0])
def test_fp8_scale_sign_and_zero(scale):
    spec = workloads.Spec("scale8", 2, (0, 0), (0, 0), 3, 16, True, "fp8", row_width=576, rope_col=512, seed=190)
    w = workloads.build(spec, n=[150, 33], p=[20, 0])
    w.softmax_scale = scale
    step = _run(w)
    bro, co, _ = check_plan(step, w)
    ref = oracle_full(w, bro[0], co[0])
    assert report(step.out.float().cpu().numpy(), ref, BAR_FP8, f"fp8scale{scale}") <= BAR_FP8


def _log2_scores(w, b, h):
    """Scores of sequence b, head h in log2 units (scale * q.k * log2 e) on the exactly
    dequantised inputs, [n_b, p_b + n_b] (keys of the sequence in cache order)."""
    import oracle
    t0, n = int(w.input_row_offsets[b]), int(w.n[b])
    g0 = int((w.n[:b] + w.p[:b]).sum())
    ctx = int(w.p[b]) + n
    codes = lambda x: x.view(torch.uint8).cpu().numpy()
    q = oracle.dequantize_e4m3fn(codes(w.q[t0:t0 + n, h]), w.scales["q"])
    kn = oracle.dequantize_e4m3fn(codes(w.k_nope[g0:g0 + ctx, h]), w.scales["k_nope"])
    kr_codes = oracle.rope_rows(w.cache.view(torch.uint8), w.spec.layer_idx, w.page_table, w.spec.page_size,
                                w.spec.rope_col, b, range(ctx))
    kr = oracle.dequantize_e4m3fn(kr_codes, w.scales["k_rope"])
    return w.softmax_scale * (q @ np.concatenate([kn, kr], axis=1).T) * np.log2(np.e)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("scale", [2.0, -2.0])
def test_fp8_running_reference_moves_on_fully_visible_tiles(scale, causal):
    """The kernel takes a fully visible key tile's e4m3 weights against its running
    reference and keeps them when every row's sum of them is at most 2^8 (so no
    weight exceeds the e4m3 range); otherwise it takes the tile max, moves the
    reference up to it and takes the weights again.  The reference is always the
    score of a key seen earlier, so a tile whose weights against the exact running
    maximum of the earlier keys sum to more than 2^8 takes that second pass
    whatever the reference is.  A large softmax scale makes such tiles, some with
    a single weight beyond 2^8 (a jump of the maximum by more than 8 in log2
    units), after earlier tiles have been summed: under the causal mask on the
    matrix core, under the null mask on the VALU.  The case first shows on the
    oracle's scores that they occur, then compares every output."""
    spec = workloads.Spec("rescale8", 2, (0, 0), (0, 0), 2, 128, True, "fp8", row_width=576, rope_col=512,
                          seed=196)
    w = workloads.build(spec, n=[160, 40], p=[700, 90])
    w.softmax_scale = scale
    x = _log2_scores(w, 0, 0)
    p0 = int(w.p[0])
    ctx = x.shape[1]
    second, jumps = 0, 0
    for i in range(x.shape[0]):
        wave_first = p0 + 32 * (i // 32)              # first query position of the row's wave
        last = p0 + i if causal else ctx - 1          # the row's last visible key
        m = None
        for kt in range(last // 64 + 1):
            keys = x[i, kt * 64:min((kt + 1) * 64, last + 1)]
            mx = keys.max()
            full = (kt + 1) * 64 <= ctx and (not causal or kt * 64 + 63 <= wave_first)
            if m is not None and full:
                second += int(np.exp2(keys - m).sum() > 256.0)
                jumps += int(mx > m + 8.0)
            m = mx if m is None else max(m, mx)
    say(f"fp8 scale {scale} causal {causal}: {second} second passes on fully visible tiles, "
        f"{jumps} of them with a weight beyond 2^8")
    assert jumps > 0 and second > jumps
    mask = "causal" if causal else "null"
    step = PrefillStep(w, "cuda", mask=mask)
    step.run()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    ref = oracle_full(w, bro[0], co[0], mask=mask)
    assert report(step.out.float().cpu().numpy(), ref, BAR_FP8, f"fp8rescale{scale}{mask}") <= BAR_FP8


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
