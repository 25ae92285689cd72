"""Latent up-projection on the GPU (K_nope / V of a buffer row from the latent
cache) against the float64 oracle, alone and followed by the attention.

Bar for K_nope / V, derived from the arithmetic: bf16 x bf16 products are exact
in fp32 and the 512-term fp32 sum adds at most ~5e-4 on these N(0, 1)-scaled
values; the result is rounded to bf16 (half an ulp = 2^-9 relative).  So
|gpu - oracle| <= 2^-8 |oracle| + 5e-4 element by element.  The attention that
consumes them keeps the bf16 accuracy bar, 1e-2, against the oracle's attention
over the oracle's K_nope / V rounded to bf16 -- the type the attention takes
them in (a value on a rounding boundary may round the other way on the GPU,
a one-ulp input difference far inside the bar).
"""
import numpy as np
import pytest
import torch

import oracle
import mla_ragged_paged_amd as m
from mla_ragged_paged_amd import workloads
from mla_ragged_paged_amd.pipeline import PrefillStep
from tests.gpu_util import check_plan, get_workload, oracle_rows, report, sample_rows, say

pytestmark = pytest.mark.gpu

REL, ABS = 2.0 ** -8, 5e-4

CASES = [
    dict(n=[130, 1, 257, 0, 64], p=[0, 300, 77, 5, 0], heads=4, ps=16, cap=None, dim=512, col=0),
    dict(n=[200], p=[1000], heads=3, ps=128, cap=500, dim=512, col=0),          # several plan rows
    dict(n=[150, 70], p=[33, 0], heads=2, ps=48, cap=None, dim=512, col=0),     # page size not a power of two
    dict(n=[40, 7], p=[10, 3], heads=5, ps=1, cap=23, dim=128, col=64),         # one token per page, narrow latent
    dict(n=[130, 40, 0, 200], p=[10, 0, 5, 64], heads=16, ps=16, cap=300, dim=512, col=0),
    dict(n=[0, 90, 0, 33], p=[0, 0, 0, 500], heads=8, ps=64, cap=1000, dim=256, col=256),   # empty contexts, spare slots
    dict(n=[300, 5], p=[700, 0], heads=12, ps=32, cap=257, dim=512, col=0),     # 12 heads, tiles past the fill
]


def _workload(case, seed_base=900):
    kw = CASES[case]
    spec = workloads.Spec("latent", len(kw["n"]), (0, 0), (0, 0), kw["heads"], kw["ps"], True, "bf16",
                          row_width=576, rope_col=512, seed=seed_base + case)
    return workloads.build(spec, n=kw["n"], p=kw["p"])


def _check(got, ref, label):
    got = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    excess = float((err - (REL * np.abs(ref) + ABS)).max()) if err.size else -1.0
    say(f"[{label}] max|gpu-oracle| = {float(err.max()) if err.size else 0.0:.3e}; worst margin to the bar "
        f"{-excess:.3e}; values = {err.size}")
    assert excess <= 0.0


@pytest.mark.parametrize("case", range(len(CASES)))
def test_latent_up_every_slot(case):
    kw = CASES[case]
    w = _workload(case)
    say(f"latent up case {kw}")
    W = workloads.draw_kv_b_weight(w.heads, kw["dim"], seed=w.spec.seed)
    step = PrefillStep(w, "cuda", cap=kw["cap"], kv_b_weight=W, latent_col=kw["col"])
    step.plan()
    torch.cuda.synchronize()
    bro, co, bl = check_plan(step, w)
    for r in range(step.rows):
        step.kn_buf.fill_(float("nan"))
        step.v_buf.fill_(float("nan"))
        step.latent_up(r)
        torch.cuda.synchronize()
        used = int(bro[r][-1])
        k_ref, v_ref = oracle.latent_up(w.cache, 0, w.page_table, w.spec.page_size, bro[r], co[r], kw["col"],
                                        kw["dim"], W, w.heads, step.cap)
        _check(step.kn_buf[:used], k_ref[:used], f"latent{case}-row{r}-k")
        _check(step.v_buf[:used], v_ref[:used], f"latent{case}-row{r}-v")
        # slots past the row's fill are not written
        assert bool(torch.isnan(step.kn_buf[used:].float()).all()) and bool(torch.isnan(step.v_buf[used:].float()).all())


@pytest.mark.parametrize("case", [0, 1, 4])
def test_latent_then_attention_every_output(case):
    """plan -> latent decompression -> attention (row mode over several rows) equals
    the oracle's attention over the oracle's K_nope / V of one row holding every key."""
    kw = CASES[case]
    w = _workload(case, seed_base=920)
    W = workloads.draw_kv_b_weight(w.heads, kw["dim"], seed=w.spec.seed)
    step = PrefillStep(w, "cuda", cap=kw["cap"], kv_b_weight=W, latent_col=kw["col"])
    step.out.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    check_plan(step, w)
    bro1, co1, _, _ = oracle.plan(w.input_row_offsets, w.cache_lengths, max(1, w.total_ctx), 1)
    k_ref, v_ref = oracle.latent_up(w.cache, 0, w.page_table, w.spec.page_size, bro1[0], co1[0], kw["col"],
                                    kw["dim"], W, w.heads, max(1, w.total_ctx))
    k_ref, v_ref = (torch.from_numpy(x).to(torch.bfloat16) for x in (k_ref, v_ref))
    ref = oracle.mla_prefill_ragged(w.q, k_ref, v_ref, w.cache, 0, w.page_table, w.spec.page_size, w.spec.rope_col,
                                    w.cache_lengths, w.input_row_offsets, bro1[0], co1[0], w.softmax_scale)
    assert report(step.out.float().cpu().numpy(), ref, 1e-2, f"latent-attn{case}") <= 1e-2


def test_full_size_latent_up_sampled():
    """The dsv3-shaped workload: 4363 slots x 128 heads x 512 latent columns; sampled slots."""
    w = get_workload("dsv3")
    W = workloads.draw_kv_b_weight(w.heads, 512, seed=w.spec.seed)
    step = PrefillStep(w, "cuda", kv_b_weight=W)
    step.plan()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    step.kn_buf.fill_(float("nan"))
    step.v_buf.fill_(float("nan"))
    step.latent_up(0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(step.kn_buf.float()).all()) and bool(torch.isfinite(step.v_buf.float()).all())
    rng = np.random.default_rng(5)
    slots = sorted(set([0, 127, 128, w.total_ctx - 1] + rng.integers(0, w.total_ctx, size=60).tolist()))
    k_ref, v_ref = oracle.latent_up(w.cache, 0, w.page_table, w.spec.page_size, bro[0], co[0], 0, 512, W, w.heads,
                                    step.cap, slots=slots)
    idx = torch.tensor(slots, device="cuda")
    _check(step.kn_buf[idx], k_ref, "dsv3-latent-k")
    _check(step.v_buf[idx], v_ref, "dsv3-latent-v")


def test_full_size_latent_then_attention_sampled():
    w = get_workload("prefix")
    W = workloads.draw_kv_b_weight(w.heads, 512, seed=w.spec.seed)
    step = PrefillStep(w, "cuda", cap=16384, kv_b_weight=W)
    say(f"prefix with latent K/V in {step.rows} rows")
    step.out.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    check_plan(step, w)
    out = step.out.float()
    assert bool(torch.isfinite(out).all())
    rows = sample_rows(w, 60, seed=13)
    bro1, co1, _, _ = oracle.plan(w.input_row_offsets, w.cache_lengths, w.total_ctx, 1)
    # the oracle's K_nope / V of the sampled head for every slot of the token's sequence, then its attention row
    got, ref = [], []
    vl = w.input_row_offsets.astype(np.int64)
    for t, h in rows:
        b = int(np.searchsorted(vl, t, side="right") - 1)
        g0, g1 = int(bro1[0][b]), int(bro1[0][b + 1])
        k_b, v_b = oracle.latent_up(w.cache, 0, w.page_table, w.spec.page_size, bro1[0], co1[0], 0, 512,
                                    W[h * 256:(h + 1) * 256], 1, w.total_ctx, slots=list(range(g0, g1)))
        kn_full = np.zeros((w.total_ctx, 1, 128))
        v_full = np.zeros((w.total_ctx, 1, 128))
        kn_full[g0:g1] = torch.from_numpy(k_b).to(torch.bfloat16).double().numpy()    # the attention's input type
        v_full[g0:g1] = torch.from_numpy(v_b).to(torch.bfloat16).double().numpy()
        one = oracle.mla_prefill_rows([(t, 0)], w.q[:, h:h + 1], kn_full, v_full, w.cache, 0, w.page_table,
                                      w.spec.page_size, w.spec.rope_col, w.cache_lengths, w.input_row_offsets,
                                      bro1[0], co1[0], w.softmax_scale)
        ref.append(one[0])
        got.append(out[t, h].cpu().numpy())
    assert report(np.stack(got), np.stack(ref), 1e-2, "prefix-latent-attn") <= 1e-2
