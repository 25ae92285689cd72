"""Key split (mla_prefill_ragged_kvsplit) on the GPU, against the float64 oracle
and against the plain attention.

Bars (the accuracy bars of the output, written here): max |gpu - oracle|
<= 1e-2 with bf16 inputs and <= 6e-2 with float8_e4m3fn inputs; log-sum-exp
bars 1e-2 and 6.5e-2 (derived in the module docstring of the lse tests: the
row sum is taken over weights rounded to bf16, relative error <= 2^-9, or over
e4m3 weights, <= 2^-4).

The call's documented rule -- a 128-query tile whose visible keys number more
than split_keys is computed as two halves and merged, every other tile whole --
is restated on the host here.  Rows of tiles it does not split are computed by
the plain kernel's arithmetic in the same order and must equal
mla_prefill_ragged's bit for bit; rows of split tiles must meet the bar against
the oracle.  The workspace and the output are filled with NaN before each call:
nothing read may be left over from an earlier call.
"""
import dataclasses
import functools

import numpy as np
import pytest
import torch

import mla_ragged_paged_amd as m
from mla_ragged_paged_amd import workloads
from mla_ragged_paged_amd.pipeline import PrefillStep, balanced_split_keys
from tests.gpu_util import check_plan, get_workload, oracle_full, oracle_rows, report, report_lse, sample_rows, say

pytestmark = pytest.mark.gpu

BAR = {"bf16": 1e-2, "fp8": 6e-2}
LSE_BAR = {"bf16": 1e-2, "fp8": 6.5e-2}

CASES = [
    dict(n=[700, 130, 1, 0], p=[0, 500, 2000, 40], heads=2, ps=16),
    dict(n=[1000], p=[0], heads=1, ps=128),                       # a head count that is not a multiple of 8
    dict(n=[300, 513], p=[900, 0], heads=8, ps=128),
    dict(n=[0, 257, 64, 400], p=[3000, 10, 0, 333], heads=16, ps=64),
    dict(n=[150, 70], p=[33, 0], heads=3, ps=48),                 # page size not a power of two
]
SPLITS = [128, 333, 100000]


def _workload(case, dtype, seed_base):
    kw = CASES[case]
    spec = workloads.Spec("kvs", len(kw["n"]), (0, 0), (0, 0), kw["heads"], kw["ps"], True, dtype,
                          row_width=576, rope_col=512, seed=seed_base + case)
    return workloads.build(spec, n=kw["n"], p=kw["p"])


@functools.lru_cache(maxsize=None)
def _case_reference(case, dtype, mask):
    """The workload and its oracle output (one buffer row), shared by the split_keys values."""
    w = _workload(case, dtype, 700)
    bro = np.zeros(w.batch + 1, dtype=np.uint32)
    bro[1:] = np.cumsum(w.n + w.p)
    return w, oracle_full(w, bro, np.zeros(w.batch, dtype=np.uint32), mask=mask)


def split_token_mask(w, split_keys, mask):
    """Tokens whose 128-query tile the call splits: visible keys of the tile (one
    buffer row holding every context: key positions 0 .. p + n - 1) > split_keys."""
    split = np.zeros(w.total_q, dtype=bool)
    vl = w.input_row_offsets.astype(np.int64)
    for b in range(w.batch):
        n, p = int(w.n[b]), int(w.p[b])
        for i0 in range(0, n, 128):
            i_last = min(n, i0 + 128) - 1
            keys = min(p + i_last + 1, p + n) if mask == "causal" else p + n
            if split_keys and keys > split_keys:
                split[vl[b] + i0:vl[b] + i_last + 1] = True
    return split


def _kvsplit(step, split_keys, out=None, lse=None, workspace=None):
    w = step.w
    sc = step.scales or {}
    out = step.out if out is None else out
    if workspace is None:
        nbytes = m.mla_prefill_kvsplit_workspace_bytes(w.total_q, w.heads)
        workspace = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    m.mla_prefill_ragged_kvsplit(out, step.q, step.k_nope, step.v, step.kv, 0, step.input_row_offsets,
                                 step.buffer_row_offsets[0], step.cache_offsets[0], w.softmax_scale, split_keys,
                                 workspace, lse=lse, q_scale=sc.get("q"), k_nope_scale=sc.get("k_nope"),
                                 v_scale=sc.get("v"), q_max_seq_len=w.max_q, mask=step.mask)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("split", SPLITS)
@pytest.mark.parametrize("mask", ["causal", "null"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_kvsplit_every_output(case, dtype, mask, split):
    say(f"kv split {dtype} {mask} split_keys {split} case {CASES[case]}")
    w, ref = _case_reference(case, dtype, mask)
    plain = PrefillStep(w, "cuda", mask=mask)
    plain.run()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(plain, w)
    assert np.array_equal(bro[0][1:], np.cumsum(w.n + w.p)) and not co[0].any()
    got = torch.full_like(plain.out, float("nan"))
    _kvsplit(plain, split, out=got)
    assert report(got.float().cpu().numpy(), ref, BAR[dtype], f"kvsplit-{dtype}-{mask}-{split}-{case}") <= BAR[dtype]
    sp = torch.from_numpy(split_token_mask(w, split, mask)).cuda()
    say(f"  split tokens {int(sp.sum())} of {w.total_q}")
    assert torch.equal(got[~sp], plain.out[~sp])
    if split == 128 and max(w.n) > 128:
        assert bool(sp.any())


@pytest.mark.parametrize("mask", ["causal", "null"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("case", [0, 3])
def test_kvsplit_lse_and_fp32_output(case, dtype, mask):
    w = _workload(case, dtype, 720)
    say(f"kv split lse {dtype} {mask} case {CASES[case]}")
    step = PrefillStep(w, "cuda", mask=mask)
    step.plan()
    bro, co, _ = check_plan(step, w)
    out32 = torch.full((w.total_q, w.heads, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((w.total_q, w.heads), float("nan"), dtype=torch.float32, device="cuda")
    _kvsplit(step, 128, out=out32, lse=lse)
    ref, ref_lse = oracle_full(w, bro[0], co[0], mask=mask, return_lse=True)
    assert report(out32.cpu().numpy(), ref, BAR[dtype], f"kvsplit32-{dtype}-{mask}{case}") <= BAR[dtype]
    assert report_lse(lse.cpu().numpy(), ref_lse, LSE_BAR[dtype], f"kvsplit-lse-{dtype}-{mask}{case}") <= LSE_BAR[dtype]
    # the bf16 output is the fp32 one rounded once
    out16 = _kvsplit(step, 128, out=torch.full_like(step.out, float("nan")))
    assert torch.equal(out32.to(torch.bfloat16), out16)


def test_kvsplit_zero_is_the_plain_call_and_reruns_are_identical():
    w = _workload(0, "bf16", 740)
    step = PrefillStep(w, "cuda")
    step.run()
    torch.cuda.synchronize()
    a = _kvsplit(step, 0, out=torch.full_like(step.out, float("nan")), workspace=None)
    assert torch.equal(a, step.out)
    ws = torch.full((m.mla_prefill_kvsplit_workspace_bytes(w.total_q, w.heads) // 4,), float("nan"),
                    dtype=torch.float32, device="cuda")
    b1 = _kvsplit(step, 128, out=torch.full_like(step.out, float("nan")), workspace=ws)
    # a second call on the workspace the first left behind, then one with another threshold
    b2 = _kvsplit(step, 128, out=torch.full_like(step.out, float("nan")), workspace=ws)
    assert torch.equal(b1, b2)
    c = _kvsplit(step, 333, out=torch.full_like(step.out, float("nan")), workspace=ws)
    fresh = _kvsplit(step, 333, out=torch.full_like(step.out, float("nan")))
    assert torch.equal(c, fresh)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_one_gpu_share_of_the_heads_sampled(dtype):
    """A DeepSeek-V3-shaped batch at 16 heads (one GPU's share under 8-way head
    parallelism), split as balanced_split_keys chooses: sampled rows against
    the oracle, every row of an unsplit tile equal to the plain call's."""
    base = get_workload("dsv3" if dtype == "bf16" else "fp8")
    w = workloads.build(dataclasses.replace(base.spec, name=base.spec.name + "_h16", heads=16))
    sk = balanced_split_keys(w.n, w.p, w.heads)
    say(f"{w.spec.name}: B={w.batch} T={w.total_q} H={w.heads} split_keys={sk}")
    step = PrefillStep(w, "cuda", split_keys=sk if sk else 256)
    plain = PrefillStep(w, "cuda")
    plain.run()
    step.plan()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(step, w)
    step.out.fill_(float("nan"))
    step.workspace.fill_(float("nan"))
    step.attention(0)
    torch.cuda.synchronize()
    out = step.out.float()
    assert bool(torch.isfinite(out).all())
    sp = torch.from_numpy(split_token_mask(w, step.split_keys, "causal")).cuda()
    say(f"  split tokens {int(sp.sum())} of {w.total_q}")
    assert bool(sp.any())
    assert torch.equal(step.out[~sp], plain.out[~sp])
    rows = sample_rows(w, 120, seed=11)
    # half the samples from split tiles
    toks = np.nonzero(sp.cpu().numpy())[0]
    rng = np.random.default_rng(12)
    rows += [(int(t), int(rng.integers(0, w.heads))) for t in rng.choice(toks, 60)]
    ref = oracle_rows(w, rows, bro[0], co[0])
    got = np.stack([out[t, h].cpu().numpy() for t, h in rows])
    assert report(got, ref, BAR[dtype], f"{w.spec.name}-kvsplit") <= BAR[dtype]


@pytest.mark.parametrize("mask", ["causal", "null"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_kvsplit_per_buffer_row_then_merged(dtype, mask):
    """A plan of four buffer rows, so rows start in the middle of sequences
    (cache_offsets > 0) and some sequences have no key in a row: each row's
    attention through the key split (split_keys 128) with its lse, the rows
    combined with mla_prefill_merge, equals the attention over every key."""
    w, ref = _case_reference(0, dtype, mask)
    say(f"kv split per buffer row {dtype} {mask}: C={w.total_ctx}")
    step = PrefillStep(w, "cuda", cap=1100, mask=mask)
    step.plan()
    check_plan(step, w)
    assert step.rows == 4
    sc = step.scales or {}
    T, H = w.total_q, w.heads
    ws = torch.full((m.mla_prefill_kvsplit_workspace_bytes(T, H) // 4,), float("nan"), dtype=torch.float32,
                    device="cuda")
    acc = acc_lse = None
    for r in range(step.rows):
        kn, v = step.row_buffers(r)
        o = torch.full((T, H, 128), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        m.mla_prefill_ragged_kvsplit(o, step.q, kn, v, step.kv, 0, step.input_row_offsets,
                                     step.buffer_row_offsets[r], step.cache_offsets[r], w.softmax_scale, 128, ws,
                                     lse=lse, q_scale=sc.get("q"), k_nope_scale=sc.get("k_nope"),
                                     v_scale=sc.get("v"), q_max_seq_len=w.max_q, mask=mask)
        if acc is None:
            acc, acc_lse = o, lse
        else:
            merged = torch.empty_like(o)
            merged_lse = torch.empty_like(lse)
            m.mla_prefill_merge(merged, merged_lse, acc, acc_lse, o, lse)
            acc, acc_lse = merged, merged_lse
    torch.cuda.synchronize()
    assert report(acc.cpu().numpy(), ref, BAR[dtype], f"kvsplit-rows-{dtype}-{mask}") <= BAR[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_kvsplit_large_scale_with_rows_that_see_no_key_of_a_half(dtype):
    """One 200-token sequence, split at 128 keys: its only tile is cut into keys 0..127
    and 128..199, and queries 0..127 see none of the second half, which must hand the
    merge an empty partial.  At a softmax scale of 1e4 (the top of the range the
    header states) every softmax is one-hot: every output equals the oracle's, the
    V row of the top key."""
    spec = workloads.Spec("kvs-large", 1, (0, 0), (0, 0), 2, 16, True, dtype, row_width=576, rope_col=512, seed=733)
    w = workloads.build(spec, n=[200], p=[0])
    w.softmax_scale = 1e4
    step = PrefillStep(w, "cuda")
    step.run()
    torch.cuda.synchronize()
    bro = np.array([0, 200], dtype=np.uint32)
    ref = oracle_full(w, bro, np.zeros(1, dtype=np.uint32))
    got = torch.full_like(step.out, float("nan"))
    _kvsplit(step, 128, out=got)
    g = got.float().cpu().numpy()
    assert not np.isnan(g).any()
    assert report(g, ref, BAR[dtype], f"kvsplit-large-{dtype}") <= BAR[dtype]
    assert report(step.out.float().cpu().numpy(), ref, BAR[dtype], f"plain-large-{dtype}") <= BAR[dtype]
