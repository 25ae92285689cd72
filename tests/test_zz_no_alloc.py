"""mla_prefill_ragged_kvsplit_noalloc on the GPU: the key split with its partials
in the library's own device array, called through the C-ABI, against
mla_prefill_ragged_kvsplit with a caller workspace (the same kernels, so the
outputs and log-sum-exps must match bit for bit), on two calls in a row -- the
second with a smaller input, while the array still holds the first call's
partials -- and against the float64 oracle on the smaller one.
"""
import numpy as np
import pytest
import torch

import mla_ragged_paged_amd as m
from mla_ragged_paged_amd import workloads
from mla_ragged_paged_amd.pipeline import PrefillStep, balanced_split_keys
from tests.gpu_util import check_plan, oracle_full, report_keys, say, visible_keys

pytestmark = pytest.mark.gpu


def _both(step, split_keys, mask="causal"):
    """(outputs, lses) of the workspace call and of the no-allocation call."""
    w = step.w
    T, H = w.total_q, w.heads
    ws = torch.empty((m.mla_prefill_kvsplit_workspace_bytes(T, H) // 4 + 1,), dtype=torch.float32, device="cuda")
    res = []
    for noalloc in (False, True):
        out = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        args = (out, step.q, step.k_nope, step.v, step.kv, 0, step.input_row_offsets, step.buffer_row_offsets[0],
                step.cache_offsets[0], w.softmax_scale, split_keys)
        if noalloc:
            m.mla_prefill_ragged_kvsplit_noalloc(*args, lse=lse, q_max_seq_len=w.max_q, mask=mask)
        else:
            m.mla_prefill_ragged_kvsplit(*args, ws, lse=lse, q_max_seq_len=w.max_q, mask=mask)
        torch.cuda.synchronize()
        res.append((out, lse))
    return res


def test_noalloc_matches_workspace_call_twice():
    # first call: a DeepSeek-V3-shaped batch at 8 heads (one GPU's share under
    # 16-way head parallelism), with the split the host heuristic picks
    big = workloads.build(workloads.Spec("na_big", 4, (512, 2048), (0, 0), 8, 128, True, "bf16", seed=2))
    sk = balanced_split_keys(big.n, big.p, big.heads)
    assert sk > 0
    say(f"no-alloc call 1: B={big.batch} T={big.total_q} H={big.heads} split_keys={sk}")
    step = PrefillStep(big, "cuda")
    step.plan()
    torch.cuda.synchronize()
    (o_ws, l_ws), (o_na, l_na) = _both(step, sk)
    assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na)
    assert bool(torch.isfinite(o_na.float()).all())
    # second call, smaller: the array still holds the first call's partials
    small = workloads.build(workloads.Spec("na_small", 2, (0, 0), (0, 0), 4, 16, True, "bf16", seed=33),
                            n=[300, 90], p=[200, 0])
    say(f"no-alloc call 2: B={small.batch} T={small.total_q} H={small.heads} split_keys=128")
    st2 = PrefillStep(small, "cuda")
    st2.plan()
    torch.cuda.synchronize()
    bro, co, _ = check_plan(st2, small)
    (o_ws, l_ws), (o_na, l_na) = _both(st2, 128)
    assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na)
    ref = oracle_full(small, bro[0], co[0])
    report_keys(o_na.float().cpu().numpy(), ref, visible_keys(small, bro[0], co[0]), 1e-2, "no-alloc small")


def test_noalloc_null_mask_and_no_split():
    w = workloads.build(workloads.Spec("na_null", 3, (0, 0), (0, 0), 8, 32, True, "bf16", seed=34),
                        n=[400, 17, 260], p=[0, 50, 300])
    step = PrefillStep(w, "cuda", mask="null")
    step.plan()
    torch.cuda.synchronize()
    for sk in (256, 0):                  # 0: nothing split, the plain kernels
        (o_ws, l_ws), (o_na, l_na) = _both(step, sk, mask="null")
        assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na)


def test_noalloc_rejects_partials_beyond_the_array():
    """A split call whose partials exceed MLA_NOALLOC_SCRATCH_BYTES is rejected before
    anything runs (65,028 token-heads is one past the limit)."""
    H, T = 4, 16257                       # 65,028 token-heads
    assert m.mla_prefill_kvsplit_workspace_bytes(T, H) > m._binding.MLA_NOALLOC_SCRATCH_BYTES
    assert m.mla_prefill_kvsplit_workspace_bytes(T - 1, H) <= m._binding.MLA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((T, H, 192), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((8, H, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((T, H, 128), dtype=torch.bfloat16, device="cuda")
    kv = m.PagedCache(torch.zeros((1, 1, 16, 1, 64), dtype=torch.bfloat16, device="cuda"),
                      torch.zeros((1, 1), dtype=torch.int32, device="cuda"),
                      torch.zeros((1,), dtype=torch.int32, device="cuda"), 0)
    vl = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    cro = torch.tensor([0, 8], dtype=torch.int32, device="cuda")
    with pytest.raises(m.MlaError) as e:
        m.mla_prefill_ragged_kvsplit_noalloc(out, q, kn, kn, kv, 0, vl, cro, None, 0.1, 256, q_max_seq_len=T)
    assert e.value.status == 2
