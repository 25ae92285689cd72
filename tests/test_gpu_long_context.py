"""One sequence whose keys in a single call span more than 4 GiB of K_nope and
of V: 131,172 keys x 128 heads x 256 bytes (bf16) and 262,244 keys x 128 heads
x 128 bytes (fp8).  The attention kernels address a work unit's K_nope / V rows
through per-tile buffer descriptors whose byte counts are 64-bit quantities,
capped at 4 GiB - 1 while more remain; this checks sampled outputs of such a
call against the oracle.  Inputs are drawn on the device (seeded) to keep the
host side small; the oracle gets the sampled heads only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mla_ragged_paged_amd import _binding as B
from tests.gpu_util import report, say

pytestmark = pytest.mark.gpu

H, N_NEW, PS = 128, 64, 128
HEADS_CHECKED = (0, 77, 127)
BAR = {"bf16": 1e-2, "fp8": 6e-2}


def _case(dtype):
    dev = torch.device("cuda:0")
    el = 2 if dtype == "bf16" else 1
    # keys past 4 GiB of K_nope at 128 heads
    prefix = (1 << 32) // (H * 128 * el) + 100 - N_NEW
    L = prefix + N_NEW
    assert (L - 1) * H * 128 * el > (1 << 32)
    g = torch.Generator(device=dev).manual_seed(4242 if dtype == "bf16" else 4343)
    q = torch.randn(N_NEW, H, 192, generator=g, device=dev, dtype=torch.bfloat16)
    kn = torch.randn(L, H, 128, generator=g, device=dev, dtype=torch.bfloat16)
    v = torch.randn(L, H, 128, generator=g, device=dev, dtype=torch.bfloat16)
    pages = math.ceil(L / PS)
    rope = torch.randn(1, pages, PS, 1, 64, generator=g, device=dev, dtype=torch.bfloat16)
    scales = None
    if dtype == "fp8":
        def quant(x):
            s = float(x.abs().max()) / 448.0
            return (x.float() / s).to(torch.float8_e4m3fn), s
        q, sq = quant(q)
        kn, skn = quant(kn)
        v, sv = quant(v)
        rope, skr = quant(rope)
        scales = {"q": sq, "k_nope": skn, "v": sv, "k_rope": skr}
    perm = torch.randperm(pages, generator=torch.Generator().manual_seed(7)).to(torch.int32)
    page_table = perm.view(1, pages).to(dev)
    cache_lengths = torch.tensor([prefix], dtype=torch.int32, device=dev)
    valid_length = torch.tensor([0, N_NEW], dtype=torch.int32, device=dev)
    row_offsets = torch.tensor([0, L], dtype=torch.int32, device=dev)
    return dict(q=q, kn=kn, v=v, rope=rope, page_table=page_table, cache_lengths=cache_lengths,
                valid_length=valid_length, row_offsets=row_offsets, prefix=prefix, L=L, scales=scales)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_keys_past_4gib_sampled(dtype):
    c = _case(dtype)
    say(f"{dtype}: one sequence, {c['L']} keys x {H} heads (K_nope {c['kn'].numel() * c['kn'].element_size() / 2**30:.2f} GiB)")
    scale = 1.0 / math.sqrt(192.0)
    sc = c["scales"]
    dev_scale = (lambda k: None) if sc is None else \
        (lambda k: torch.tensor([sc[k]], dtype=torch.float32, device="cuda:0"))
    kv = B.PagedCache(data=c["rope"], page_table=c["page_table"], cache_lengths=c["cache_lengths"], rope_col=0,
                      scale=dev_scale("k_rope"))
    out = torch.full((N_NEW, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    B.mla_prefill_ragged(out, c["q"], c["kn"], c["v"], kv, 0, c["valid_length"], c["row_offsets"], None, scale,
                         q_scale=dev_scale("q"), k_nope_scale=dev_scale("k_nope"), v_scale=dev_scale("v"),
                         q_max_seq_len=N_NEW)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    # the oracle, one checked head at a time (it copies that head's rows to the host)
    got, ref = [], []
    for h in HEADS_CHECKED:
        qh, knh, vh = (x[:, h:h + 1].contiguous() for x in (c["q"], c["kn"], c["v"]))
        r = oracle.mla_prefill_ragged(qh, knh, vh, c["rope"], 0, c["page_table"].cpu().numpy(), PS, 0,
                                      c["cache_lengths"].cpu().numpy(), c["valid_length"].cpu().numpy(),
                                      c["row_offsets"].cpu().numpy(), None, scale, scales=sc)
        ref.append(r[:, 0])
        got.append(out[:, h].float().cpu().numpy())
    assert report(np.stack(got), np.stack(ref), BAR[dtype], f"long context {dtype}") <= BAR[dtype]
