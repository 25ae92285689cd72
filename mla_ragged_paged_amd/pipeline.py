"""One prefill step on the device: plan -> gather -> attention.

Holds a workload's tensors in device memory, allocates the plan, gather and
output buffers once, and calls the three C entry points on the current
stream.  No arithmetic of the method happens here.
"""
from __future__ import annotations

import torch

from . import _binding as B
from .workloads import Workload


def _u32(a, device):
    return torch.from_numpy(a.astype("int64")).to(torch.int32).to(device)


class PrefillStep:
    """Device-resident inputs and outputs of one ragged paged MLA prefill step.

    ``cap`` is the buffer-row capacity handed to the plan (default: the whole
    batch's context, one row).  ``gather_cols`` = (col_begin, col_count) of the
    cache rows the gather copies (default: the whole row).
    """

    def __init__(self, w: Workload, device="cuda", cap: int | None = None, gather_cols=None):
        self.w = w
        self.device = torch.device(device)
        dev = self.device
        self.fp8 = w.spec.dtype == "fp8"
        self.input_row_offsets = _u32(w.input_row_offsets, dev)
        self.cache_lengths = _u32(w.cache_lengths, dev)
        self.page_table = _u32(w.page_table, dev)
        self.cache_data = w.cache.to(dev)
        self.q = w.q.to(dev)
        self.k_nope = w.k_nope.to(dev)
        self.v = w.v.to(dev)
        if self.fp8:
            self.scales = {k: torch.tensor([v], dtype=torch.float32, device=dev) for k, v in w.scales.items()}
        else:
            self.scales = None
        self.kv = B.PagedCache(self.cache_data, self.page_table, self.cache_lengths, w.spec.rope_col,
                               scale=self.scales["k_rope"] if self.fp8 else None)
        Bsz = w.batch
        C = w.total_ctx
        self.cap = max(1, C if cap is None else int(cap))
        self.rows = max(1, -(-C // self.cap))
        self.buffer_row_offsets = torch.zeros((self.rows, Bsz + 1), dtype=torch.int32, device=dev)
        self.cache_offsets = torch.zeros((self.rows, Bsz), dtype=torch.int32, device=dev)
        self.buffer_lengths = torch.zeros((self.rows,), dtype=torch.int32, device=dev)
        self.status = torch.zeros((1,), dtype=torch.int32, device=dev)
        width = w.cache.shape[4]
        self.gather_cols = (0, width) if gather_cols is None else tuple(gather_cols)
        self.gathered = torch.zeros((self.cap, self.gather_cols[1]), dtype=w.cache.dtype, device=dev)
        self.out = torch.zeros((w.total_q, w.heads, 128), dtype=torch.bfloat16, device=dev)

    def plan(self, stream=None):
        B.mla_prefill_plan(self.input_row_offsets, self.kv, self.w.spec.layer_idx, self.cap,
                           self.buffer_row_offsets, self.cache_offsets, self.buffer_lengths, self.status, stream)

    def gather(self, row: int = 0, stream=None):
        B.mla_prefill_gather(self.kv, self.w.spec.layer_idx, self.buffer_row_offsets[row], self.cache_offsets[row],
                             self.gather_cols[0], self.gather_cols[1], self.gathered, stream)

    def attention(self, row: int = 0, k_nope=None, v=None, out=None, cache_offsets="plan", stream=None):
        """Attention over plan row ``row``; k_nope / v default to the workload's buffer (one-row layout)."""
        co = self.cache_offsets[row] if isinstance(cache_offsets, str) else cache_offsets
        sc = self.scales or {}
        B.mla_prefill_ragged(self.out if out is None else out, self.q, self.k_nope if k_nope is None else k_nope,
                             self.v if v is None else v, self.kv, self.w.spec.layer_idx, self.input_row_offsets,
                             self.buffer_row_offsets[row], co, self.w.softmax_scale, sc.get("q"),
                             sc.get("k_nope"), sc.get("v"), self.w.max_q, stream)

    def run(self, stream=None):
        """The whole step: plan, gather of row 0, attention over row 0."""
        self.plan(stream)
        self.gather(0, stream)
        self.attention(0, stream=stream)
