"""One prefill step on the device: plan -> gather -> attention (-> merge).

Holds a workload's tensors in device memory, allocates the plan, gather and
output buffers once, and calls the C entry points on the current stream.  No
arithmetic of the method happens here.

By default the gather copies each buffer row's K_rope column window of the
cache rows into contiguous rows laid out like K_nope / V, and the attention of a
one-row plan reads K_rope from those rows (mla_prefill_ragged_krope); other
attention calls read K_rope through the page table.

With a buffer-row capacity below the batch's context the plan makes several
rows; each row's attention is a partial softmax over the keys the row holds,
and the rows are combined through their log-sum-exps (the merge is fused into
the attention's epilogue: a sequence's first row writes an fp32 partial and its
lse, its middle rows merge into them in place, its last row merges and writes
the bf16 output).
"""
from __future__ import annotations

import torch

from . import _binding as B
from .workloads import Workload

# Workgroup slots of the attention grid: 256 CUs x 2 resident workgroups.
ATTENTION_SLOTS = 512
QUERY_TILE = 128


def _u32(a, device):
    return torch.from_numpy(a.astype("int64")).to(torch.int32).to(device)


def balanced_split_keys(new_lengths, cache_lengths, heads: int, causal: bool = True,
                        slots: int = ATTENTION_SLOTS) -> int:
    """split_keys for mla_prefill_ragged_kvsplit from the host-side lengths of a batch.

    The attention grid has one workgroup per (head, sequence, 128-query tile).
    When it holds fewer of them than the chip has workgroup slots, every tile
    runs at once and the launch lasts as long as its costliest tile: splitting
    the tiles that see more than half the most keys any tile sees halves that.
    With at least as many tiles as slots the kernel runs at full occupancy
    until its tail and the split only adds the merge pass (measured on
    DeepSeek-V3-shaped batches at 8, 16 and 32 heads): 0, no split.
    """
    tiles = 0
    most = 0
    for n, p in zip((int(x) for x in new_lengths), (int(x) for x in cache_lengths)):
        for i0 in range(0, n, QUERY_TILE):
            tiles += 1
            keys = p + min(n, i0 + QUERY_TILE) if causal else p + n
            most = max(most, keys)
    if heads * tiles >= slots:
        return 0
    threshold = max(128, -(-most // 2))
    return threshold if most > threshold else 0


class PrefillStep:
    """Device-resident inputs and outputs of one ragged paged MLA prefill step.

    ``cap`` is the buffer-row capacity handed to the plan (default: the whole
    batch's context, one row).  ``gather_cols`` = (col_begin, col_count) of the
    cache rows the gather copies (default: the 64-column K_rope window, which the
    attention of each buffer row then reads; any other window is gathered only).  With ``kv_b_weight``
    ([H*256, latent_dim] bf16) K_nope / V are not the workload's tensors but are
    decompressed per buffer row from the latent cache (columns
    ``latent_col`` .. +latent_dim); the gather then lays out only the K_rope
    window.
    ``split_keys`` > 0 (one buffer row only) runs the attention through
    mla_prefill_ragged_kvsplit with that threshold and a workspace allocated
    here; "auto" takes balanced_split_keys of the workload.
    """

    def __init__(self, w: Workload, device="cuda", cap: int | None = None, gather_cols=None, mask="causal",
                 kv_b_weight=None, latent_col=0, split_keys=0):
        self.w = w
        self.mask = mask
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
        self.rope_gather = gather_cols is None
        self.gather_cols = (w.spec.rope_col, 64) if gather_cols is None else tuple(gather_cols)
        self.gathered = torch.zeros((self.cap, self.gather_cols[1]), dtype=w.cache.dtype, device=dev)
        self.out = torch.zeros((w.total_q, w.heads, 128), dtype=torch.bfloat16, device=dev)
        self.kv_b_weight = None if kv_b_weight is None else kv_b_weight.to(dev).contiguous()
        self.latent_col = latent_col
        if self.kv_b_weight is not None:
            self.kn_buf = torch.zeros((self.cap, w.heads, 128), dtype=torch.bfloat16, device=dev)
            self.v_buf = torch.zeros((self.cap, w.heads, 128), dtype=torch.bfloat16, device=dev)
        # fp32 partial and log-sum-exp carried between buffer rows
        self.acc = None
        self.lse = None
        if self.rows > 1:
            self.acc = torch.zeros((w.total_q, w.heads, 128), dtype=torch.float32, device=dev)
            self.lse = torch.zeros((w.total_q, w.heads), dtype=torch.float32, device=dev)
        if split_keys == "auto":
            split_keys = balanced_split_keys(w.n, w.p, w.heads, causal=mask == "causal")
        self.split_keys = int(split_keys)
        self.workspace = None
        if self.split_keys:
            if self.rows > 1:
                raise ValueError("split_keys needs a single buffer row")
            nbytes = B.mla_prefill_kvsplit_workspace_bytes(w.total_q, w.heads)
            self.workspace = torch.empty((max(1, nbytes // 4),), dtype=torch.float32, device=dev)

    def row_buffers(self, row: int):
        """K_nope / V of plan row ``row``.  The workload's buffers hold every
        sequence's context end to end in batch order (the one-row layout), and
        row r covers positions [r * cap, r * cap + buffer_lengths[r]) of that
        stream, so a row's buffer is a view at offset r * cap."""
        if self.kv_b_weight is not None:
            return self.kn_buf, self.v_buf
        lo = row * self.cap
        return self.k_nope[lo:], self.v[lo:]

    def plan(self, stream=None):
        B.mla_prefill_plan(self.input_row_offsets, self.kv, self.w.spec.layer_idx, self.cap,
                           self.buffer_row_offsets, self.cache_offsets, self.buffer_lengths, self.status, stream)

    def gather(self, row: int = 0, stream=None):
        B.mla_prefill_gather(self.kv, self.w.spec.layer_idx, self.buffer_row_offsets[row], self.cache_offsets[row],
                             self.gather_cols[0], self.gather_cols[1], self.gathered, stream)

    def latent_up(self, row: int = 0, stream=None):
        """K_nope / V of plan row ``row`` from the latent cache into the row buffers."""
        B.mla_prefill_latent_up(self.kv, self.w.spec.layer_idx, self.buffer_row_offsets[row], self.cache_offsets[row],
                                self.kv_b_weight, self.kn_buf, self.v_buf, latent_col=self.latent_col,
                                latent_dim=self.kv_b_weight.shape[1], stream=stream)

    def attention(self, row: int = 0, k_nope=None, v=None, out=None, cache_offsets="plan", stream=None,
                  rope="gathered"):
        """Attention over plan row ``row``; k_nope / v default to the workload's buffer (one-row layout).
        K_rope comes from the gathered rows when the step gathers them and the plan has one
        row (``rope="gathered"``), else (or with ``rope="paged"``) through the page table."""
        co = self.cache_offsets[row] if isinstance(cache_offsets, str) else cache_offsets
        sc = self.scales or {}
        if rope == "gathered" and self.rope_gather and self.rows == 1 and not self.split_keys:
            B.mla_prefill_ragged_krope(self.out if out is None else out, self.q,
                                       self.k_nope if k_nope is None else k_nope, self.v if v is None else v,
                                       self.gathered.view(self.cap, 1, 64), self.cache_lengths,
                                       self.input_row_offsets, self.buffer_row_offsets[row], co, self.w.softmax_scale,
                                       k_rope_scale=sc.get("k_rope"), q_scale=sc.get("q"),
                                       k_nope_scale=sc.get("k_nope"), v_scale=sc.get("v"), q_max_seq_len=self.w.max_q,
                                       stream=stream, mask=self.mask)
            return
        if self.split_keys:
            B.mla_prefill_ragged_kvsplit(self.out if out is None else out, self.q,
                                         self.k_nope if k_nope is None else k_nope, self.v if v is None else v,
                                         self.kv, self.w.spec.layer_idx, self.input_row_offsets,
                                         self.buffer_row_offsets[row], co, self.w.softmax_scale, self.split_keys,
                                         self.workspace, q_scale=sc.get("q"), k_nope_scale=sc.get("k_nope"),
                                         v_scale=sc.get("v"), q_max_seq_len=self.w.max_q, stream=stream,
                                         mask=self.mask)
            return
        B.mla_prefill_ragged(self.out if out is None else out, self.q, self.k_nope if k_nope is None else k_nope,
                             self.v if v is None else v, self.kv, self.w.spec.layer_idx, self.input_row_offsets,
                             self.buffer_row_offsets[row], co, self.w.softmax_scale, sc.get("q"),
                             sc.get("k_nope"), sc.get("v"), self.w.max_q, stream, mask=self.mask)

    def attention_row_merged(self, row: int, stream=None, rope="gathered"):
        """Attention over plan row ``row`` of several (rows run in order): each
        token's partial is carried in the fp32 accumulator from its sequence's
        first row to the row holding its last visible key, which writes the bf16
        output.  K_rope comes from the row's gathered rows (the gather of this
        row must have run) when the step gathers them (``rope="gathered"``), else
        (or with ``rope="paged"``) through the page table."""
        kn, v = self.row_buffers(row)
        sc = self.scales or {}
        if rope == "gathered" and self.rope_gather:
            B.mla_prefill_ragged_row_krope(self.out, self.acc, self.lse, self.q, kn, v,
                                           self.gathered.view(self.cap, 1, 64), self.cache_lengths,
                                           self.input_row_offsets, self.buffer_row_offsets[row],
                                           self.cache_offsets[row], self.w.softmax_scale,
                                           k_rope_scale=sc.get("k_rope"), q_scale=sc.get("q"),
                                           k_nope_scale=sc.get("k_nope"), v_scale=sc.get("v"),
                                           q_max_seq_len=self.w.max_q, stream=stream, mask=self.mask)
            return
        B.mla_prefill_ragged_row(self.out, self.acc, self.lse, self.q, kn, v, self.kv, self.w.spec.layer_idx,
                                 self.input_row_offsets, self.buffer_row_offsets[row], self.cache_offsets[row],
                                 self.w.softmax_scale, q_scale=sc.get("q"), k_nope_scale=sc.get("k_nope"),
                                 v_scale=sc.get("v"), q_max_seq_len=self.w.max_q, stream=stream, mask=self.mask)

    def run(self, stream=None):
        """The whole step: plan, then per buffer row its gather (with a weight
        matrix, its latent decompression and the gather of the K_rope window) and
        its attention (merged across rows when there are several)."""
        self.plan(stream)
        latent = self.kv_b_weight is not None
        for r in range(self.rows):
            if latent:
                self.latent_up(r, stream)
            if not latent or self.rope_gather:
                self.gather(r, stream)
            if self.rows == 1:
                kn, v = self.row_buffers(0)
                self.attention(0, k_nope=kn, v=v, stream=stream)
            else:
                self.attention_row_merged(r, stream)


class CapturedStep:
    """One ``PrefillStep.run()`` captured as a HIP graph and replayed.

    The step's kernels are recorded once on a side stream (torch's graph
    capture, which drives hipStreamBeginCapture / hipGraphInstantiate); a replay
    launches the whole step -- plan, then per buffer row its gather or latent
    decompression and its attention -- with one graph launch and no per-kernel
    host work.  The step's device buffers are the graph's: inputs are changed
    by writing into ``step``'s tensors in place.  None of the captured kernels
    issues a memset.
    """

    def __init__(self, step: PrefillStep, warmup: int = 2):
        self.step = step
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                step.run()
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            step.run()

    def replay(self):
        self.graph.replay()
