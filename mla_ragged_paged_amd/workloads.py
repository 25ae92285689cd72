"""Seeded synthetic inputs for ragged paged MLA prefill.

This module only draws and lays out inputs: sequence lengths, cached-prefix
lengths, page tables, the paged cache, Q, K_nope and V.  It contains none of
the prefill arithmetic (no plan, no gather, no attention), so both the HIP
path and the test oracle can consume what it produces.

Recipe (same for every workload):

* integer lengths "uniform in [a, b]" are drawn inclusive with
  ``numpy.random.default_rng(seed).integers(a, b + 1)``: first the new-token
  counts n_b, then the cached-prefix lengths p_b, then the page permutation;
* tensors are drawn on the CPU from ``torch.Generator().manual_seed(1000 + seed)``
  as float32 N(0, 1) in the fixed order Q, K_nope, V, cache, then rounded to
  bfloat16, or quantised to float8_e4m3fn with one fp32 scale per tensor
  (scale = amax / 448, codes = round-to-nearest-even of x / scale);
* the paged cache is [layers][pages][page_size][1][row_width]; sequence b's
  positions 0 .. p_b + n_b - 1 occupy ceil((p_b + n_b) / page_size) pages
  whose physical ids are a seeded permutation (or the identity);
* K_nope and V are the ragged K/V buffer [rows, H, 128]: sequence b's keys
  for cache positions 0 .. p_b + n_b - 1 in batch order (the layout one
  buffer row of capacity >= sum(p_b + n_b) holds).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

NOPE_DEPTH = 128
ROPE_DEPTH = 64
Q_DEPTH = NOPE_DEPTH + ROPE_DEPTH
E4M3_MAX = 448.0


@dataclass
class Spec:
    """Shape recipe of one workload."""
    name: str
    batch: int
    n_range: tuple          # inclusive range of new tokens per sequence
    p_range: tuple          # inclusive range of cached-prefix tokens per sequence
    heads: int
    page_size: int
    permute_pages: bool
    dtype: str              # "bf16" or "fp8"
    row_width: int = ROPE_DEPTH + 512   # DeepSeek-V3 latent cache row: 512 latent + 64 rope
    rope_col: int = 512
    num_layers: int = 1
    layer_idx: int = 0
    seed: int = 0
    description: str = ""


# The five workloads the measurements and parity tests use (shapes of a
# DeepSeek-V3 MLA layer: 128 heads, q_depth 192 = 128 nope + 64 rope).
SPECS = {
    "tiny": Spec("tiny", 1, (64, 64), (0, 0), 2, 16, False, "bf16", row_width=64, rope_col=0, seed=1,
                 description="1 sequence of 64 new tokens, no prefix, H=2, page 16, identity page table, "
                             "rope-only cache rows"),
    "dsv3": Spec("dsv3", 4, (512, 2048), (0, 0), 128, 128, True, "bf16", seed=2,
                 description="DeepSeek-V3-shaped prefill: 4 sequences, new tokens U[512,2048], no prefix, "
                             "H=128, page 128, permuted page table"),
    "prefix": Spec("prefix", 16, (256, 1024), (0, 4096), 128, 128, True, "bf16", seed=3,
                   description="16 sequences, new tokens U[256,1024], cached prefix U[0,4096], H=128, "
                               "page 128, shuffled pages"),
    "long": Spec("long", 1, (16384, 16384), (0, 0), 128, 128, True, "bf16", seed=4,
                 description="1 sequence of 16384 new tokens, no prefix, H=128, page 128"),
    "fp8": Spec("fp8", 8, (1024, 4096), (0, 2048), 128, 128, True, "fp8", seed=5,
                description="8 sequences, new tokens U[1024,4096], cached prefix U[0,2048], H=128, "
                            "float8_e4m3fn Q/K_nope/V/cache with per-tensor fp32 scales, bf16 output"),
}


@dataclass
class Workload:
    spec: Spec
    n: np.ndarray                  # int64 [B] new tokens
    p: np.ndarray                  # int64 [B] cached prefix
    input_row_offsets: np.ndarray  # uint32 [B+1]
    cache_lengths: np.ndarray      # uint32 [B]
    page_table: np.ndarray         # uint32 [B][max_pages_per_seq]
    num_pages: int
    cache: torch.Tensor            # [layers, pages, page_size, 1, row_width] bf16 / float8_e4m3fn
    q: torch.Tensor                # [T, H, 192]
    k_nope: torch.Tensor           # [C, H, 128]
    v: torch.Tensor                # [C, H, 128]
    scales: dict | None = None     # fp8: {"q","k_nope","v","k_rope"} -> python float (fp32 value)
    softmax_scale: float = 1.0 / math.sqrt(Q_DEPTH)
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.n.shape[0])

    @property
    def heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def total_q(self) -> int:
        return int(self.n.sum())

    @property
    def total_ctx(self) -> int:
        return int((self.n + self.p).sum())

    @property
    def max_q(self) -> int:
        return int(self.n.max()) if self.n.size else 0

    def kv_row_offsets(self) -> np.ndarray:
        """Where each sequence's keys start in k_nope / v (uint32 [B+1])."""
        out = np.zeros(self.batch + 1, dtype=np.int64)
        out[1:] = np.cumsum(self.n + self.p)
        return out.astype(np.uint32)


def _quantize_e4m3(x: torch.Tensor):
    amax = float(x.abs().max()) if x.numel() else 1.0
    scale = np.float32(amax / E4M3_MAX if amax > 0 else 1.0)
    codes = (x / float(scale)).to(torch.float8_e4m3fn)
    return codes, float(scale)


def _draw(gen: torch.Generator, shape, dtype: str):
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if dtype == "bf16":
        return x.to(torch.bfloat16), None
    return _quantize_e4m3(x)


def build(spec: Spec, n=None, p=None, page_permutation=None) -> Workload:
    """Draw one workload.  ``n``/``p`` override the drawn lengths (edge-case tests)."""
    rng = np.random.default_rng(spec.seed)
    B = spec.batch
    n_draw = rng.integers(spec.n_range[0], spec.n_range[1] + 1, size=B)
    p_draw = rng.integers(spec.p_range[0], spec.p_range[1] + 1, size=B)
    n = np.asarray(n_draw if n is None else n, dtype=np.int64)
    p = np.asarray(p_draw if p is None else p, dtype=np.int64)
    B = int(n.shape[0])
    L = n + p
    ps = spec.page_size
    pages_per_seq = [(int(x) + ps - 1) // ps for x in L]
    num_pages = max(1, sum(pages_per_seq))
    if page_permutation is not None:
        perm = np.asarray(page_permutation, dtype=np.int64)
    elif spec.permute_pages:
        perm = rng.permutation(num_pages)
    else:
        perm = np.arange(num_pages)
    max_pages = max([1] + pages_per_seq)
    page_table = np.zeros((B, max_pages), dtype=np.uint32)  # unused entries point at page 0
    k = 0
    for b in range(B):
        for j in range(pages_per_seq[b]):
            page_table[b, j] = perm[k]
            k += 1
    iro = np.zeros(B + 1, dtype=np.int64)
    iro[1:] = np.cumsum(n)

    gen = torch.Generator().manual_seed(1000 + spec.seed)
    T, C, H = int(n.sum()), int(L.sum()), spec.heads
    q, sq = _draw(gen, (T, H, Q_DEPTH), spec.dtype)
    kn, skn = _draw(gen, (C, H, NOPE_DEPTH), spec.dtype)
    v, sv = _draw(gen, (C, H, NOPE_DEPTH), spec.dtype)
    cache, skr = _draw(gen, (spec.num_layers, num_pages, ps, 1, spec.row_width), spec.dtype)
    scales = None if spec.dtype == "bf16" else {"q": sq, "k_nope": skn, "v": sv, "k_rope": skr}
    return Workload(spec=spec, n=n, p=p, input_row_offsets=iro.astype(np.uint32),
                    cache_lengths=p.astype(np.uint32), page_table=page_table, num_pages=num_pages,
                    cache=cache, q=q, k_nope=kn, v=v, scales=scales)


def split_query(w: Workload):
    """The query as the two tensors of the split-Q calls: q_nope = columns 0..127
    of w.q (bf16, or e4m3 codes that keep w.scales["q"]), q_rope [T, H, 64] bf16 =
    columns 128..191 of w.q for a bf16 workload and, for an fp8 workload, a fresh
    N(0, 1) draw rounded to bf16 (``torch.Generator().manual_seed(1000 + seed + 7919)``)."""
    q_nope = w.q[..., :NOPE_DEPTH].contiguous()
    if w.spec.dtype == "bf16":
        return q_nope, w.q[..., NOPE_DEPTH:].contiguous()
    gen = torch.Generator().manual_seed(1000 + w.spec.seed + 7919)
    q_rope = torch.randn((w.total_q, w.heads, ROPE_DEPTH), generator=gen, dtype=torch.float32)
    return q_nope, q_rope.to(torch.bfloat16)


def draw_rope_rows(rows: int, seed: int) -> torch.Tensor:
    """Contiguous K_rope rows [rows, 1, 64], N(0, 1) rounded to bf16
    (``torch.Generator().manual_seed(1000 + seed + 104729)``)."""
    gen = torch.Generator().manual_seed(1000 + seed + 104729)
    return torch.randn((rows, 1, ROPE_DEPTH), generator=gen, dtype=torch.float32).to(torch.bfloat16)


def draw_kv_b_weight(heads: int, latent_dim: int, seed: int) -> torch.Tensor:
    """Synthetic up-projection weight [heads * 256, latent_dim] bf16 (per head 128
    key rows then 128 value rows), N(0, 1 / latent_dim) so that K_nope and V of an
    N(0, 1) latent are about N(0, 1)
    (``torch.Generator().manual_seed(1000 + seed + 15485863)``)."""
    gen = torch.Generator().manual_seed(1000 + seed + 15485863)
    w = torch.randn((heads * 256, latent_dim), generator=gen, dtype=torch.float32) / math.sqrt(latent_dim)
    return w.to(torch.bfloat16)


def causal_pairs(n, p) -> int:
    """Visible (query, key) pairs: every new token sees its prefix and itself."""
    n = np.asarray(n, dtype=np.int64)
    p = np.asarray(p, dtype=np.int64)
    return int(np.sum(n * p + n * (n + 1) // 2))


def causal_flops(n, p, heads: int) -> float:
    """Algorithmic FLOPs: 2 * H * (192 + 128) per visible pair (QK^T over 192, PV over 128)."""
    return 2.0 * heads * (Q_DEPTH + NOPE_DEPTH) * causal_pairs(n, p)


def null_mask_pairs(n, p) -> int:
    """(query, key) pairs under the null mask: every new token sees all of its sequence's keys."""
    n = np.asarray(n, dtype=np.int64)
    p = np.asarray(p, dtype=np.int64)
    return int(np.sum(n * (n + p)))


def null_mask_flops(n, p, heads: int) -> float:
    """Algorithmic FLOPs under the null mask (same per-pair count as causal_flops)."""
    return 2.0 * heads * (Q_DEPTH + NOPE_DEPTH) * null_mask_pairs(n, p)


def algorithmic_bytes(w: Workload) -> float:
    """Bytes a prefill call must move at least once: Q, K_nope, V, K_rope in; O out (bf16)."""
    el = 1 if w.spec.dtype == "fp8" else 2
    T, C, H = w.total_q, w.total_ctx, w.heads
    return float(T * H * Q_DEPTH * el + 2 * C * H * NOPE_DEPTH * el + C * ROPE_DEPTH * el + T * H * NOPE_DEPTH * 2)
