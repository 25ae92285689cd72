"""Float64 numpy oracle for ragged paged MLA prefill.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP path never
imports this module and this module imports nothing from the HIP path.

Sources, all Modular MAX API documentation pages:

* "generic_flare_mla_prefill_ragged_paged_plan" -- description paragraph and
  Args section (meaning of input_row_offsets, buffer_token_size,
  buffer_row_offsets, cache_offsets, buffer_lengths).
* "flare_mla_prefill" -- description paragraph (tensor shapes, the 64 rope
  columns of K taken from the cache and shared by every head, the reduced
  output depth, ragged valid lengths) and Args section (valid_length,
  cache_row_offsets, cache_offsets, scale, output dtype).
* "mla_prefill_v2_ragged" -- Args section (the mask predicate -- causal,
  null and others -- the softmax scale, start position taken from the cache
  length).
* "generic_flare_mla_prefill_ragged_paged_plan" again for several buffer
  rows: each row holds part of the keys, so a row's attention is a partial
  softmax; its log-sum-exp and the combine of partials (``merge_partials``)
  make the rows add up to the attention over every key.

Where the pages leave a step open the plain reading is taken; each such
reading is named in the docstring of the function that relies on it
(reading ids R-a ... R-r, listed together in the design notes).

Precision: every floating-point step is float64.  The pages fix no
precision for the attention arithmetic; float64 makes the oracle's own
rounding negligible next to the bf16/fp8 tolerances it is compared with.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "E4M3FN_MAX",
    "decode_e4m3fn",
    "dequantize_e4m3fn",
    "plan",
    "gather",
    "rope_rows",
    "MASKS",
    "mla_prefill_ragged",
    "mla_prefill_rows",
    "mla_prefill_ragged_split",
    "mla_prefill_rows_split",
    "latent_up",
    "merge_partials",
]

NOPE_DEPTH = 128  # per-head K/V depth for DeepSeek V2/3 ("flare_mla_prefill", description)
ROPE_DEPTH = 64   # q_depth - depth, the shared K_rope width ("flare_mla_prefill", Args: k_rope)
Q_DEPTH = NOPE_DEPTH + ROPE_DEPTH

# ---------------------------------------------------------------------------
# float8_e4m3fn -- "flare_mla_prefill", Parameters: dtype may be bfloat16 or
# float8_e4m3fn.  Decoded from the format's definition (OCP 8-bit floating
# point, E4M3 "fn" variant): 1 sign bit, 4 exponent bits with bias 7, 3
# mantissa bits; exponent field 0 is subnormal; no infinities; the all-ones
# exponent+mantissa pattern (S.1111.111) is NaN.
# ---------------------------------------------------------------------------
E4M3FN_MAX = 448.0


def decode_e4m3fn(codes) -> np.ndarray:
    """Map uint8 e4m3fn bit patterns to their exact float64 values."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp_field = (c >> 3) & 0xF
    mant = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + mant / 8.0, exp_field - 7)
    subnormal = sign * np.ldexp(mant / 8.0, -6)
    out = np.where(exp_field == 0, subnormal, normal)
    out = np.where((c & 0x7F) == 0x7F, np.nan, out)
    return out


def dequantize_e4m3fn(codes, scale: float) -> np.ndarray:
    """Exact value of a per-tensor-scaled fp8 tensor: decode(code) * scale.

    Reading R-l: each fp8 operand carries one fp32 scale for the whole
    tensor, and the attention is defined on the dequantised values.
    """
    return decode_e4m3fn(codes) * np.float64(np.float32(scale))


# ---------------------------------------------------------------------------
# Plan -- "generic_flare_mla_prefill_ragged_paged_plan", description and Args.
# ---------------------------------------------------------------------------
def plan(input_row_offsets, cache_lengths, buffer_token_size: int, num_buffer_rows: int):
    """Split the batch's cached contexts over fixed-capacity buffer rows.

    Inputs: ``input_row_offsets`` [B+1] (start of each sequence in the ragged
    token dimension), ``cache_lengths`` [B] (tokens already in the cache
    before this step, the start position), ``buffer_token_size`` (capacity
    of one buffer row) and the number of rows R the caller allocated.

    Readings used:
      R-c/R-h  sequence b's context is its cached prefix plus its new tokens,
               L_b = cache_lengths[b] + n_b, all of it in the cache.
      R-g      the contexts are laid end to end in batch order and cut into
               rows of ``buffer_token_size`` tokens; a sequence may straddle
               rows.  For row r:
                 buffer_row_offsets[r][b]  where sequence b's slice starts in
                                           the row (b = 0..B, so [b]..[b+1]
                                           is its start and end),
                 cache_offsets[r][b]       the first cache position of that
                                           slice within sequence b,
                 buffer_lengths[r]         tokens the row holds; rows the
                                           batch does not reach get -1 and
                                           all-zero offsets.
      status   1 when R rows cannot hold the whole batch, else 0.

    Returns (buffer_row_offsets uint32 [R][B+1], cache_offsets uint32 [R][B],
    buffer_lengths int32 [R], status int).
    """
    iro = np.asarray(input_row_offsets, dtype=np.int64)
    p = np.asarray(cache_lengths, dtype=np.int64)
    B = p.shape[0]
    assert iro.shape == (B + 1,)
    cap = int(buffer_token_size)
    R = int(num_buffer_rows)
    assert cap > 0 and R >= 0
    n = iro[1:] - iro[:-1]
    L = p + n                                   # context length of each sequence
    start = np.zeros(B + 1, dtype=np.int64)     # where each context starts in the stream
    start[1:] = np.cumsum(L)
    total = int(start[B])
    rows_needed = -(-total // cap)              # ceil(total / cap)

    bro = np.zeros((R, B + 1), dtype=np.int64)
    co = np.zeros((R, B), dtype=np.int64)
    bl = np.full(R, -1, dtype=np.int64)
    for r in range(min(R, rows_needed)):
        lo = r * cap                            # stream window [lo, lo + cap)
        for b in range(B + 1):
            bro[r, b] = min(max(start[b] - lo, 0), cap)
        for b in range(B):
            co[r, b] = min(max(lo - start[b], 0), L[b])
        bl[r] = bro[r, B]
    status = 1 if rows_needed > R else 0
    return bro.astype(np.uint32), co.astype(np.uint32), bl.astype(np.int32), status


def _host_array(x):
    """torch (CPU or device) or numpy -> numpy on the host, keeping the values.

    bfloat16 has no numpy dtype, so it is widened to float64 (exact);
    float8_e4m3fn is viewed as its uint8 bit patterns.
    """
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu")
            if x.dtype == torch.float8_e4m3fn:
                return x.view(torch.uint8).numpy()
            if x.dtype == torch.bfloat16:
                return x.to(torch.float64).numpy()
            return x.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x)


# ---------------------------------------------------------------------------
# Paged cache addressing -- reading R-b: cache rows live at
# [layer][physical page][slot in page][kv head 0][column]; the page of logical
# position ``pos`` of sequence b is page_table[b][pos // page_size] and its
# slot is pos % page_size.
# ---------------------------------------------------------------------------
def _cache_row(cache, layer_idx, page_table, page_size, b, pos):
    page = int(page_table[b][pos // page_size])
    return cache[layer_idx, page, pos % page_size, 0, :]


def gather(cache, layer_idx: int, page_table, page_size: int, buffer_row_offsets_r,
           cache_offsets_r, col_begin: int, col_count: int, out):
    """Copy one buffer row's K/V entries from the paged cache into ``out``.

    "generic_flare_mla_prefill_ragged_paged_plan", description: the plan
    exists so that K/V entries can be collected into one contiguous buffer.
    For every sequence b and every j < bro[b+1]-bro[b], buffer slot
    bro[b]+j receives cache position cache_offsets[b]+j of sequence b,
    columns [col_begin, col_begin+col_count) (reading R-r).  Slots the row
    does not use are left as they were.  Returns ``out`` (modified copy).
    """
    cache = _host_array(cache)
    page_table = _host_array(page_table)
    out = np.array(_host_array(out), copy=True)
    bro = _host_array(buffer_row_offsets_r).astype(np.int64)
    co = _host_array(cache_offsets_r).astype(np.int64)
    for b in range(co.shape[0]):
        for j in range(int(bro[b + 1] - bro[b])):
            row = _cache_row(cache, layer_idx, page_table, page_size, b, int(co[b] + j))
            out[bro[b] + j, :] = row[col_begin:col_begin + col_count]
    return out


# ---------------------------------------------------------------------------
# Attention -- "flare_mla_prefill" and "mla_prefill_v2_ragged".
# ---------------------------------------------------------------------------
MASKS = ("causal", "null")


def _visible(qpos, kpos, mask="causal"):
    """Mask [n, m]: is key j visible to query i?

    "mla_prefill_v2_ragged", Args (mask_t, mask_functor): the mask is a
    predicate chosen per call, causal or null among others.
      causal  kpos[j] <= qpos[i]; reading R-e makes the diagonal inclusive
              (a token sees itself).
      null    every key the buffer row holds for the sequence is visible,
              whatever the positions (reading R-s).
    """
    if mask == "causal":
        return kpos[None, :] <= qpos[:, None]
    if mask == "null":
        return np.ones((qpos.shape[0], kpos.shape[0]), dtype=bool)
    raise ValueError(f"unknown mask {mask!r}")


def _query_positions(cache_lengths, b, count):
    """Cache positions of sequence b's new tokens: cache_lengths[b] + i.

    "mla_prefill_v2_ragged", Args (k_nope): the start position is the
    sequence's cache length (readings R-c, R-h).
    """
    return np.int64(cache_lengths[b]) + np.arange(count, dtype=np.int64)


def _key_positions(cache_offsets, b, count):
    """Cache positions of the keys held by one buffer row: cache_offsets[b] + j.

    "flare_mla_prefill", Args (cache_offsets): starting offsets into the
    paged cache, absent for a contiguous cache (reading R-d: absent = 0).
    """
    c0 = 0 if cache_offsets is None else np.int64(cache_offsets[b])
    return c0 + np.arange(count, dtype=np.int64)


def _attend(q_rows, k_nope, k_rope, v, scale, qpos, kpos, mask="causal"):
    """Masked softmax attention of query rows over one key set, float64.

    q_rows [n, 192] (columns 0..127 nope, 128..191 rope: reading R-a);
    k_nope [m, 128] (this head); k_rope [m, 64] (shared by every head);
    v [m, 128]; qpos [n], kpos [m] absolute positions.

    score = scale * (q_nope . k_nope + q_rope . k_rope)   (scale multiplies
    the whole product: "flare_mla_prefill" Args, scale; reading R-f);
    visibility from ``_visible`` (causal: readings R-e; null: R-s);
    output = softmax over visible keys applied to v; a query with no
    visible key gets 0 (reading R-i).

    Returns (out [n, 128], lse [n]) where lse = ln(sum over visible keys of
    exp(score)), -inf for a query with no visible key (reading R-u).
    """
    n = q_rows.shape[0]
    out = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    if n == 0 or k_nope.shape[0] == 0:
        return out, lse
    s = q_rows[:, :NOPE_DEPTH] @ k_nope.T + q_rows[:, NOPE_DEPTH:] @ k_rope.T
    s = s * np.float64(scale)
    visible = _visible(qpos, kpos, mask)
    s = np.where(visible, s, -np.inf)
    has_key = visible.any(axis=1)
    m = np.where(has_key, s.max(axis=1, initial=-np.inf), 0.0)
    w = np.exp(s - m[:, None])                    # exp(-inf) = 0 for hidden keys
    denom = w.sum(axis=1)
    num = w @ v
    out[has_key] = num[has_key] / denom[has_key, None]
    lse[has_key] = m[has_key] + np.log(denom[has_key])
    return out, lse


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Combine two partial attentions over disjoint key sets, float64.

    Each partial is (o, lse): the softmax-weighted mean of its keys' values
    and the log-sum-exp of its keys' scores, as ``_attend`` returns them.
    Softmax over the union weights every key by exp(score - lse) with
    lse = ln(exp(lse_a) + exp(lse_b)), so the union's output is
    exp(lse_a - lse) * o_a + exp(lse_b - lse) * o_b (reading R-v).  Where
    both sides saw no key (lse -inf on both), the result is 0 with lse -inf
    (reading R-i).  o_* [..., D], lse_* [...]; returns (o, lse).
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    some = np.isfinite(lse)
    safe = np.where(some, lse, 0.0)
    wa = np.where(some, np.exp(lse_a - safe), 0.0)
    wb = np.where(some, np.exp(lse_b - safe), 0.0)
    o = wa[..., None] * o_a + wb[..., None] * o_b
    return o, lse


def _as_f64(x, scale=None):
    """Operand values in float64; fp8 codes are decoded and scaled when ``scale`` is given."""
    a = _host_array(x)
    if scale is not None:
        return dequantize_e4m3fn(a.astype(np.uint8), scale)
    return a.astype(np.float64)


def _sequence_keys(b, cache_row_offsets):
    """First buffer row and number of keys of sequence b ("flare_mla_prefill", Args: cache_row_offsets)."""
    g0 = int(cache_row_offsets[b])
    return g0, int(cache_row_offsets[b + 1]) - g0


def mla_prefill_rows(rows, q, k_nope, v, cache, layer_idx, page_table, page_size, rope_col,
                     cache_lengths, valid_length, cache_row_offsets, cache_offsets, scale,
                     scales=None, mask="causal", return_lse=False):
    """Output of selected (token, head) pairs, float64 [len(rows), 128].

    ``rows`` is a list of (t, h).  Same definition as ``mla_prefill_ragged``
    evaluated one output row at a time (used to check large problems on a
    sample of outputs).  ``scales`` = dict(q=, k_nope=, v=, k_rope=) when the
    inputs are fp8 codes (reading R-l), else None.  With ``return_lse`` the
    log-sum-exp of each pair is returned too, (out, lse [len(rows)]).
    """
    sc = scales or {}
    fp8 = scales is not None
    vl = np.asarray(valid_length, dtype=np.int64)
    cro = np.asarray(cache_row_offsets, dtype=np.int64)
    co = None if cache_offsets is None else np.asarray(cache_offsets, dtype=np.int64)
    p = np.asarray(cache_lengths, dtype=np.int64)
    B = vl.shape[0] - 1
    out = np.zeros((len(rows), NOPE_DEPTH), dtype=np.float64)
    lse = np.full(len(rows), -np.inf, dtype=np.float64)
    for idx, (t, h) in enumerate(rows):
        b = int(np.searchsorted(vl, t, side="right") - 1)
        assert 0 <= b < B and vl[b] <= t < vl[b + 1]
        i = t - vl[b]
        g0, count = _sequence_keys(b, cro)
        kpos = _key_positions(co, b, count)
        qpos = _query_positions(p, b, i + 1)[i:i + 1]
        qrow = _as_f64(q[t:t + 1, h, :], sc.get("q") if fp8 else None)
        kn = _as_f64(k_nope[g0:g0 + count, h, :], sc.get("k_nope") if fp8 else None)
        vv = _as_f64(v[g0:g0 + count, h, :], sc.get("v") if fp8 else None)
        kr_codes = rope_rows(cache, layer_idx, page_table, page_size, rope_col, b, kpos)
        kr = _as_f64(kr_codes, sc.get("k_rope") if fp8 else None)
        o1, l1 = _attend(qrow, kn, kr, vv, scale, qpos, kpos, mask)
        out[idx], lse[idx] = o1[0], l1[0]
    return (out, lse) if return_lse else out


def rope_rows(cache, layer_idx, page_table, page_size, rope_col, b, positions):
    """Raw K_rope cache entries of sequence b at ``positions`` [len, 64] (host numpy).

    "flare_mla_prefill", description and Args (k_rope): the 64 columns of K
    beyond the per-head depth come from the KV cache, one single-head row
    per cache position, and are shared by every head.  Reading R-b: they
    sit at columns rope_col .. rope_col+63 of the cache row.  Values are
    returned as stored (bf16 widened exactly, fp8 as codes).
    """
    cache = _host_array(cache)
    page_table = _host_array(page_table)
    rows = [_cache_row(cache, layer_idx, page_table, page_size, b, int(pos))[rope_col:rope_col + ROPE_DEPTH]
            for pos in positions]
    if not rows:
        return np.zeros((0, ROPE_DEPTH), dtype=cache.dtype)
    return np.stack(rows)


def mla_prefill_ragged(q, k_nope, v, cache, layer_idx, page_table, page_size, rope_col,
                       cache_lengths, valid_length, cache_row_offsets, cache_offsets, scale,
                       scales=None, q_block=512, mask="causal", return_lse=False):
    """Full output [T, H, 128] float64 of one ragged MLA prefill call.

    Shapes ("flare_mla_prefill", description and Args):
      q        [T, H, 192]        ragged over the batch by ``valid_length``
      k_nope   [rows, H, 128]     ragged K/V buffer, sequence b's keys at rows
      v        [rows, H, 128]     cache_row_offsets[b] .. cache_row_offsets[b+1]
      cache    [layers, pages, page_size, 1, width]  paged KV cache holding
               K_rope at columns rope_col .. rope_col+63 (reading R-b)
    For sequence b (readings R-c, R-d, R-h):
      query i (token valid_length[b]+i) sits at position cache_lengths[b]+i;
      key j (buffer row cache_row_offsets[b]+j) sits at position
      cache_offsets[b]+j (0 when cache_offsets is None: a contiguous cache).
    ``scales`` (fp8 inputs, reading R-l): dict(q=, k_nope=, v=, k_rope=) of
    per-tensor fp32 scales; the inputs are then uint8/float8 codes.
    ``mask`` is "causal" or "null" (``_visible``).  With ``return_lse``
    returns (out, lse [T, H]), the log-sum-exp of each (token, head) over the
    keys this call sees (reading R-u).
    Query rows are processed in blocks of ``q_block`` only to bound memory;
    every output row is computed exactly as its definition states.
    """
    sc = scales or {}
    fp8 = scales is not None
    vl = np.asarray(valid_length, dtype=np.int64)
    cro = np.asarray(cache_row_offsets, dtype=np.int64)
    co = None if cache_offsets is None else np.asarray(cache_offsets, dtype=np.int64)
    p = np.asarray(cache_lengths, dtype=np.int64)
    B = vl.shape[0] - 1
    T, H = int(q.shape[0]), int(q.shape[1])
    out = np.zeros((T, H, NOPE_DEPTH), dtype=np.float64)
    lse = np.full((T, H), -np.inf, dtype=np.float64)
    for b in range(B):
        t0, t1 = int(vl[b]), int(vl[b + 1])
        if t1 == t0:
            continue
        g0, count = _sequence_keys(b, cro)
        kpos = _key_positions(co, b, count)
        kr = _as_f64(rope_rows(cache, layer_idx, page_table, page_size, rope_col, b, kpos),
                     sc.get("k_rope") if fp8 else None)
        qpos_all = _query_positions(p, b, t1 - t0)
        for h in range(H):
            kn = _as_f64(k_nope[g0:g0 + count, h, :], sc.get("k_nope") if fp8 else None)
            vv = _as_f64(v[g0:g0 + count, h, :], sc.get("v") if fp8 else None)
            for s0 in range(t0, t1, q_block):
                s1 = min(s0 + q_block, t1)
                qb = _as_f64(q[s0:s1, h, :], sc.get("q") if fp8 else None)
                out[s0:s1, h, :], lse[s0:s1, h] = _attend(qb, kn, kr, vv, scale,
                                                          qpos_all[s0 - t0:s1 - t0], kpos, mask)
    return (out, lse) if return_lse else out


def mla_prefill_ragged_split(q_nope, q_rope, k_nope, v, cache_lengths, valid_length, cache_row_offsets,
                             cache_offsets, scale, k_rope_rows=None, cache=None, layer_idx=0, page_table=None,
                             page_size=None, rope_col=None, scales=None, mask="causal", return_lse=False):
    """Split-Q attention: "flare_mla_prefill", the overloads whose query comes in
    two tensors, q_nope [T, H, 128] (with q_scale when fp8) and q_rope [T, H, 64],
    and whose K carries k_scales; K_rope either paged (from the cache, as in
    ``mla_prefill_ragged``) or contiguous.

    Reading R-w: the score is the one of ``mla_prefill_ragged`` with the query's
    columns 0..127 taken from q_nope and 128..191 from q_rope; q_rope is never
    quantised (its type is not tied to q_nope's), so q_scale applies to q_nope
    only.  ``scales`` (fp8 operands) = dict(q=, k_nope=, v=, k_rope=): q scales
    q_nope, k_nope is the pages' k_scales (one fp32 per tensor, reading R-l),
    k_rope the cache's scale (paged fp8 cache only).
    Reading R-x: a contiguous K_rope ``k_rope_rows`` [rows, 1, 64] (or [rows, 64])
    is laid out like K and V: key j of sequence b uses row
    cache_row_offsets[b] + j.  Without it, K_rope comes from the paged cache.
    Returns [T, H, 128] float64 (and lse [T, H] with ``return_lse``).
    """
    sc = scales or {}
    fp8 = scales is not None
    qn = _as_f64(q_nope, sc.get("q") if fp8 else None)
    qr = _as_f64(q_rope)
    q = np.concatenate([qn, qr], axis=2)
    vl = np.asarray(valid_length, dtype=np.int64)
    cro = np.asarray(cache_row_offsets, dtype=np.int64)
    co = None if cache_offsets is None else np.asarray(cache_offsets, dtype=np.int64)
    p = np.asarray(cache_lengths, dtype=np.int64)
    B = vl.shape[0] - 1
    T, H = int(q.shape[0]), int(q.shape[1])
    out = np.zeros((T, H, NOPE_DEPTH), dtype=np.float64)
    lse = np.full((T, H), -np.inf, dtype=np.float64)
    contig = None
    if k_rope_rows is not None:
        contig = _as_f64(k_rope_rows).reshape(-1, ROPE_DEPTH)
    for b in range(B):
        t0, t1 = int(vl[b]), int(vl[b + 1])
        if t1 == t0:
            continue
        g0, count = _sequence_keys(b, cro)
        kpos = _key_positions(co, b, count)
        if contig is not None:
            kr = contig[g0:g0 + count]
        else:
            kr = _as_f64(rope_rows(cache, layer_idx, page_table, page_size, rope_col, b, kpos),
                         sc.get("k_rope") if fp8 else None)
        qpos = _query_positions(p, b, t1 - t0)
        for h in range(H):
            kn = _as_f64(k_nope[g0:g0 + count, h, :], sc.get("k_nope") if fp8 else None)
            vv = _as_f64(v[g0:g0 + count, h, :], sc.get("v") if fp8 else None)
            out[t0:t1, h, :], lse[t0:t1, h] = _attend(q[t0:t1, h, :], kn, kr, vv, scale, qpos, kpos, mask)
    return (out, lse) if return_lse else out


def mla_prefill_rows_split(rows, q_nope, q_rope, k_nope, v, cache_lengths, valid_length, cache_row_offsets,
                           cache_offsets, scale, k_rope_rows=None, cache=None, layer_idx=0, page_table=None,
                           page_size=None, rope_col=None, scales=None, mask="causal"):
    """Selected (t, h) outputs of ``mla_prefill_ragged_split``, float64 [len(rows), 128],
    evaluated one output row at a time (for large problems)."""
    sc = scales or {}
    fp8 = scales is not None
    vl = np.asarray(valid_length, dtype=np.int64)
    cro = np.asarray(cache_row_offsets, dtype=np.int64)
    co = None if cache_offsets is None else np.asarray(cache_offsets, dtype=np.int64)
    p = np.asarray(cache_lengths, dtype=np.int64)
    B = vl.shape[0] - 1
    out = np.zeros((len(rows), NOPE_DEPTH), dtype=np.float64)
    for idx, (t, h) in enumerate(rows):
        b = int(np.searchsorted(vl, t, side="right") - 1)
        assert 0 <= b < B and vl[b] <= t < vl[b + 1]
        i = t - vl[b]
        g0, count = _sequence_keys(b, cro)
        kpos = _key_positions(co, b, count)
        qpos = _query_positions(p, b, i + 1)[i:i + 1]
        qrow = np.concatenate([_as_f64(q_nope[t:t + 1, h, :], sc.get("q") if fp8 else None),
                               _as_f64(q_rope[t:t + 1, h, :])], axis=1)
        kn = _as_f64(k_nope[g0:g0 + count, h, :], sc.get("k_nope") if fp8 else None)
        vv = _as_f64(v[g0:g0 + count, h, :], sc.get("v") if fp8 else None)
        if k_rope_rows is not None:
            kr = _as_f64(k_rope_rows[g0:g0 + count]).reshape(count, ROPE_DEPTH)
        else:
            kr = _as_f64(rope_rows(cache, layer_idx, page_table, page_size, rope_col, b, kpos),
                         sc.get("k_rope") if fp8 else None)
        out[idx] = _attend(qrow, kn, kr, vv, scale, qpos, kpos, mask)[0][0]
    return out


def latent_up(cache, layer_idx, page_table, page_size, buffer_row_offsets_r, cache_offsets_r, latent_col,
              latent_dim, w_kv, heads, cap, slots=None):
    """Per-head K_nope and V of one buffer row from the latent cache, float64.

    The pages call the cache a latent cache ("mla_prefill_v2_ragged", Args: the
    V operand is the nope segment of the latent cache) and give no
    decompression step; reading R-y takes the DeepSeek-V2/V3 form: each cache
    row holds a latent vector c (columns latent_col .. latent_col+latent_dim-1)
    and the per-head keys and values are linear in it,
      K_nope[g][h][d] = sum_c w_kv[h*256 + d][c]       * c_g[c]
      V[g][h][d]      = sum_c w_kv[h*256 + 128 + d][c] * c_g[c]
    with w_kv [heads*256][latent_dim] (per head, 128 key rows then 128 value
    rows) and c_g the latent of the cache position that buffer slot g holds
    under the plan row (``gather``).  Returns (k_nope, v), each [cap, heads,
    128]; slots the row does not use are 0.  With ``slots`` (a list of slot
    indices) only those slots are computed: [len(slots), heads, 128] each.
    """
    lat = gather(cache, layer_idx, page_table, page_size, buffer_row_offsets_r, cache_offsets_r,
                 latent_col, latent_dim, np.zeros((cap, latent_dim)))
    lat = np.asarray(lat, dtype=np.float64)
    used = int(np.asarray(_host_array(buffer_row_offsets_r), dtype=np.int64)[-1])
    lat[used:] = 0.0
    if slots is not None:
        lat = lat[np.asarray(slots, dtype=np.int64)]
    w = _as_f64(w_kv).reshape(heads, 2, NOPE_DEPTH, latent_dim)
    kv = np.einsum("gc,hpdc->gphd", lat, w, optimize=True)   # [slots, 2, heads, 128]
    return kv[:, 0], kv[:, 1]

