"""ctypes binding of ``include/mla_prefill.h``: argument marshalling only.

Every function takes device tensors (torch, on the current HIP device) and
passes their data pointers, sizes and the current stream to the C entry point
of the same name.  A non-zero status raises ``MlaError``.  Integer index arrays
may be torch.int32 or torch.uint32 tensors (4-byte elements, values < 2**31
when int32).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmla_prefill.so")

MLA_BF16 = 0
MLA_FP8_E4M3FN = 1
MLA_FP32 = 2
MLA_MASK_CAUSAL = 0
MLA_MASK_NULL = 1
_MASKS = {"causal": MLA_MASK_CAUSAL, "null": MLA_MASK_NULL}
MLA_MAX_BATCH = 8192
MLA_ERR_PRECONDITION = 7
MLA_VIOLATION_Q_OFFSETS = 1
MLA_VIOLATION_ROW_OFFSETS = 2
MLA_VIOLATION_POSITIONS = 4
MLA_VIOLATION_PAGE_IDS = 8

_STATUS_NAMES = {0: "MLA_OK", 1: "MLA_ERR_NULL_ARG", 2: "MLA_ERR_BAD_SHAPE", 3: "MLA_ERR_UNSUPPORTED_DTYPE",
                 4: "MLA_ERR_UNSUPPORTED_DIMS", 5: "MLA_ERR_UNSUPPORTED_MASK", 6: "MLA_ERR_HIP",
                 7: "MLA_ERR_PRECONDITION"}


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {mla_status_string(status)}"
        if status == 6:
            msg += f" (hipError {mla_prefill_last_hip_error()})"
        super().__init__(msg)


class _Cache(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int), ("num_layers", ctypes.c_uint32),
                ("num_pages", ctypes.c_uint32), ("page_size", ctypes.c_uint32), ("row_width", ctypes.c_uint32),
                ("rope_col", ctypes.c_uint32), ("page_table", ctypes.c_void_p),
                ("max_pages_per_seq", ctypes.c_uint32), ("cache_lengths", ctypes.c_void_p),
                ("scale", ctypes.c_void_p)]


def library_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python mla_ragged_paged_amd/build.py` "
                          "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    u32, vp, i32 = ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
    cp = ctypes.POINTER(_Cache)
    lib.mla_prefill_plan.argtypes = [vp, u32, cp, u32, u32, u32, vp, vp, vp, vp, vp]
    lib.mla_prefill_plan.restype = i32
    lib.mla_prefill_gather.argtypes = [cp, u32, u32, vp, vp, u32, u32, u32, vp, vp]
    lib.mla_prefill_gather.restype = i32
    lib.mla_prefill_ragged.argtypes = [vp, i32, vp, i32, vp, vp, cp, u32, vp, vp, vp, u32, u32, u32, u32, u32,
                                       i32, ctypes.c_float, vp, vp, vp, u32, vp]
    lib.mla_prefill_ragged.restype = i32
    lib.mla_prefill_ragged_lse.argtypes = [vp, i32, vp, vp, vp, vp, i32, vp, vp, cp, u32, vp, vp, vp, u32, u32, u32,
                                           u32, u32, i32, ctypes.c_float, vp, vp, vp, u32, vp]
    lib.mla_prefill_ragged_lse.restype = i32
    lib.mla_prefill_ragged_row.argtypes = [vp, i32, vp, vp, vp, vp, i32, vp, vp, cp, u32, vp, vp, vp, u32, u32, u32,
                                           u32, u32, i32, ctypes.c_float, vp, vp, vp, u32, vp]
    lib.mla_prefill_ragged_row.restype = i32
    lib.mla_prefill_ragged_split.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, cp, u32, vp, vp, vp,
                                             u32, u32, u32, u32, i32, ctypes.c_float, u32, vp]
    lib.mla_prefill_ragged_split.restype = i32
    lib.mla_prefill_ragged_kvsplit.argtypes = [vp, i32, vp, vp, i32, vp, vp, cp, u32, vp, vp, vp, u32, u32, u32, u32,
                                               u32, i32, ctypes.c_float, vp, vp, vp, u32, u32, vp, ctypes.c_uint64,
                                               vp]
    lib.mla_prefill_ragged_kvsplit.restype = i32
    lib.mla_prefill_ragged_kvsplit_noalloc.argtypes = [vp, i32, vp, vp, i32, vp, vp, cp, u32, vp, vp, vp, u32, u32,
                                                       u32, u32, u32, i32, ctypes.c_float, vp, vp, vp, u32, u32, vp]
    lib.mla_prefill_ragged_kvsplit_noalloc.restype = i32
    lib.mla_prefill_kvsplit_workspace_bytes.argtypes = [u32, u32]
    lib.mla_prefill_kvsplit_workspace_bytes.restype = ctypes.c_uint64
    lib.mla_prefill_ragged_krope.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, u32, u32, u32, u32, u32,
                                             i32, ctypes.c_float, vp, vp, vp, u32, vp]
    lib.mla_prefill_ragged_krope.restype = i32
    lib.mla_prefill_ragged_row_krope.argtypes = [vp, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, u32, u32,
                                                 u32, u32, u32, i32, ctypes.c_float, vp, vp, vp, u32, vp]
    lib.mla_prefill_ragged_row_krope.restype = i32
    lib.mla_prefill_latent_up.argtypes = [cp, u32, u32, vp, vp, u32, u32, vp, u32, u32, vp, vp, vp]
    lib.mla_prefill_latent_up.restype = i32
    lib.mla_prefill_merge.argtypes = [vp, i32, vp, vp, vp, vp, vp, u32, u32, u32, vp]
    lib.mla_prefill_merge.restype = i32
    lib.mla_prefill_check.argtypes = [cp, vp, u32, u32, u32, vp, vp, u32, vp, vp]
    lib.mla_prefill_check.restype = i32
    lib.mla_prefill_set_debug.argtypes = [i32]
    lib.mla_prefill_set_debug.restype = i32
    lib.mla_status_string.argtypes = [i32]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_prefill_last_hip_error.argtypes = []
    lib.mla_prefill_last_hip_error.restype = i32
    return lib


_lib = _load()


def mla_status_string(status: int) -> str:
    return _lib.mla_status_string(int(status)).decode()


def mla_prefill_last_hip_error() -> int:
    return int(_lib.mla_prefill_last_hip_error())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _idx(t, name):
    if t is None:
        return None
    if t.element_size() != 4 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous 4-byte integer tensor")
    return _ptr(t)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    if t.dtype == torch.float32:
        return MLA_FP32
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return MLA_FP8_E4M3FN
    raise TypeError(f"unsupported dtype {t.dtype}")


@dataclass
class PagedCache:
    """Host-side description of one paged KV cache (``mla_paged_cache_t``).

    data:          [num_layers, num_pages, page_size, 1, row_width] bf16 or float8_e4m3fn
    page_table:    [batch, max_pages_per_seq] int32/uint32
    cache_lengths: [batch] int32/uint32
    scale:         [1] float32 device tensor (fp8 caches only)
    """
    data: torch.Tensor
    page_table: torch.Tensor
    cache_lengths: torch.Tensor
    rope_col: int
    scale: torch.Tensor | None = None

    def as_struct(self) -> _Cache:
        d = self.data
        if d.dim() != 5 or d.shape[3] != 1 or not d.is_contiguous():
            raise ValueError("cache data must be a contiguous [layers, pages, page_size, 1, row_width] tensor")
        return _Cache(data=d.data_ptr(), dtype=_dtype_code(d), num_layers=d.shape[0], num_pages=d.shape[1],
                      page_size=d.shape[2], row_width=d.shape[4], rope_col=self.rope_col,
                      page_table=_idx(self.page_table, "page_table").value,
                      max_pages_per_seq=self.page_table.shape[1],
                      cache_lengths=_idx(self.cache_lengths, "cache_lengths").value,
                      scale=None if self.scale is None else self.scale.data_ptr())


def _check(status: int, where: str):
    if status != 0:
        raise MlaError(status, where)


def mla_prefill_plan(input_row_offsets, kv: PagedCache, layer_idx, buffer_token_size, buffer_row_offsets,
                     cache_offsets, buffer_lengths, device_status=None, stream=None):
    """Fill the plan outputs [R][B+1], [R][B], [R] (and the status flag) for the batch."""
    batch = input_row_offsets.shape[0] - 1
    rows = buffer_lengths.shape[0]
    s = kv.as_struct()
    _check(_lib.mla_prefill_plan(_idx(input_row_offsets, "input_row_offsets"), batch, ctypes.byref(s), layer_idx,
                                 buffer_token_size, rows, _idx(buffer_row_offsets, "buffer_row_offsets"),
                                 _idx(cache_offsets, "cache_offsets"), _idx(buffer_lengths, "buffer_lengths"),
                                 _idx(device_status, "device_status"), _stream(stream)), "mla_prefill_plan")


def mla_prefill_gather(kv: PagedCache, layer_idx, buffer_row_offsets_r, cache_offsets_r, col_begin, col_count,
                       out, stream=None):
    """Copy one plan row's cache entries, columns [col_begin, +col_count), into out [cap, col_count]."""
    batch = cache_offsets_r.shape[0]
    s = kv.as_struct()
    _check(_lib.mla_prefill_gather(ctypes.byref(s), layer_idx, batch, _idx(buffer_row_offsets_r, "bro"),
                                   _idx(cache_offsets_r, "cache_offsets"), col_begin, col_count, out.shape[0],
                                   _ptr(out), _stream(stream)), "mla_prefill_gather")


def _mask_code(mask) -> int:
    if mask not in _MASKS:
        raise ValueError(f"mask must be one of {sorted(_MASKS)}, got {mask!r}")
    return _MASKS[mask]


def _contiguous(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _shapes(T, H, rows=(), lses=()):
    """Output-side arrays must be [T, H, 128] (rows) and [T, H] (lses): the kernels
    touch every (token, head)."""
    for name, t in rows:
        if t is not None and tuple(t.shape) != (T, H, 128):
            raise ValueError(f"{name} must have shape {(T, H, 128)}, got {tuple(t.shape)}")
    for name, t in lses:
        if t is not None and tuple(t.shape) != (T, H):
            raise ValueError(f"{name} must have shape {(T, H)}, got {tuple(t.shape)}")


def _kv(H, dtype, k_nope, v):
    """K_nope and V must be [rows, H, 128] with H and the element type of the query:
    the kernels stride their rows by the query's head count and read them in its type."""
    for name, t in (("k_nope", k_nope), ("v", v)):
        if t.dim() != 3 or tuple(t.shape[1:]) != (H, 128):
            raise ValueError(f"{name} must have shape [rows, {H}, 128], got {tuple(t.shape)}")
        if _dtype_code(t) != _dtype_code_of(dtype):
            raise TypeError(f"{name} must have the query's element type {dtype}, got {t.dtype}")
    if k_nope.shape[0] != v.shape[0]:
        raise ValueError(f"k_nope and v must have the same rows, got {k_nope.shape[0]} and {v.shape[0]}")


def _dtype_code_of(dtype) -> int:
    if dtype == torch.bfloat16:
        return MLA_BF16
    if dtype in (torch.float8_e4m3fn, torch.uint8):
        return MLA_FP8_E4M3FN
    raise TypeError(f"unsupported query dtype {dtype}")


def _f32(t, name):
    if t is not None and t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    return _ptr(t)


def mla_prefill_ragged(output, q, k_nope, v, k_rope: PagedCache, layer_idx, valid_length, cache_row_offsets,
                       cache_offsets, scale, q_scale=None, k_nope_scale=None, v_scale=None, q_max_seq_len=0,
                       stream=None, mask="causal"):
    """MLA prefill: output [T, H, 128] (bf16 or fp32) from q [T, H, 192] and the ragged K/V buffer.

    ``mask`` is "causal" or "null"."""
    T, H, qd = q.shape
    _contiguous(output=output, q=q, k_nope=k_nope, v=v)
    _shapes(T, H, rows=[("output", output)])
    _kv(H, q.dtype, k_nope, v)
    s = k_rope.as_struct()
    _check(_lib.mla_prefill_ragged(_ptr(output), _dtype_code(output), _ptr(q), _dtype_code(q), _ptr(k_nope),
                                   _ptr(v), ctypes.byref(s), layer_idx, _idx(valid_length, "valid_length"),
                                   _idx(cache_row_offsets, "cache_row_offsets"),
                                   _idx(cache_offsets, "cache_offsets"), valid_length.shape[0] - 1, T, H, qd,
                                   k_nope.shape[2], _mask_code(mask), float(scale), _ptr(q_scale),
                                   _ptr(k_nope_scale), _ptr(v_scale), int(q_max_seq_len), _stream(stream)),
           "mla_prefill_ragged")


def mla_prefill_ragged_lse(output, lse, q, k_nope, v, k_rope: PagedCache, layer_idx, valid_length,
                           cache_row_offsets, cache_offsets, scale, prev_output=None, prev_lse=None, q_scale=None,
                           k_nope_scale=None, v_scale=None, q_max_seq_len=0, stream=None, mask="causal"):
    """One buffer row's attention with its log-sum-exp lse [T, H] (float32, or None),
    merged with an earlier partial (prev_output fp32 [T, H, 128], prev_lse [T, H]) when given.
    output / lse may be the same tensors as prev_output / prev_lse."""
    T, H, qd = q.shape
    _contiguous(output=output, lse=lse, q=q, k_nope=k_nope, v=v, prev_output=prev_output, prev_lse=prev_lse)
    _shapes(T, H, rows=[("output", output), ("prev_output", prev_output)], lses=[("lse", lse), ("prev_lse", prev_lse)])
    _kv(H, q.dtype, k_nope, v)
    s = k_rope.as_struct()
    _check(_lib.mla_prefill_ragged_lse(_ptr(output), _dtype_code(output), _f32(lse, "lse"),
                                       _f32(prev_output, "prev_output"), _f32(prev_lse, "prev_lse"), _ptr(q),
                                       _dtype_code(q), _ptr(k_nope), _ptr(v), ctypes.byref(s), layer_idx,
                                       _idx(valid_length, "valid_length"),
                                       _idx(cache_row_offsets, "cache_row_offsets"),
                                       _idx(cache_offsets, "cache_offsets"), valid_length.shape[0] - 1, T, H, qd,
                                       k_nope.shape[2], _mask_code(mask), float(scale), _ptr(q_scale),
                                       _ptr(k_nope_scale), _ptr(v_scale), int(q_max_seq_len), _stream(stream)),
           "mla_prefill_ragged_lse")


def mla_prefill_check(kv: PagedCache, violations, valid_length=None, total_q_tokens=None, q_max_seq_len=0,
                      row_offsets=None, row_positions=None, row_capacity=0, stream=None):
    """Device-side check of a call's device data: ORs MLA_VIOLATION_* bits into ``violations``
    (a one-element int32 device tensor the caller zeroes).  ``total_q_tokens`` None: not checked."""
    if violations.dtype != torch.int32 or violations.numel() < 1:
        raise TypeError("violations must be an int32 tensor")
    batch = (valid_length if valid_length is not None else row_offsets).shape[0] - 1
    s = kv.as_struct()
    T = 0xFFFFFFFF if total_q_tokens is None else int(total_q_tokens)
    _check(_lib.mla_prefill_check(ctypes.byref(s), _idx(valid_length, "valid_length"), batch, T, int(q_max_seq_len),
                                  _idx(row_offsets, "row_offsets"), _idx(row_positions, "row_positions"),
                                  int(row_capacity), _ptr(violations), _stream(stream)),
           "mla_prefill_check")


def mla_prefill_set_debug(on: bool) -> bool:
    """Debug mode on or off (every call checks its device data first); returns the previous setting."""
    return bool(_lib.mla_prefill_set_debug(1 if on else 0))


def mla_prefill_kvsplit_workspace_bytes(total_q_tokens: int, num_heads: int) -> int:
    """Bytes of the fp32 workspace mla_prefill_ragged_kvsplit needs for T tokens and H heads."""
    return int(_lib.mla_prefill_kvsplit_workspace_bytes(int(total_q_tokens), int(num_heads)))


def mla_prefill_ragged_kvsplit(output, q, k_nope, v, k_rope: PagedCache, layer_idx, valid_length,
                               cache_row_offsets, cache_offsets, scale, split_keys, workspace, lse=None,
                               q_scale=None, k_nope_scale=None, v_scale=None, q_max_seq_len=0, stream=None,
                               mask="causal"):
    """The attention of mla_prefill_ragged (and its log-sum-exp lse [T, H] when given) with
    each 128-query tile that sees more than ``split_keys`` keys computed as two halves of its
    key tiles and merged; ``workspace`` is a float32 tensor of at least
    mla_prefill_kvsplit_workspace_bytes(T, H) bytes (unused when split_keys is 0)."""
    T, H, qd = q.shape
    _contiguous(output=output, lse=lse, q=q, k_nope=k_nope, v=v, workspace=workspace)
    _shapes(T, H, rows=[("output", output)], lses=[("lse", lse)])
    _kv(H, q.dtype, k_nope, v)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = k_rope.as_struct()
    _check(_lib.mla_prefill_ragged_kvsplit(_ptr(output), _dtype_code(output), _f32(lse, "lse"), _ptr(q),
                                           _dtype_code(q), _ptr(k_nope), _ptr(v), ctypes.byref(s), layer_idx,
                                           _idx(valid_length, "valid_length"),
                                           _idx(cache_row_offsets, "cache_row_offsets"),
                                           _idx(cache_offsets, "cache_offsets"), valid_length.shape[0] - 1, T, H,
                                           qd, k_nope.shape[2], _mask_code(mask), float(scale), _ptr(q_scale),
                                           _ptr(k_nope_scale), _ptr(v_scale), int(q_max_seq_len), int(split_keys),
                                           _f32(workspace, "workspace"), nbytes, _stream(stream)),
           "mla_prefill_ragged_kvsplit")


MLA_NOALLOC_SCRATCH_BYTES = 64 << 20


def mla_prefill_ragged_kvsplit_noalloc(output, q, k_nope, v, k_rope: PagedCache, layer_idx, valid_length,
                                       cache_row_offsets, cache_offsets, scale, split_keys, lse=None, q_scale=None,
                                       k_nope_scale=None, v_scale=None, q_max_seq_len=0, stream=None,
                                       mask="causal"):
    """mla_prefill_ragged_kvsplit with the partials in the library's own device array
    (MLA_NOALLOC_SCRATCH_BYTES per GPU): no workspace, nothing allocated.  Split calls
    that may overlap in time on one GPU race."""
    T, H, qd = q.shape
    _contiguous(output=output, lse=lse, q=q, k_nope=k_nope, v=v)
    _shapes(T, H, rows=[("output", output)], lses=[("lse", lse)])
    _kv(H, q.dtype, k_nope, v)
    s = k_rope.as_struct()
    _check(_lib.mla_prefill_ragged_kvsplit_noalloc(_ptr(output), _dtype_code(output), _f32(lse, "lse"), _ptr(q),
                                                   _dtype_code(q), _ptr(k_nope), _ptr(v), ctypes.byref(s),
                                                   layer_idx, _idx(valid_length, "valid_length"),
                                                   _idx(cache_row_offsets, "cache_row_offsets"),
                                                   _idx(cache_offsets, "cache_offsets"), valid_length.shape[0] - 1,
                                                   T, H, qd, k_nope.shape[2], _mask_code(mask), float(scale),
                                                   _ptr(q_scale), _ptr(k_nope_scale), _ptr(v_scale),
                                                   int(q_max_seq_len), int(split_keys), _stream(stream)),
           "mla_prefill_ragged_kvsplit_noalloc")


def mla_prefill_ragged_row(output, acc, acc_lse, q, k_nope, v, k_rope: PagedCache, layer_idx, valid_length,
                           cache_row_offsets, cache_offsets, scale, lse=None, q_scale=None, k_nope_scale=None,
                           v_scale=None, q_max_seq_len=0, stream=None, mask="causal"):
    """One row of a multi-row plan (rows called in order): each token's partial carried in acc fp32
    [T, H, 128] / acc_lse [T, H] from its sequence's first row to the row holding its last visible
    key, which writes output (and lse)."""
    T, H, qd = q.shape
    _contiguous(output=output, lse=lse, acc=acc, acc_lse=acc_lse, q=q, k_nope=k_nope, v=v)
    _shapes(T, H, rows=[("output", output), ("acc", acc)], lses=[("lse", lse), ("acc_lse", acc_lse)])
    _kv(H, q.dtype, k_nope, v)
    s = k_rope.as_struct()
    _check(_lib.mla_prefill_ragged_row(_ptr(output), _dtype_code(output), _f32(lse, "lse"), _f32(acc, "acc"),
                                       _f32(acc_lse, "acc_lse"), _ptr(q), _dtype_code(q), _ptr(k_nope), _ptr(v),
                                       ctypes.byref(s), layer_idx, _idx(valid_length, "valid_length"),
                                       _idx(cache_row_offsets, "cache_row_offsets"),
                                       _idx(cache_offsets, "cache_offsets"), valid_length.shape[0] - 1, T, H, qd,
                                       k_nope.shape[2], _mask_code(mask), float(scale), _ptr(q_scale),
                                       _ptr(k_nope_scale), _ptr(v_scale), int(q_max_seq_len), _stream(stream)),
           "mla_prefill_ragged_row")


def mla_prefill_ragged_split(output, q_nope, q_rope, k_nope, v, kv: PagedCache, layer_idx, valid_length,
                             cache_row_offsets, cache_offsets, scale, q_scale=None, k_scales=None, v_scale=None,
                             k_rope_rows=None, lse=None, q_max_seq_len=0, stream=None, mask="causal",
                             k_rope_scale=None):
    """Split-query attention: q_nope [T, H, 128] (bf16 or fp8 with q_scale), q_rope [T, H, 64] bf16;
    K_rope from ``kv`` (paged) or from contiguous rows ``k_rope_rows`` [rows, 1, 64], bf16 or
    (with an fp8 q_nope) float8_e4m3fn with its scale ``k_rope_scale`` ([1] float32)."""
    T, H, qd = q_nope.shape
    _contiguous(output=output, lse=lse, q_nope=q_nope, q_rope=q_rope, k_nope=k_nope, v=v, k_rope_rows=k_rope_rows)
    _shapes(T, H, rows=[("output", output)], lses=[("lse", lse)])
    _kv(H, q_nope.dtype, k_nope, v)
    if tuple(q_rope.shape) != (T, H, 64) or q_rope.dtype != torch.bfloat16:
        raise ValueError(f"q_rope must be bf16 of shape {(T, H, 64)}")
    if k_rope_rows is not None:
        if k_rope_rows.shape[-1] != 64 or k_rope_rows.dtype not in (torch.bfloat16, torch.float8_e4m3fn):
            raise ValueError("k_rope_rows must be bf16 or float8_e4m3fn [rows, 1, 64]")
        if (k_rope_rows.dtype == torch.float8_e4m3fn) != (k_rope_scale is not None):
            raise ValueError("e4m3 k_rope_rows need k_rope_scale (and bf16 rows take none)")
        s = _Cache(data=None, dtype=_dtype_code(k_rope_rows), num_layers=0, num_pages=0, page_size=0, row_width=0,
                   rope_col=0, page_table=None, max_pages_per_seq=0,
                   cache_lengths=_idx(kv.cache_lengths, "cache_lengths").value,
                   scale=None if k_rope_scale is None else k_rope_scale.data_ptr())
    else:
        s = kv.as_struct()
    _check(_lib.mla_prefill_ragged_split(_ptr(output), _dtype_code(output), _f32(lse, "lse"), _ptr(q_nope),
                                         _ptr(q_rope), _dtype_code(q_nope), _ptr(q_scale), _ptr(k_nope),
                                         _ptr(k_scales), _ptr(v), _ptr(v_scale), _ptr(k_rope_rows),
                                         ctypes.byref(s), layer_idx, _idx(valid_length, "valid_length"),
                                         _idx(cache_row_offsets, "cache_row_offsets"),
                                         _idx(cache_offsets, "cache_offsets"), valid_length.shape[0] - 1, T, H,
                                         k_nope.shape[2], _mask_code(mask), float(scale), int(q_max_seq_len),
                                         _stream(stream)),
           "mla_prefill_ragged_split")


def mla_prefill_ragged_krope(output, q, k_nope, v, k_rope, cache_lengths, valid_length, cache_row_offsets,
                             cache_offsets, scale, k_rope_scale=None, q_scale=None, k_nope_scale=None, v_scale=None,
                             q_max_seq_len=0, stream=None, mask="causal"):
    """Attention with K_rope given as rows laid out like K: k_rope [rows, 1, 64] of q's element
    type (float8_e4m3fn with k_rope_scale [1] float32), start positions cache_lengths [B]."""
    T, H, qd = q.shape
    _contiguous(output=output, q=q, k_nope=k_nope, v=v, k_rope=k_rope)
    _shapes(T, H, rows=[("output", output)])
    _kv(H, q.dtype, k_nope, v)
    if k_rope.dim() != 3 or tuple(k_rope.shape[1:]) != (1, 64) or _dtype_code(k_rope) != _dtype_code(q):
        raise ValueError(f"k_rope must be [rows, 1, 64] of q's element type, got {tuple(k_rope.shape)} {k_rope.dtype}")
    _check(_lib.mla_prefill_ragged_krope(_ptr(output), _dtype_code(output), _ptr(q), _dtype_code(q), _ptr(k_nope),
                                         _ptr(v), _ptr(k_rope), _f32(k_rope_scale, "k_rope_scale"),
                                         _idx(cache_lengths, "cache_lengths"), _idx(valid_length, "valid_length"),
                                         _idx(cache_row_offsets, "cache_row_offsets"),
                                         _idx(cache_offsets, "cache_offsets"), valid_length.shape[0] - 1, T, H, qd,
                                         k_nope.shape[2], _mask_code(mask), float(scale), _ptr(q_scale),
                                         _ptr(k_nope_scale), _ptr(v_scale), int(q_max_seq_len), _stream(stream)),
           "mla_prefill_ragged_krope")


def mla_prefill_ragged_row_krope(output, acc, acc_lse, q, k_nope, v, k_rope, cache_lengths, valid_length,
                                 cache_row_offsets, cache_offsets, scale, lse=None, k_rope_scale=None, q_scale=None,
                                 k_nope_scale=None, v_scale=None, q_max_seq_len=0, stream=None, mask="causal"):
    """mla_prefill_ragged_row with K_rope given as this row's rows laid out like K: k_rope
    [rows, 1, 64] of q's element type (float8_e4m3fn with k_rope_scale [1] float32)."""
    T, H, qd = q.shape
    _contiguous(output=output, lse=lse, acc=acc, acc_lse=acc_lse, q=q, k_nope=k_nope, v=v, k_rope=k_rope)
    _shapes(T, H, rows=[("output", output), ("acc", acc)], lses=[("lse", lse), ("acc_lse", acc_lse)])
    _kv(H, q.dtype, k_nope, v)
    if k_rope.dim() != 3 or tuple(k_rope.shape[1:]) != (1, 64) or _dtype_code(k_rope) != _dtype_code(q):
        raise ValueError(f"k_rope must be [rows, 1, 64] of q's element type, got {tuple(k_rope.shape)} {k_rope.dtype}")
    _check(_lib.mla_prefill_ragged_row_krope(_ptr(output), _dtype_code(output), _f32(lse, "lse"), _f32(acc, "acc"),
                                             _f32(acc_lse, "acc_lse"), _ptr(q), _dtype_code(q), _ptr(k_nope),
                                             _ptr(v), _ptr(k_rope), _f32(k_rope_scale, "k_rope_scale"),
                                             _idx(cache_lengths, "cache_lengths"), _idx(valid_length, "valid_length"),
                                             _idx(cache_row_offsets, "cache_row_offsets"),
                                             _idx(cache_offsets, "cache_offsets"), valid_length.shape[0] - 1, T, H,
                                             qd, k_nope.shape[2], _mask_code(mask), float(scale), _ptr(q_scale),
                                             _ptr(k_nope_scale), _ptr(v_scale), int(q_max_seq_len), _stream(stream)),
           "mla_prefill_ragged_row_krope")


def mla_prefill_latent_up(kv: PagedCache, layer_idx, buffer_row_offsets_r, cache_offsets_r, w_kv, k_nope, v,
                          latent_col=0, latent_dim=512, stream=None):
    """K_nope / V [cap, H, 128] of one plan row from the latent cache and w_kv [H*256, latent_dim] (bf16)."""
    cap, H, d = k_nope.shape
    _contiguous(w_kv=w_kv, k_nope=k_nope, v=v)
    if d != 128 or tuple(v.shape) != (cap, H, 128):
        raise ValueError("k_nope and v must be [cap, H, 128]")
    if tuple(w_kv.shape) != (H * 256, latent_dim) or w_kv.dtype != torch.bfloat16:
        raise ValueError(f"w_kv must be bf16 of shape {(H * 256, latent_dim)}")
    batch = cache_offsets_r.shape[0]
    s = kv.as_struct()
    _check(_lib.mla_prefill_latent_up(ctypes.byref(s), layer_idx, batch, _idx(buffer_row_offsets_r, "bro"),
                                      _idx(cache_offsets_r, "cache_offsets"), latent_col, latent_dim, _ptr(w_kv), H,
                                      cap, _ptr(k_nope), _ptr(v), _stream(stream)),
           "mla_prefill_latent_up")


def mla_prefill_merge(output, lse, o_a, lse_a, o_b, lse_b, stream=None):
    """Log-sum-exp combine of two partials: output [T, H, 128] (bf16 or fp32), lse [T, H] or None."""
    T, H, D = o_a.shape
    _contiguous(output=output, lse=lse, o_a=o_a, lse_a=lse_a, o_b=o_b, lse_b=lse_b)
    _shapes(T, H, rows=[("output", output), ("o_b", o_b)], lses=[("lse", lse), ("lse_a", lse_a), ("lse_b", lse_b)])
    _check(_lib.mla_prefill_merge(_ptr(output), _dtype_code(output), _f32(lse, "lse"), _f32(o_a, "o_a"),
                                  _f32(lse_a, "lse_a"), _f32(o_b, "o_b"), _f32(lse_b, "lse_b"), T, H, D,
                                  _stream(stream)), "mla_prefill_merge")
