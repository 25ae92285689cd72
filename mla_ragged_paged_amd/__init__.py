"""MI355X-native ragged paged MLA prefill.

The compute path is the HIP library ``libmla_prefill.so`` (built from ``csrc/``
for gfx950).  This package is a thin binding over its C ABI: the functions below
have the same names as the C entry points and only marshal torch tensors into
pointers and sizes.  Importing the package fails loudly when the library has not
been built; there is no fallback.
"""
from ._binding import (  # noqa: F401
    MLA_BF16,
    MLA_ERR_PRECONDITION,
    MLA_FP8_E4M3FN,
    MLA_FP32,
    MLA_MASK_CAUSAL,
    MLA_MASK_NULL,
    MLA_MAX_BATCH,
    MLA_VIOLATION_PAGE_IDS,
    MLA_VIOLATION_POSITIONS,
    MLA_VIOLATION_Q_OFFSETS,
    MLA_VIOLATION_ROW_OFFSETS,
    MlaError,
    PagedCache,
    library_path,
    mla_prefill_check,
    mla_prefill_gather,
    mla_prefill_kvsplit_workspace_bytes,
    mla_prefill_last_hip_error,
    mla_prefill_plan,
    mla_prefill_latent_up,
    mla_prefill_merge,
    mla_prefill_ragged,
    mla_prefill_ragged_krope,
    mla_prefill_ragged_kvsplit,
    mla_prefill_ragged_kvsplit_noalloc,
    mla_prefill_ragged_lse,
    mla_prefill_ragged_row,
    mla_prefill_ragged_row_krope,
    mla_prefill_ragged_split,
    mla_prefill_set_debug,
    mla_status_string,
)
