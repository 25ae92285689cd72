"""Parity oracle for ragged, masked (causal or null) MLA prefill over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test-suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP path (``mla_ragged_paged_amd``) and imports
nothing from it.

Everything here is a plain, slow, float64 numpy statement of what the three
Modular MAX API pages define:

* ``generic_flare_mla_prefill_ragged_paged_plan`` (plan outputs),
* ``flare_mla_prefill`` (the attention itself),
* ``mla_prefill_v2_ragged`` (argument semantics of the AMD launcher).
"""
from .mla_oracle import (  # noqa: F401
    E4M3FN_MAX,
    decode_e4m3fn,
    dequantize_e4m3fn,
    plan,
    gather,
    rope_rows,
    mla_prefill_ragged,
    mla_prefill_rows,
    mla_prefill_ragged_split,
    mla_prefill_rows_split,
    latent_up,
    merge_partials,
    MASKS,
)
