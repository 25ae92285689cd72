"""The C-ABI library loads and exports every entry point its header declares (CPU only).

Only host-side validation paths are called here: each returns its error code
before any HIP call, so no GPU is needed.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_prefill.h")
LIB = os.path.join(ROOT, "mla_ragged_paged_amd", "libmla_prefill.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built: run python mla_ragged_paged_amd/build.py")
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    assert declared_functions() == ["mla_prefill_check", "mla_prefill_gather", "mla_prefill_kvsplit_workspace_bytes",
                                    "mla_prefill_last_hip_error", "mla_prefill_latent_up", "mla_prefill_merge",
                                    "mla_prefill_plan", "mla_prefill_ragged", "mla_prefill_ragged_krope",
                                    "mla_prefill_ragged_kvsplit", "mla_prefill_ragged_kvsplit_noalloc",
                                    "mla_prefill_ragged_lse", "mla_prefill_ragged_row", "mla_prefill_ragged_row_krope",
                                    "mla_prefill_ragged_split",
                                    "mla_prefill_set_debug", "mla_status_string"]


def test_binding_exposes_every_entry_point():
    import mla_ragged_paged_amd as m
    for name in declared_functions():
        assert callable(getattr(m, name)), name


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    lib.mla_status_string.restype = ctypes.c_char_p
    for code in range(8):
        assert lib.mla_status_string(code).decode().startswith("MLA_")
    assert lib.mla_status_string(99) == b"unknown mla_status_t"


def test_binding_validation_without_gpu():
    import mla_ragged_paged_amd as m
    # NULL pointers are rejected before anything is enqueued
    lib = m._binding._lib
    assert lib.mla_prefill_plan(None, 1, None, 0, 8, 1, None, None, None, None, None) == 1
    assert lib.mla_prefill_gather(None, 0, 1, None, None, 0, 1, 1, None, None) == 1
    assert m.mla_prefill_last_hip_error() == 0
    assert "NULL" in m.mla_status_string(1)


def test_validation_codes_without_gpu():
    import mla_ragged_paged_amd._binding as b
    lib = b._lib
    dummy = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    s = b._Cache(data=16, dtype=0, num_layers=1, num_pages=1, page_size=16, row_width=64, rope_col=0,
                 page_table=16, max_pages_per_seq=1, cache_lengths=16, scale=None)
    ref = ctypes.byref(s)
    # plan: zero capacity, zero rows, batch too large, layer out of range
    assert lib.mla_prefill_plan(dummy, 1, ref, 0, 0, 1, dummy, dummy, dummy, None, None) == 2
    assert lib.mla_prefill_plan(dummy, 1, ref, 0, 8, 0, dummy, dummy, dummy, None, None) == 2
    assert lib.mla_prefill_plan(dummy, 8193, ref, 0, 8, 1, dummy, dummy, dummy, None, None) == 2
    assert lib.mla_prefill_plan(dummy, 1, ref, 1, 8, 1, dummy, dummy, dummy, None, None) == 2
    # gather: column window beyond the row
    assert lib.mla_prefill_gather(ref, 0, 1, dummy, dummy, 60, 8, 4, dummy, None) == 2
    # attention: dims, mask, dtype combinations, fp8 without scales, bf16 with scales, bad rope window
    args = lambda **kw: [kw.get("out", dummy), kw.get("odt", 0), dummy, kw.get("qdt", 0), dummy, dummy, ref, 0,
                         dummy, dummy, None, 1, 4, 2, kw.get("qd", 192), kw.get("d", 128), kw.get("mask", 0),
                         ctypes.c_float(0.07), kw.get("qs"), None, None, 0, None]
    assert lib.mla_prefill_ragged(*args(qd=576)) == 4
    assert lib.mla_prefill_ragged(*args(d=512)) == 4
    assert lib.mla_prefill_ragged(*args(mask=2)) == 5
    assert lib.mla_prefill_ragged(*args(odt=1)) == 3
    assert lib.mla_prefill_ragged(*args(qdt=1)) == 3        # cache dtype bf16 != q dtype
    assert lib.mla_prefill_ragged(*args(qs=dummy)) == 3     # scales given for bf16
    assert lib.mla_prefill_ragged(*args(out=None)) == 1
    s.rope_col = 8
    assert lib.mla_prefill_ragged(*args()) == 2             # rope window past the row
    s.rope_col = 0
    s.dtype = 1
    fp8 = args(qdt=1)
    assert lib.mla_prefill_ragged(*fp8) == 1                # fp8 needs every scale
    s.dtype = 0


def test_lse_and_merge_validation_without_gpu():
    import mla_ragged_paged_amd._binding as b
    lib = b._lib
    dummy = ctypes.c_void_p(16)
    s = b._Cache(data=16, dtype=0, num_layers=1, num_pages=1, page_size=16, row_width=64, rope_col=0,
                 page_table=16, max_pages_per_seq=1, cache_lengths=16, scale=None)
    ref = ctypes.byref(s)

    def lse_args(**kw):
        return [dummy, kw.get("odt", 2), kw.get("lse", dummy), kw.get("po"), kw.get("pl"), dummy, 0, dummy, dummy,
                ref, 0, dummy, dummy, None, 1, 4, 2, 192, kw.get("d", 128), kw.get("mask", 1),
                ctypes.c_float(0.07), None, None, None, 0, None]
    assert lib.mla_prefill_ragged_lse(*lse_args(po=dummy)) == 1            # prev_output without prev_lse
    assert lib.mla_prefill_ragged_lse(*lse_args(pl=dummy)) == 1            # prev_lse without prev_output
    assert lib.mla_prefill_ragged_lse(*lse_args(odt=1)) == 3               # fp8 output
    assert lib.mla_prefill_ragged_lse(*lse_args(mask=7)) == 5
    assert lib.mla_prefill_ragged_lse(*lse_args(d=64)) == 4
    assert lib.mla_prefill_ragged_lse(*lse_args(po=dummy, pl=ctypes.c_void_p(18))) == 2   # misaligned lse
    assert lib.mla_prefill_ragged_lse(*lse_args(po=ctypes.c_void_p(24), pl=dummy)) == 2   # misaligned partial

    def row_args(**kw):
        return [dummy, 0, None, kw.get("acc", dummy), kw.get("acc_lse", dummy), dummy, 0, dummy, dummy, ref, 0,
                dummy, dummy, None, 1, 4, 2, 192, 128, 0, ctypes.c_float(0.07), None, None, None, 0, None]
    assert lib.mla_prefill_ragged_row(*row_args(acc=None)) == 1
    assert lib.mla_prefill_ragged_row(*row_args(acc_lse=None)) == 1
    assert lib.mla_prefill_ragged_row(*row_args(acc=ctypes.c_void_p(24))) == 2    # misaligned accumulator

    def split_args(**kw):
        return [dummy, 0, None, dummy, kw.get("qr", dummy), kw.get("dt", 0), kw.get("qs"), dummy, kw.get("ks"),
                dummy, kw.get("vs"), kw.get("rows", dummy), ref, 0, dummy, dummy, None, 1, 4, 2, kw.get("d", 128),
                0, ctypes.c_float(0.07), 0, None]
    assert lib.mla_prefill_ragged_split(*split_args(qr=None)) == 1            # q_rope missing
    assert lib.mla_prefill_ragged_split(*split_args(dt=1)) == 1               # fp8 without scales
    assert lib.mla_prefill_ragged_split(*split_args(qs=dummy)) == 3           # scales given for bf16
    assert lib.mla_prefill_ragged_split(*split_args(d=64)) == 4
    assert lib.mla_prefill_ragged_split(*split_args(rows=ctypes.c_void_p(24))) == 2   # misaligned rope rows
    s.dtype = 1
    assert lib.mla_prefill_ragged_split(*split_args(rows=None)) == 3          # bf16 q_nope with an e4m3 cache
    s.dtype = 0

    # key split: 4 tokens x 2 heads need 4 * 2 * (2 * 128 + 2) * 4 bytes of workspace
    lib.mla_prefill_kvsplit_workspace_bytes.restype = ctypes.c_uint64
    assert lib.mla_prefill_kvsplit_workspace_bytes(4, 2) == 8256
    assert lib.mla_prefill_kvsplit_workspace_bytes(0, 16) == 0

    def kvs_args(**kw):
        return [dummy, 0, None, dummy, 0, dummy, dummy, ref, 0, dummy, dummy, None, 1, 4, 2, kw.get("qd", 192), 128,
                0, ctypes.c_float(0.07), None, None, None, 0, kw.get("sk", 256), kw.get("ws", dummy),
                ctypes.c_uint64(kw.get("wb", 8256)), None]
    assert lib.mla_prefill_ragged_kvsplit(*kvs_args(ws=None)) == 1          # split without a workspace
    assert lib.mla_prefill_ragged_kvsplit(*kvs_args(sk=64)) == 2            # split_keys below 128
    assert lib.mla_prefill_ragged_kvsplit(*kvs_args(sk=1)) == 2
    assert lib.mla_prefill_ragged_kvsplit(*kvs_args(wb=8255)) == 2          # workspace one byte short
    assert lib.mla_prefill_ragged_kvsplit(*kvs_args(ws=ctypes.c_void_p(24))) == 2   # misaligned workspace
    assert lib.mla_prefill_ragged_kvsplit(*kvs_args(qd=128)) == 4           # split query is not offered

    def lat_args(**kw):
        return [ref, 0, kw.get("b", 1), dummy, dummy, kw.get("col", 0), kw.get("dim", 64), kw.get("w", dummy), 2,
                kw.get("cap", 4), dummy, dummy, None]
    assert lib.mla_prefill_latent_up(*lat_args(w=None)) == 1
    assert lib.mla_prefill_latent_up(*lat_args(dim=48)) == 2                # not a multiple of 64
    assert lib.mla_prefill_latent_up(*lat_args(col=8)) == 2                 # window past the 64-wide row
    assert lib.mla_prefill_latent_up(*lat_args(b=8193)) == 2
    assert lib.mla_prefill_latent_up(*lat_args(w=ctypes.c_void_p(24))) == 2
    assert lib.mla_prefill_latent_up(*lat_args(b=0)) == 0                   # empty batch: a no-op
    s.dtype = 1
    assert lib.mla_prefill_latent_up(*lat_args()) == 3                      # e4m3 cache
    s.dtype = 0

    def merge_args(**kw):
        return [kw.get("out", dummy), kw.get("odt", 0), kw.get("lse"), kw.get("oa", dummy), dummy, dummy,
                kw.get("lb", dummy), kw.get("t", 4), 2, kw.get("d", 128), None]
    assert lib.mla_prefill_merge(*merge_args(out=None)) == 1
    assert lib.mla_prefill_merge(*merge_args(lb=None)) == 1
    assert lib.mla_prefill_merge(*merge_args(d=64)) == 4
    assert lib.mla_prefill_merge(*merge_args(odt=1)) == 3
    assert lib.mla_prefill_merge(*merge_args(oa=ctypes.c_void_p(20))) == 2
    assert lib.mla_prefill_merge(*merge_args(lb=ctypes.c_void_p(18))) == 2
    assert lib.mla_prefill_merge(*merge_args(t=0)) == 0                    # empty: a no-op


def test_check_validation_and_debug_switch_without_gpu():
    import subprocess
    import sys
    import mla_ragged_paged_amd._binding as b
    lib = b._lib
    dummy = ctypes.c_void_p(16)
    s = b._Cache(data=16, dtype=0, num_layers=1, num_pages=1, page_size=16, row_width=64, rope_col=0,
                 page_table=16, max_pages_per_seq=1, cache_lengths=16, scale=None)
    ref = ctypes.byref(s)

    def chk(kv=ref, vl=dummy, batch=1, rows=None, viol=dummy):
        return lib.mla_prefill_check(kv, vl, batch, 4, 0, rows, None, 0, viol, None)
    assert chk(kv=None) == 1
    assert chk(viol=None) == 1
    assert chk(vl=None, rows=None) == 1                  # nothing to check
    assert chk(batch=8193) == 2
    assert chk(batch=0) == 0                             # empty batch: a no-op
    s.page_size = 0
    assert chk() == 2                                    # a page table without a page size
    s.page_size = 16
    s.cache_lengths = None
    assert chk() == 1
    # the debug switch returns the previous setting; the environment sets it at load
    prev = lib.mla_prefill_set_debug(1)
    assert lib.mla_prefill_set_debug(prev) == 1
    code = ("import ctypes; lib = ctypes.CDLL(%r); print(lib.mla_prefill_set_debug(0), lib.mla_prefill_set_debug(0))"
            % LIB)
    for env, want in (("1", "1 0"), ("0", "0 0"), ("", "0 0")):
        out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                             env={**os.environ, "MLA_PREFILL_DEBUG": env}).stdout.split()
        assert " ".join(out) == want, (env, out)


def test_package_fails_loudly_without_the_library(tmp_path):
    """The product path has no fallback: importing the package without its HIP
    library raises ImportError (a copy of the package sources, no library)."""
    import shutil
    import subprocess
    import sys
    src = os.path.join(ROOT, "mla_ragged_paged_amd")
    dst = tmp_path / "mla_ragged_paged_amd"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.so", "*.so.tmp", "__pycache__", "csrc"))
    assert not any(p.suffix == ".so" for p in dst.iterdir())
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n    import mla_ragged_paged_amd\nexcept ImportError as e:\n    print('ImportError:', e); sys.exit(3)\n"
            "sys.exit(0)\n") % str(tmp_path)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert res.returncode == 3, res.stdout + res.stderr
    assert "is missing" in res.stdout


def test_first_build_needs_no_library():
    """The build entry point loads the build script by path, so it does not import
    the package (which would load the library it is about to build)."""
    text = open(os.path.join(ROOT, "__graft_entry__.py")).read()
    build_src = text[text.index("def build()"):text.index("def smoke()")]
    assert "spec_from_file_location" in build_src
    assert "from mla_ragged_paged_amd import build" not in build_src


def test_launch_failure_reports_hip_error_without_gpu():
    """MLA_ERR_HIP and mla_prefill_last_hip_error(): with MLA_PREFILL_FAIL_LAUNCH set
    as the library loads, calls that pass their host-side checks return MLA_ERR_HIP
    carrying that HIP error code, and enqueue nothing (no GPU is touched)."""
    import subprocess
    import sys
    code = r'''
import ctypes, sys
sys.path.insert(0, %r)
import mla_ragged_paged_amd._binding as b
lib = b._lib
d = ctypes.c_void_p(256)
s = b._Cache(data=256, dtype=0, num_layers=1, num_pages=4, page_size=16, row_width=64, rope_col=0,
             page_table=256, max_pages_per_seq=4, cache_lengths=256, scale=None)
r = ctypes.byref(s)
out = []
out.append(lib.mla_prefill_last_hip_error())
out.append(lib.mla_prefill_plan(d, 1, r, 0, 64, 1, d, d, d, None, None))
out.append(lib.mla_prefill_last_hip_error())
out.append(lib.mla_prefill_gather(r, 0, 1, d, d, 0, 64, 64, d, None))
out.append(lib.mla_prefill_ragged(d, 0, d, 0, d, d, r, 0, d, d, None, 1, 4, 2, 192, 128, 0,
                                  ctypes.c_float(0.07), None, None, None, 0, None))
out.append(lib.mla_prefill_merge(d, 0, None, d, d, d, d, 4, 2, 128, None))
out.append(lib.mla_prefill_plan(None, 1, r, 0, 64, 1, d, d, d, None, None))   # host check still first
print(" ".join(map(str, out)))
''' % ROOT
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                         env={**os.environ, "MLA_PREFILL_FAIL_LAUNCH": "98", "MLA_PREFILL_DEBUG": "0"})
    assert res.returncode == 0, res.stderr
    assert res.stdout.split() == ["0", "6", "98", "6", "6", "6", "1"], res.stdout


def test_binding_rejects_mismatched_k_nope_and_v():
    """K_nope / V with other heads than q, other widths, or another element type
    than q are rejected in the binding before the library is called."""
    import torch
    import mla_ragged_paged_amd as m
    T, H = 4, 2
    q = torch.zeros((T, H, 192), dtype=torch.bfloat16)
    out = torch.zeros((T, H, 128), dtype=torch.bfloat16)
    ok = torch.zeros((8, H, 128), dtype=torch.bfloat16)
    bad = {"fewer heads": torch.zeros((8, 1, 128), dtype=torch.bfloat16),
           "other width": torch.zeros((8, H, 64), dtype=torch.bfloat16),
           "other dtype": torch.zeros((8, H, 128), dtype=torch.float8_e4m3fn),
           "other rows": torch.zeros((9, H, 128), dtype=torch.bfloat16)}
    kv = m.PagedCache(torch.zeros((1, 1, 16, 1, 64), dtype=torch.bfloat16), torch.zeros((1, 1), dtype=torch.int32),
                      torch.zeros((1,), dtype=torch.int32), 0)
    idx = torch.zeros((2,), dtype=torch.int32)
    for label, t in bad.items():
        for kn, v in ((t, ok), (ok, t)):
            if label == "other rows" and kn is ok:
                continue
            with pytest.raises((ValueError, TypeError)):
                m.mla_prefill_ragged(out, q, kn, v, kv, 0, idx, idx, None, 0.1)
            with pytest.raises((ValueError, TypeError)):
                m.mla_prefill_ragged_lse(out.float(), None, q, kn, v, kv, 0, idx, idx, None, 0.1)
            with pytest.raises((ValueError, TypeError)):
                m.mla_prefill_ragged_row(out, out.float(), torch.zeros((T, H)), q, kn, v, kv, 0, idx, idx, None, 0.1)
            with pytest.raises((ValueError, TypeError)):
                m.mla_prefill_ragged_kvsplit(out, q, kn, v, kv, 0, idx, idx, None, 0.1, 0, None)
            with pytest.raises((ValueError, TypeError)):
                m.mla_prefill_ragged_split(out, q[..., :128].contiguous(), q[..., 128:].contiguous(), kn, v, kv, 0,
                                           idx, idx, None, 0.1)


def test_krope_validation_without_gpu():
    """mla_prefill_ragged_krope: host-side checks return their codes before anything is enqueued."""
    import mla_ragged_paged_amd._binding as b
    lib = b._lib
    d = ctypes.c_void_p(256)

    def args(**kw):
        return [kw.get("out", d), kw.get("odt", 0), d, kw.get("qdt", 0), d, d, kw.get("rows", d), kw.get("rs"),
                kw.get("cl", d), d, d, None, kw.get("b", 1), 4, 2, kw.get("qd", 192), 128, kw.get("mask", 0),
                ctypes.c_float(0.07), kw.get("qs"), kw.get("qs"), kw.get("qs"), 0, None]
    assert lib.mla_prefill_ragged_krope(*args(rows=None)) == 1                # no K_rope rows
    assert lib.mla_prefill_ragged_krope(*args(cl=None)) == 1                  # no start positions
    assert lib.mla_prefill_ragged_krope(*args(rs=d)) == 3                     # a rows scale for bf16
    assert lib.mla_prefill_ragged_krope(*args(qdt=1, qs=d)) == 1              # e4m3 rows without their scale
    assert lib.mla_prefill_ragged_krope(*args(qdt=2)) == 3                    # fp32 inputs
    assert lib.mla_prefill_ragged_krope(*args(qd=128)) == 4
    assert lib.mla_prefill_ragged_krope(*args(mask=3)) == 5
    assert lib.mla_prefill_ragged_krope(*args(rows=ctypes.c_void_p(264))) == 2   # rows not 16-byte aligned
    assert lib.mla_prefill_ragged_krope(*args(out=None)) == 1
    assert lib.mla_prefill_ragged_krope(*args(b=0)) == 0                      # empty batch: a no-op


def test_row_krope_validation_without_gpu():
    """mla_prefill_ragged_row_krope: the row call's and the contiguous rows' host-side checks
    return their codes before anything is enqueued."""
    import mla_ragged_paged_amd._binding as b
    lib = b._lib
    d = ctypes.c_void_p(256)

    def args(**kw):
        return [kw.get("out", d), 0, None, kw.get("acc", d), kw.get("acc_lse", d), d, kw.get("qdt", 0), d, d,
                kw.get("rows", d), kw.get("rs"), kw.get("cl", d), d, d, None, kw.get("b", 1), 4, 2, 192, 128,
                kw.get("mask", 0), ctypes.c_float(0.07), kw.get("qs"), kw.get("qs"), kw.get("qs"), 0, None]
    assert lib.mla_prefill_ragged_row_krope(*args(acc=None)) == 1            # row mode needs the accumulator
    assert lib.mla_prefill_ragged_row_krope(*args(acc_lse=None)) == 1
    assert lib.mla_prefill_ragged_row_krope(*args(rows=None)) == 1           # no K_rope rows
    assert lib.mla_prefill_ragged_row_krope(*args(cl=None)) == 1             # no start positions
    assert lib.mla_prefill_ragged_row_krope(*args(rs=d)) == 3                # a rows scale for bf16
    assert lib.mla_prefill_ragged_row_krope(*args(qdt=1, qs=d)) == 1         # e4m3 rows without their scale
    assert lib.mla_prefill_ragged_row_krope(*args(mask=3)) == 5
    assert lib.mla_prefill_ragged_row_krope(*args(acc=ctypes.c_void_p(264))) == 2   # acc not 16-byte aligned
    assert lib.mla_prefill_ragged_row_krope(*args(b=0)) == 0                 # empty batch: a no-op


def test_kvsplit_noalloc_validation_without_gpu():
    """mla_prefill_ragged_kvsplit_noalloc: size and argument checks return before any HIP call."""
    import mla_ragged_paged_amd._binding as b
    lib = b._lib
    d = ctypes.c_void_p(256)
    s = b._Cache(data=256, dtype=0, num_layers=1, num_pages=1, page_size=16, row_width=64, rope_col=0,
                 page_table=256, max_pages_per_seq=1, cache_lengths=256, scale=None)
    ref = ctypes.byref(s)

    def args(**kw):
        return [kw.get("out", d), 0, None, d, 0, d, d, ref, 0, d, d, None, kw.get("b", 1), kw.get("t", 4),
                kw.get("h", 2), 192, 128, 0, ctypes.c_float(0.07), None, None, None, 0, kw.get("sk", 256), None]
    assert lib.mla_prefill_ragged_kvsplit_noalloc(*args(t=16257, h=4)) == 2      # partials past 64 MiB
    assert lib.mla_prefill_ragged_kvsplit_noalloc(*args(sk=64)) == 2              # split_keys below 128
    assert lib.mla_prefill_ragged_kvsplit_noalloc(*args(out=None, sk=0)) == 1
    assert lib.mla_prefill_ragged_kvsplit_noalloc(*args(b=0)) == 0                # empty batch: a no-op
