"""Compile the HIP sources of the library into ``libmla_prefill.so`` (gfx950 only).

Run as ``python mla_ragged_paged_amd/build.py`` (by path: importing the package
loads the library, which a first build does not have yet).  hipcc cross-compiles, so no GPU is
needed.  Packed fp32 VALU instructions are disabled for every kernel.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla_prefill.so")
SOURCES = ["api.hip", "plan_gather.hip", "prefill_bf16.hip", "prefill_fp8.hip", "merge.hip", "latent_up.hip", "check.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile each source to an object in parallel, then link the shared library."""
    import concurrent.futures
    import tempfile

    objdir = tempfile.mkdtemp(prefix="mla_build_")
    compile_flags = [f for f in FLAGS if f != "-shared"]

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *compile_flags, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        return src, cmd, obj, res

    workers = max(1, min(len(SOURCES), os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(compile_one, SOURCES))
    objs = []
    for src, cmd, obj, res in results:
        out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
        if verbose:
            print(" ".join(cmd), flush=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src} ({res.returncode}):\n{out}")
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    os.rmdir(objdir)
    return LIB
