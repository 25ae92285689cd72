"""Benchmark of one ragged paged MLA prefill step on one MI355X.

A step is the whole hot path over one batch of synthetic, device-resident
input: plan -> gather (each cache row's K_rope window into contiguous rows laid
out like K_nope / V) -> causal MLA attention reading those rows.  Prints one
JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3|prefix|long|fp8|tiny]
                  [--no-cpu-baseline] [--cpu-seconds S]

value    = causal FLOPs of the step / measured step time (TFLOP/s).
roofline = the attention kernel (the dominant one): algorithmic FLOPs per launch
           over its average launch time from HIP events on its launch stream,
           against the MI355X dense MFMA peak of the compute dtype.
cpu_baseline = the float64 oracle timed on the host on a bounded sample of the
           same workload (a subset of heads), scaled to TFLOP/s.
configs  = each H=128 workload (dsv3, prefix, long, fp8): its attention launch
           timed alone (mean / median / min), TFLOP/s, fraction of its own
           dtype's MFMA peak, HBM traffic over algorithmic bytes, and its own
           bounded oracle sample.
Also reported: the attention time (mean, median, min over the timed steps, from
the two events around each attention launch, the only events in the timed
loop), plan / gather times (from events around them in a second run of the same
steps after the timed one), the attention time with L2 and MALL flushed by a 512 MiB write before
each launch (cold_cache), and the gather kernel's bandwidth on a >= 1 GiB
paged cache of 576-wide bf16 rows (gather_bench).
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}      # MI355X dense MFMA peaks
HBM_PEAK_GBS = 8000.0


def _code_only(text: str) -> str:
    """Source text without comments, trailing blanks and empty lines (the kernel sources
    hold no comment markers inside string literals)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(dtype: str = "bf16") -> str:
    """Hash of the code of the attention kernel sources of one dtype (its .hip file and the
    shared headers, comments left out): a committed traffic summary is used only when it
    was taken on this code."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mla_ragged_paged_amd", "csrc")
    for name in sorted([f"prefill_{dtype}.hip", "device_common.h", "kernels.h"]):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update((name + _code_only(f.read())).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, kernel_hash: str):
    """HBM bytes per attention launch from a committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"prefill_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, budget_s: float):
    """The oracle on the host over heads 0..k-1 of the same workload until ~budget_s of work."""
    import numpy as np

    import oracle
    from mla_ragged_paged_amd import workloads
    blas = []
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([int(i.get("num_threads", 1)) for i in info] + [1])
        blas = [f"{i.get('internal_api', '?')}:{i.get('num_threads', '?')}" for i in info]
    except Exception:  # pragma: no cover
        threads = 1
    q, kn, v = w.q, w.k_nope, w.v
    bro = np.concatenate([[0], np.cumsum(w.n + w.p)]).astype(np.uint32)
    co = np.zeros(w.batch, dtype=np.uint32)
    t0 = time.perf_counter()
    heads = 0
    while heads < w.heads and time.perf_counter() - t0 < budget_s:
        h = heads
        oracle.mla_prefill_ragged(q[:, h:h + 1], kn[:, h:h + 1], v[:, h:h + 1], w.cache, w.spec.layer_idx,
                                  w.page_table, w.spec.page_size, w.spec.rope_col, w.cache_lengths,
                                  w.input_row_offsets, bro, co, w.softmax_scale, scales=w.scales)
        heads += 1
    dt = time.perf_counter() - t0
    flops = workloads.causal_flops(w.n, w.p, heads)
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 numpy oracle, heads 0..{heads - 1} of {w.heads} (all {w.batch} sequences), "
                      f"{dt:.1f} s wall on the host, {threads} BLAS threads; elementwise softmax single-threaded",
            "cpu_count": os.cpu_count(), "affinity_cpus": affinity, "blas": blas}


def config_bench(torch, name, reps=20, warmup=5, cpu_seconds=6.0):
    """One H=128 workload's attention launch, timed alone on its launch stream after
    `warmup` launches: mean / median / min over `reps` HIP-event intervals, TFLOP/s
    and the fraction of its own dtype's dense MFMA peak, the HBM traffic of its
    committed counter summary (when taken on the current kernel sources) over the
    algorithmic bytes, and the oracle timed on a bounded sample of it (None when
    cpu_seconds is 0)."""
    from mla_ragged_paged_amd import workloads
    from mla_ragged_paged_amd.pipeline import PrefillStep
    w = workloads.build(workloads.SPECS[name])
    flops = workloads.causal_flops(w.n, w.p, w.heads)
    step = PrefillStep(w, "cuda:0")
    stream = torch.cuda.current_stream()
    step.run()
    for _ in range(warmup):
        step.attention(0)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        step.attention(0)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    mean = sum(ms) / len(ms)
    med = ms[len(ms) // 2]
    peak = PEAK_TFLOPS[w.spec.dtype]
    alg = workloads.algorithmic_bytes(w)
    traffic = traffic_from_profiles(name, kernel_source_hash(w.spec.dtype))
    out = {"workload": f"{name}: {w.spec.description}", "dtype": w.spec.dtype, "batch": w.batch,
           "new_tokens": w.total_q, "context_tokens": w.total_ctx, "causal_tflop": round(flops / 1e12, 5),
           "attention_mean_ms": round(mean, 4), "attention_median_ms": round(med, 4),
           "attention_min_ms": round(ms[0], 4), "TFLOPs_mean": round(flops / (mean * 1e-3) / 1e12, 2),
           "TFLOPs_median": round(flops / (med * 1e-3) / 1e12, 2), "peak_TFLOPs": peak,
           "frac_mean": round(flops / (mean * 1e-3) / 1e12 / peak, 4),
           "frac_median": round(flops / (med * 1e-3) / 1e12 / peak, 4),
           "algorithmic_bytes": alg, "traffic_bytes": traffic,
           "traffic_over_algorithmic": None if traffic is None else round(traffic / alg, 3),
           "reps": reps, "warmup": warmup}
    del step
    if cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(w, cpu_seconds)
    del w
    torch.cuda.empty_cache()
    return out


def gather_bench(torch, batch=64, n_range=(8192, 24576), width=576, page_size=128, seed=11, reps=5):
    """Bandwidth of the gather kernel on a large paged cache (>= 1 GiB of 576-wide bf16
    rows, shuffled physical pages): median over `reps` launches, bytes read + written."""
    import numpy as np

    from mla_ragged_paged_amd import _binding as B
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(seed)
    L = rng.integers(n_range[0], n_range[1] + 1, size=batch)
    pages = (L + page_size - 1) // page_size
    num_pages = int(pages.sum())
    perm = rng.permutation(num_pages)
    table = np.zeros((batch, int(pages.max())), dtype=np.int64)
    k = 0
    for b in range(batch):
        table[b, :pages[b]] = perm[k:k + pages[b]]
        k += int(pages[b])
    C = int(L.sum())
    gen = torch.Generator(device=dev).manual_seed(seed)
    cache = torch.randn((1, num_pages, page_size, 1, width), generator=gen, device=dev).to(torch.bfloat16)
    page_table = torch.from_numpy(table).to(torch.int32).to(dev)
    zeros = torch.zeros(batch, dtype=torch.int32, device=dev)
    iro = torch.from_numpy(np.concatenate([[0], np.cumsum(L)])).to(torch.int32).to(dev)
    kv = B.PagedCache(cache, page_table, zeros, width - 64)
    bro = torch.zeros(batch + 1, dtype=torch.int32, device=dev)
    co = torch.zeros(batch, dtype=torch.int32, device=dev)
    bl = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty((C, width), dtype=torch.bfloat16, device=dev)
    B.mla_prefill_plan(iro, kv, 0, C, bro.view(1, -1), co.view(1, -1), bl, None, None)
    for _ in range(2):
        B.mla_prefill_gather(kv, 0, bro, co, 0, width, out, None)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        B.mla_prefill_gather(kv, 0, bro, co, 0, width, out, None)
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    # spot check: sampled rows equal the cache rows the page table names (exact copy)
    rows = torch.from_numpy(rng.integers(0, C, size=256)).to(dev)
    starts = torch.from_numpy(np.concatenate([[0], np.cumsum(L)[:-1]])).to(dev)
    b_of = torch.searchsorted(starts, rows, right=True) - 1
    pos = rows - starts[b_of]
    ref = cache[0, page_table[b_of, pos // page_size].long(), pos % page_size, 0, :]
    exact = bool(torch.equal(ref, out[rows]))
    moved = 2.0 * C * width * 2
    med = ms[len(ms) // 2]
    return {"tokens": C, "row_bytes": width * 2, "page_size": page_size, "bytes_moved": moved,
            "median_ms": round(med, 4), "min_ms": round(ms[0], 4), "GBps": round(moved / (med * 1e-3) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * moved / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 1), "sample_rows_exact": exact}


def _median_ms(torch, fn, reps, stream):
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return ms[len(ms) // 2], ms[0]


def _alternating_median_ms(torch, fns, reps, stream):
    """Median launch time of each of `fns`, timed in alternation (fn0, fn1, fn0, ...) so
    that all of them see the same clock state of the chip."""
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(reps)]
    for row in ev:
        for fn, (e0, e1) in zip(fns, row):
            e0.record(stream)
            fn()
            e1.record(stream)
    torch.cuda.synchronize()
    out = []
    for i in range(len(fns)):
        ms = sorted(row[i][0].elapsed_time(row[i][1]) for row in ev)
        out.append(ms[len(ms) // 2])
    return out


def next_rows_bench(torch, w, reps=9):
    """The paths beside the headline step, on the same workload:
    the null mask (every key visible), the context cut into three buffer rows
    whose partials merge in the attention epilogue, the split-query calls (also
    on the fp8 workload), the latent decompression (and the step that uses it
    instead of the gather), and the standalone merge kernel's bandwidth on fp32
    partials."""
    from mla_ragged_paged_amd import _binding as B
    from mla_ragged_paged_amd import workloads
    from mla_ragged_paged_amd.pipeline import PrefillStep, balanced_split_keys
    stream = torch.cuda.current_stream()
    peak = PEAK_TFLOPS[w.spec.dtype]
    out = {}

    nm = PrefillStep(w, "cuda:0", mask="null")
    nm.run()
    med, best = _median_ms(torch, lambda: nm.attention(0), reps, stream)
    fl = workloads.null_mask_flops(w.n, w.p, w.heads)
    out["null_mask"] = {"attention_median_ms": round(med, 4), "attention_min_ms": round(best, 4),
                        "tflop": round(fl / 1e12, 5), "achieved_TFLOPs": round(fl / (med * 1e-3) / 1e12, 2),
                        "frac_of_peak": round(fl / (med * 1e-3) / 1e12 / peak, 4)}
    del nm

    cap = -(-w.total_ctx // 3)
    mr = PrefillStep(w, "cuda:0", cap=cap)
    mr.run()
    step_med, _ = _median_ms(torch, mr.run, reps, stream)

    def rows_attention():
        # attention launches only: the gathered K_rope rows then hold the last row's
        # window for every row, which changes no work (the step time above is whole)
        for r in range(mr.rows):
            mr.attention_row_merged(r)
    attn_med, attn_best = _median_ms(torch, rows_attention, reps, stream)
    # the ratio to one row is taken against one-row launches timed in alternation
    # with the rows (the same clock state; the headline is timed minutes earlier)
    one = PrefillStep(w, "cuda:0")
    one.run()
    alt_rows, alt_one = _alternating_median_ms(torch, [rows_attention, lambda: one.attention(0)], reps, stream)
    del one
    fl = workloads.causal_flops(w.n, w.p, w.heads)
    out["rows_merged"] = {"cap": cap, "rows": mr.rows, "step_median_ms": round(step_med, 4),
                          "attention_median_ms": round(attn_med, 4), "attention_min_ms": round(attn_best, 4),
                          "achieved_TFLOPs": round(fl / (attn_med * 1e-3) / 1e12, 2),
                          "frac_of_peak": round(fl / (attn_med * 1e-3) / 1e12 / peak, 4),
                          "attention_time_vs_one_row": round(alt_rows / alt_one, 3),
                          "alternating_ms": {"rows": round(alt_rows, 4), "one_row": round(alt_one, 4)}}
    del mr

    # split query: bf16 on this workload (contiguous K_rope rows), and the fp8
    # workload's e4m3 q_nope / K / V with a bf16 q_rope, K_rope from its e4m3 cache
    # and from contiguous bf16 rows
    out["split_q"] = {}
    for wl in ([w] + ([workloads.build(workloads.SPECS["fp8"])] if w.spec.dtype == "bf16" else [])):
        st = PrefillStep(wl, "cuda:0")
        st.plan()
        q_nope, q_rope = workloads.split_query(wl)
        q_nope, q_rope = q_nope.to("cuda:0"), q_rope.to("cuda:0")
        rows = workloads.draw_rope_rows(wl.total_ctx, seed=wl.spec.seed).to("cuda:0")
        o = torch.empty((wl.total_q, wl.heads, 128), dtype=torch.bfloat16, device="cuda:0")
        sc = st.scales or {}
        fl = workloads.causal_flops(wl.n, wl.p, wl.heads)
        pk = PEAK_TFLOPS[wl.spec.dtype]
        for rope in (["paged", "contiguous"] if wl.spec.dtype == "fp8" else ["contiguous"]):
            def call():
                B.mla_prefill_ragged_split(o, q_nope, q_rope, st.k_nope, st.v, st.kv, 0, st.input_row_offsets,
                                           st.buffer_row_offsets[0], st.cache_offsets[0], wl.softmax_scale,
                                           q_scale=sc.get("q"), k_scales=sc.get("k_nope"), v_scale=sc.get("v"),
                                           k_rope_rows=rows if rope == "contiguous" else None,
                                           q_max_seq_len=wl.max_q)
            call()
            med, best = _median_ms(torch, call, reps, stream)
            out["split_q"][f"{wl.spec.name}_{rope}_rope"] = {
                "dtype": wl.spec.dtype, "attention_median_ms": round(med, 4), "attention_min_ms": round(best, 4),
                "achieved_TFLOPs": round(fl / (med * 1e-3) / 1e12, 2),
                "frac_of_peak": round(fl / (med * 1e-3) / 1e12 / pk, 4)}
        del st

    # latent decompression (K_nope / V from the latent cache, synthetic weights)
    # and the step that uses it in place of the gather
    if w.spec.dtype == "bf16":
        Wkv = workloads.draw_kv_b_weight(w.heads, 512, seed=w.spec.seed)
        ls = PrefillStep(w, "cuda:0", kv_b_weight=Wkv)
        ls.run()
        med_up, best_up = _median_ms(torch, lambda: ls.latent_up(0), reps, stream)
        med_step, _ = _median_ms(torch, ls.run, reps, stream)
        fl_up = 2.0 * w.total_ctx * 512 * w.heads * 256
        out["latent_up"] = {"slots": w.total_ctx, "latent_dim": 512, "heads": w.heads, "tflop": round(fl_up / 1e12, 5),
                            "median_ms": round(med_up, 4), "min_ms": round(best_up, 4),
                            "achieved_TFLOPs": round(fl_up / (med_up * 1e-3) / 1e12, 2),
                            "frac_of_peak": round(fl_up / (med_up * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4),
                            "latent_step_median_ms": round(med_step, 4)}
        del ls

    # one GPU's share of the same batch under 8-way head parallelism: 16 heads,
    # the same sequence lengths (the work-unit count, not the arithmetic, changes)
    import dataclasses
    share = workloads.build(dataclasses.replace(w.spec, name=w.spec.name + "_h16", heads=w.heads // 8))
    ss = PrefillStep(share, "cuda:0")
    ss.run()
    med, best = _median_ms(torch, lambda: ss.attention(0), reps, stream)
    fl = workloads.causal_flops(share.n, share.p, share.heads)
    out["tp8_share"] = {"heads": share.heads, "tflop": round(fl / 1e12, 5), "attention_median_ms": round(med, 4),
                        "attention_min_ms": round(best, 4), "achieved_TFLOPs": round(fl / (med * 1e-3) / 1e12, 2),
                        "frac_of_peak": round(fl / (med * 1e-3) / 1e12 / peak, 4),
                        "split_keys": balanced_split_keys(share.n, share.p, share.heads)}
    del ss

    # 8 heads (16-way head parallelism): fewer query tiles than workgroup slots, where
    # the key split (mla_prefill_ragged_kvsplit, attention + merge pass) is chosen
    share8 = workloads.build(dataclasses.replace(w.spec, name=w.spec.name + "_h8", heads=w.heads // 16))
    sk8 = balanced_split_keys(share8.n, share8.p, share8.heads)
    fl8 = workloads.causal_flops(share8.n, share8.p, share8.heads)
    row = {"heads": share8.heads, "tflop": round(fl8 / 1e12, 5), "split_keys": sk8}
    for label, sk in (("plain", 0), ("kvsplit", sk8)):
        st8 = PrefillStep(share8, "cuda:0", split_keys=sk)
        st8.run()
        med, _ = _median_ms(torch, lambda: st8.attention(0), reps, stream)
        row[f"{label}_median_ms"] = round(med, 4)
        row[f"{label}_TFLOPs"] = round(fl8 / (med * 1e-3) / 1e12, 2)
        del st8
    out["tp16_share"] = row

    # the whole step captured as a HIP graph and replayed, against eager launches
    # (timed in alternation: back-to-back launches run at a clock that drifts)
    from mla_ragged_paged_amd.pipeline import CapturedStep
    out["graph_step"] = {}
    for wl in (w, workloads.build(workloads.SPECS["tiny"])):
        gs = PrefillStep(wl, "cuda:0")
        cs = CapturedStep(gs)
        med_e, med_g = _alternating_median_ms(torch, [gs.run, cs.replay], reps, stream)
        out["graph_step"][wl.spec.name] = {"eager_median_ms": round(med_e, 4), "graph_median_ms": round(med_g, 4)}
        del cs, gs

    T, H = 16384, 128
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(12)
    o_a = torch.randn((T, H, 128), generator=gen, device=dev)
    o_b = torch.randn((T, H, 128), generator=gen, device=dev)
    l_a = torch.randn((T, H), generator=gen, device=dev)
    l_b = torch.randn((T, H), generator=gen, device=dev)
    o = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    B.mla_prefill_merge(o, None, o_a, l_a, o_b, l_b)
    med, best = _median_ms(torch, lambda: B.mla_prefill_merge(o, None, o_a, l_a, o_b, l_b), reps, stream)
    moved = T * H * (2 * 128 * 4 + 2 * 4 + 128 * 2)
    out["merge_kernel"] = {"tokens": T, "heads": H, "output": "bf16", "bytes_moved": moved,
                           "median_ms": round(med, 4), "GBps": round(moved / (med * 1e-3) / 1e9, 1),
                           "pct_of_hbm_peak": round(100 * moved / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload attention timings")
    ap.add_argument("--config-cpu-seconds", type=float, default=6.0,
                    help="oracle time budget per workload in the per-workload section")
    ap.add_argument("--no-extras", action="store_true", help="skip the cold-cache, gather-bandwidth, null-mask, buffer-row and merge measurements")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (scales HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not offered (the prefill path has no "
              "cross-GPU step; run with --gpus 1)", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return

    from mla_ragged_paged_amd import workloads
    from mla_ragged_paged_amd.pipeline import PrefillStep

    spec = workloads.SPECS[args.workload]
    w = workloads.build(spec)
    flops = workloads.causal_flops(w.n, w.p, w.heads)
    step = PrefillStep(w, "cuda:0")
    torch.cuda.synchronize()
    print(f"[bench] {spec.name}: B={w.batch} n={w.n.tolist()} p={w.p.tolist()} T={w.total_q} C={w.total_ctx} "
          f"H={w.heads} causal TFLOP={flops / 1e12:.4f}", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    # The timed steps carry two HIP events each, around the attention launch (its
    # duration gives the roofline figure); every further event pair in the loop
    # would add a few microseconds of its own to the measured step.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step.plan()
        step.gather(0)
        ev[k][0].record(stream)
        step.attention(0)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    attn_all = sorted(e[0].elapsed_time(e[1]) for e in ev)
    attn_ms = sum(attn_all) / args.steps
    attn_best = attn_all[0]
    attn_median = attn_all[len(attn_all) // 2]
    # plan and gather times: the same launches, bracketed by events, after the timed steps
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps):
        e = sev[k]
        e[0].record(stream)
        step.plan()
        e[1].record(stream)
        step.gather(0)
        e[2].record(stream)
        step.attention(0)
    torch.cuda.synchronize()
    plan_ms = sum(e[0].elapsed_time(e[1]) for e in sev) / args.steps
    gather_ms = sum(e[1].elapsed_time(e[2]) for e in sev) / args.steps

    dtype = spec.dtype
    achieved = flops / (attn_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    khash = kernel_source_hash(dtype)
    traffic = traffic_from_profiles(spec.name, khash)
    el = 1 if dtype == "fp8" else 2
    gather_bytes = 2.0 * w.total_ctx * step.gather_cols[1] * el      # read + write of the gathered window
    result = {
        "metric": "MLA prefill TFLOP/s (causal, H=128, bf16/fp8) and % of MFMA peak, 1 GPU",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"{spec.name}: {spec.description}", "batch": w.batch, "heads": w.heads,
                   "new_tokens": w.total_q, "context_tokens": w.total_ctx, "page_size": spec.page_size,
                   "q_depth": 192, "depth": 128, "rope": 64, "seed": spec.seed},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic},
        "stages_ms": {"plan": round(plan_ms, 4), "gather": round(gather_ms, 4), "attention": round(attn_ms, 4),
                      "attention_median": round(attn_median, 4), "attention_best": round(attn_best, 4)},
        "pct_of_bf16_peak": round(100 * flops / (ms_step * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 2),
        "gather_GBps": round(gather_bytes / (gather_ms * 1e-3) / 1e9, 1),
        "causal_tflop_per_step": round(flops / 1e12, 5),
        "kernel_source_hash": khash,
    }
    if dtype == "fp8":
        result["pct_of_fp8_peak"] = round(100 * flops / (ms_step * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 2)
    def guarded(name, fn):
        """A side measurement; its failure is reported in the line instead of losing the line."""
        try:
            result[name] = fn()
        except Exception as e:  # noqa: BLE001 -- any failure of a side measurement
            result[name] = {"error": f"{type(e).__name__}: {e}"}
            print(f"[bench] {name} failed: {e!r}", file=sys.stderr, flush=True)

    def cold_cache():
        # attention with L2 and MALL flushed by a 512 MiB write before each launch
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
        cold = []
        for _ in range(7):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step.attention(0)
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del flush
        cold.sort()
        return {"flush_mib": 512, "attention_median_ms": round(cold[len(cold) // 2], 4),
                "attention_min_ms": round(cold[0], 4),
                "achieved_TFLOPs_median": round(flops / (cold[len(cold) // 2] * 1e-3) / 1e12, 2)}

    if not args.no_extras:
        guarded("cold_cache", cold_cache)
        print("[bench] gather bandwidth on a >= 1 GiB paged cache", file=sys.stderr, flush=True)
        guarded("gather_bench", lambda: gather_bench(torch))
        print("[bench] null mask, buffer rows, split query, decompression, graphs, merge", file=sys.stderr, flush=True)
        guarded("next_rows", lambda: next_rows_bench(torch, w))
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host (bounded sample)", file=sys.stderr, flush=True)
        guarded("cpu_baseline", lambda: cpu_baseline(w, args.cpu_seconds))
    if not args.no_configs:
        # every H=128 workload: its attention alone, with a bounded oracle sample each
        result["configs"] = {}
        for name in ("dsv3", "prefix", "long", "fp8"):
            print(f"[bench] config {name}", file=sys.stderr, flush=True)
            try:
                result["configs"][name] = config_bench(
                    torch, name, cpu_seconds=0.0 if args.no_cpu_baseline else args.config_cpu_seconds)
            except Exception as e:  # noqa: BLE001 -- report, keep the line
                result["configs"][name] = {"error": f"{type(e).__name__}: {e}"}
                print(f"[bench] config {name} failed: {e!r}", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
