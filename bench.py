#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

The metric has two halves, each reported against its roofline:

* decode KV-read GB/s (headline `value`, `roofline`): the 8B-shaped
  large-batch decode step at block size 16 -- 512 sequences, H_q=32,
  H_kv=8, D=128, bf16, context lengths log-uniform in [512, 32768], a pool
  of 1.1x the needed blocks with random placement (the largest decode
  workload). One step is pa_store_decode: the scatter of the 512 new tokens
  and the decode over every sequence's whole history in one launch (plus
  the split-K merge); the same step as two calls (pa_store_kvcache, then
  pa_decode) is timed too;
* prefill TFLOP/s (`roofline_prefill`): the chunked varlen prefill -- 16384
  query tokens over 24 sequences with shared cached prefixes; pa_prefill_varlen
  after the chunk's pa_store_kvcache, and the same step as one
  pa_store_prefill launch.

Inputs are generated on the device (seed 0) before timing; an untimed read
of a 1 GiB buffer evicts L2/MALL before each timed call, so every call reads
its KV cold, as a layer's KV would be in a model step (a read, not a write,
so no dirty lines are left for the call to write back). Every workload runs
`--warmup` untimed and `--steps` timed calls of each variant; the JSON
reports means (value, rooflines), medians and p10/p90.

Also measured (unless --quick): the same decode at block size 256, the
Qwen3-0.6B-shaped decode, the 131072-token long-context split-K decode, the
fp8 (E4M3) cache variants, and small-batch decode issued eagerly and as HIP
graph replays.

Prints one JSON line. `cpu_baseline` / `cpu_baseline_prefill` time the fp64
oracle on the host over a bounded sample of the decode and prefill
workloads. `library` is pa_version(), whose source hash must equal this
tree's (checked before anything runs).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, AMD published
METRIC = "decode KV-read GB/s (% HBM peak) + prefill TFLOP/s (% MFMA peak), 1 GPU"
HEADLINE = "8b-decode-bs16"
PREFILL = "chunked-prefill"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--quick", action="store_true", help="the two roofline workloads only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget per baseline")
    ap.add_argument("--partition", type=int, default=0, help="decode partition (0 = library default)")
    return ap.parse_args()


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def stored_traffic(workload, kind):
    """Per-launch HBM bytes of the workload's timed call from committed
    rocprofv3 --pmc runs, or None when absent or taken on other kernel
    sources (the stamp is the SHA-256 of the kernel family's sources)."""
    from paged_kv_cache_66_amd import srchash
    try:
        with open(traffic_file(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha256") != srchash.kernel_sha256(kind):
        return None
    return rec.get("bytes_per_launch")


def flush_caches(scratch):
    """Evict L2 and MALL by streaming a 1 GiB buffer through them (reads)."""
    scratch.view(-1).amax()


class Timer:
    """Per-step HIP events on the current stream (the stream the library's
    calls are enqueued on)."""

    def __init__(self, torch, n, marks):
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(marks)] for _ in range(n)]

    def rec(self, step, mark):
        self.ev[step][mark].record()

    def span(self, a, b):
        return [e[a].elapsed_time(e[b]) for e in self.ev]


def summary(ms):
    """mean, median, p10, p90 of a list of per-call times (ms)."""
    s = sorted(ms)
    n = len(s)
    return dict(mean=sum(s) / n, median=s[n // 2], p10=s[n // 10], p90=s[min(n - 1, (9 * n) // 10)])


def rounded(d, nd=5):
    if isinstance(d, dict):
        return {k: rounded(v, nd) for k, v in d.items()}
    if isinstance(d, list):
        return [rounded(v, nd) for v in d]
    return round(d, nd) if isinstance(d, float) else d


def run_decode(torch, binding, wl, w, steps, warmup, flush, scratch, partition=0):
    """Time one decode workload: the step as two calls (store, then decode;
    events around each) and as one fused call, `warmup` untimed and `steps`
    timed calls of each, the caches evicted before every timed call."""
    t = wl.make_device_tensors(w)
    slots = torch.from_numpy(w.slot_mapping).cuda()
    tables = torch.from_numpy(w.block_tables).cuda()
    ctx = torch.from_numpy(w.context_lens).cuda()
    out = torch.empty_like(t["q"].contiguous())
    need = binding.pa_decode_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                            w.block_size, w.max_blocks_per_seq, partition)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    fp8 = w.cache_dtype == "fp8e4m3"

    def store():
        if fp8:
            binding.pa_store_kvcache_fp8(t["k"], t["v"], t["k_cache"], t["v_cache"], slots, w.k_scale,
                                         w.v_scale)
        else:
            binding.pa_store_kvcache(t["k"], t["v"], t["k_cache"], t["v_cache"], slots)

    def dec():
        if fp8:
            binding.pa_decode_fp8(t["q"], t["k_cache"], t["v_cache"], tables, ctx, w.scale, w.k_scale,
                                  w.v_scale, out=out, workspace=ws, partition_size=partition)
        else:
            binding.pa_decode(t["q"], t["k_cache"], t["v_cache"], tables, ctx, w.scale, out=out,
                              workspace=ws, partition_size=partition)

    def fused():
        if fp8:
            binding.pa_store_decode_fp8(t["q"], t["k"], t["v"], slots, t["k_cache"], t["v_cache"], tables,
                                        ctx, w.scale, w.k_scale, w.v_scale, out=out, workspace=ws,
                                        partition_size=partition)
        else:
            binding.pa_store_decode(t["q"], t["k"], t["v"], slots, t["k_cache"], t["v_cache"], tables, ctx,
                                    w.scale, out=out, workspace=ws, partition_size=partition)

    for _ in range(warmup):  # cold like the timed calls, so every call of a kernel sees the same state
        for fn in (store, dec, fused):
            if flush:
                flush_caches(scratch)
            fn()
    torch.cuda.synchronize()
    timer = Timer(torch, steps, 3)
    for s in range(steps):
        if flush:
            flush_caches(scratch)
        timer.rec(s, 0)
        store()
        timer.rec(s, 1)
        dec()
        timer.rec(s, 2)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all()), f"{w.name}: non-finite decode output"
    ftimer = Timer(torch, steps, 2)
    for s in range(steps):
        if flush:
            flush_caches(scratch)
        ftimer.rec(s, 0)
        fused()
        ftimer.rec(s, 1)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all()), f"{w.name}: non-finite fused output"
    res = dict(
        workload=w.name,
        steps=steps,
        fused_ms=summary(ftimer.span(0, 1)),
        two_call_ms=summary(timer.span(0, 2)),
        decode_ms=summary(timer.span(1, 2)),
        store_ms=summary(timer.span(0, 1)),
        bytes_logical=w.algorithmic_bytes(unique=False),
        bytes_unique=w.algorithmic_bytes(unique=True),
        flops=w.flops(),
    )
    # the fused call also writes the new rows and reads the slot mapping
    res["fused_bytes"] = res["bytes_logical"] + w.num_seqs * 2 * w.num_kv_heads * w.head_dim * \
        (1 if fp8 else w.elem_bytes) + 4 * w.num_seqs
    for key in ("fused_ms", "decode_ms"):
        m = res[key]["mean"] * 1e-3
        res[key.replace("_ms", "_GBps")] = res["bytes_logical"] / m / 1e9
        res[key.replace("_ms", "_GBps_unique")] = res["bytes_unique"] / m / 1e9
    res["hbm_frac_unique"] = res["fused_GBps_unique"] / HBM_PEAK_GBS
    g = w.num_q_heads // w.num_kv_heads
    tag = "Fp8Tag" if fp8 else ("BF16Tag" if w.elem_bytes == 2 else "float")
    # block trips (the last template argument) need G >= 8, a 16-bit or fp8 cache and 256+ row blocks;
    # the partition the library picks decides the rest, so the name says "BT" where they may apply
    trips = "BT" if g >= 8 and tag != "float" and w.block_size >= 256 else "false"
    res["kernel"] = (f"pa_store_decode (decode_partition_kernel<{tag}, {w.head_dim}, {g}, true, {trips}> "
                     f"+ decode_reduce_kernel)")
    del t
    return res


def run_prefill(torch, binding, wl, w, steps, warmup, flush, scratch):
    """Time the prefill step: the chunk's scatter then pa_prefill_varlen
    (events around each), and the same step as one fused call."""
    t = wl.make_device_tensors(w)
    slots = torch.from_numpy(w.slot_mapping).cuda()
    cuq = torch.from_numpy(w.cu_seqlens_q).cuda()
    cuk = torch.from_numpy(w.cu_seqlens_k).cuda()
    tables = torch.from_numpy(w.block_tables).cuda()
    out = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=t["q"].dtype, device="cuda")
    fp8 = w.cache_dtype == "fp8e4m3"

    def store():
        if fp8:
            binding.pa_store_kvcache_fp8(t["k"], t["v"], t["k_cache"], t["v_cache"], slots, w.k_scale,
                                         w.v_scale)
        else:
            binding.pa_store_kvcache(t["k"], t["v"], t["k_cache"], t["v_cache"], slots)

    def pre():
        if fp8:
            binding.pa_prefill_varlen_fp8(t["q"], t["k_cache"], t["v_cache"], cuq, cuk, w.max_seqlen_q,
                                          w.max_seqlen_k, tables, w.scale, w.k_scale, w.v_scale, out=out)
        else:
            binding.pa_prefill_varlen(t["q"], t["k_cache"], t["v_cache"], cuq, cuk, w.max_seqlen_q,
                                      w.max_seqlen_k, tables, w.scale, out=out)

    def fused():
        if fp8:
            binding.pa_store_prefill_fp8(t["q"], t["k"], t["v"], slots, t["k_cache"], t["v_cache"], cuq, cuk,
                                         w.max_seqlen_q, w.max_seqlen_k, tables, w.scale, w.k_scale,
                                         w.v_scale, out=out)
        else:
            binding.pa_store_prefill(t["q"], t["k"], t["v"], slots, t["k_cache"], t["v_cache"], cuq, cuk,
                                     w.max_seqlen_q, w.max_seqlen_k, tables, w.scale, out=out)

    for _ in range(warmup):
        for fn in (store, pre, fused):
            if flush:
                flush_caches(scratch)
            fn()
    torch.cuda.synchronize()
    timer = Timer(torch, steps, 3)
    for s in range(steps):
        if flush:
            flush_caches(scratch)
        timer.rec(s, 0)
        store()
        timer.rec(s, 1)
        pre()
        timer.rec(s, 2)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all()), "prefill: non-finite output"
    ftimer = Timer(torch, steps, 2)
    for s in range(steps):
        if flush:
            flush_caches(scratch)
        ftimer.rec(s, 0)
        fused()
        ftimer.rec(s, 1)
    torch.cuda.synchronize()
    flops = w.flops()
    res = dict(
        workload=w.name,
        steps=steps,
        prefill_ms=summary(timer.span(1, 2)),
        store_ms=summary(timer.span(0, 1)),
        two_call_ms=summary(timer.span(0, 2)),
        fused_ms=summary(ftimer.span(0, 1)),
        flops=flops,
        store_bytes=w.store_bytes(),
    )
    res["prefill_TFLOPs"] = flops / (res["prefill_ms"]["mean"] * 1e-3) / 1e12
    res["prefill_TFLOPs_median"] = flops / (res["prefill_ms"]["median"] * 1e-3) / 1e12
    res["fused_TFLOPs"] = flops / (res["fused_ms"]["mean"] * 1e-3) / 1e12
    res["mfma_frac"] = res["prefill_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS
    res["store_GBps"] = w.store_bytes() / (res["store_ms"]["mean"] * 1e-3) / 1e9
    del t
    return res


def run_graph_small(torch, binding, wl, steps=100):
    """Small decode batches are launch-bound: time back-to-back steps issued
    eagerly and as one HIP-graph replay per step, wall clock over the whole
    run, no cache eviction. A step is the attention of 1 layer, or of the 28
    layers of a Qwen3-0.6B-shaped model (each layer its own cache), as a
    serving engine captures the whole decode forward per batch bucket."""
    w = wl.custom_decode([512] * 8, block_size=256, num_q_heads=16, num_kv_heads=8, head_dim=128,
                         dtype="bf16", seed=5, width=2)
    t = wl.make_device_tensors(w)
    slots = torch.from_numpy(w.slot_mapping).cuda()
    tables = torch.from_numpy(w.block_tables).cuda()
    ctx = torch.from_numpy(w.context_lens).cuda()
    out = torch.empty_like(t["q"].contiguous())
    need = binding.pa_decode_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                            w.block_size, w.max_blocks_per_seq, 0)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    n_layers = 28
    caches = [(t["k_cache"].clone(), t["v_cache"].clone()) for _ in range(n_layers)]

    def step(layers):
        def run():
            for kc, vc in caches[:layers]:
                binding.pa_store_kvcache(t["k"], t["v"], kc, vc, slots)
                binding.pa_decode(t["q"], kc, vc, tables, ctx, w.scale, out=out, workspace=ws)
        return run

    def fused(layers):
        def run():
            for kc, vc in caches[:layers]:
                binding.pa_store_decode(t["q"], t["k"], t["v"], slots, kc, vc, tables, ctx, w.scale,
                                        out=out, workspace=ws)
        return run

    res = {}
    for layers in (1, n_layers):
        fns = {"eager": step(layers), "eager_fused": fused(layers)}
        for name in ("eager", "eager_fused"):
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(3):
                    fns[name]()
            torch.cuda.current_stream().wait_stream(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fns[name]()
            fns[name.replace("eager", "graph")] = g.replay
        torch.cuda.synchronize()
        for name in ("eager", "eager_fused", "graph", "graph_fused"):
            fn = fns[name]
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
            res[f"{layers}L_{name}_us_per_step"] = round((time.perf_counter() - t0) / steps * 1e6, 2)
    res["workload"] = ("8 seqs x 512 tokens, qwen3-0.6b attention shapes; per step 1 layer or 28 layers "
                       "of store + decode (two calls, or the fused call)")
    del t, caches
    return res


def host_info():
    """Host cores and the BLAS NumPy uses (vendor, threads)."""
    import numpy as np
    info = {"cpu_count": os.cpu_count()}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        info["blas"] = f"{blas.get('name')} {blas.get('version', '')}".strip()
    except Exception:  # noqa: BLE001 - older numpy: no dict mode
        info["blas"] = None
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        info["blas_threads"] = max((p.get("num_threads", 1) for p in pools), default=1)
        info["threadpools"] = [f"{p.get('internal_api')}:{p.get('num_threads')}" for p in pools]
    except Exception:  # noqa: BLE001
        info["blas_threads"] = None
    return info


def one_thread():
    """Context that holds NumPy's BLAS to one thread, so the oracle's
    timing uses exactly one core (a no-op context without threadpoolctl,
    which the host report then shows)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except Exception:  # noqa: BLE001
        import contextlib
        return contextlib.nullcontext()


def cpu_baseline_decode(torch, wl, w, seconds):
    """fp64 oracle on the host over the decode workload, sequence by
    sequence in order: each sequence's blocks are copied to the host
    (untimed), then the oracle's store of the new row and its decode run
    (timed), until the time budget is spent. One thread runs the oracle."""
    import numpy as np

    import oracle
    from tests.helpers import to_host

    t = wl.make_device_tensors(w)
    bs = w.block_size
    q_h, k_h, v_h = (to_host(t[x], w.dtype) for x in ("q", "k", "v"))
    done_bytes, done, spent = 0, 0, 0.0
    for b in range(w.num_seqs):
        n = int(w.context_lens[b])
        nb = wl.num_blocks_for(n, bs)
        ids = torch.from_numpy(w.block_tables[b, :nb].astype(np.int64)).cuda()
        kh = to_host(t["k_cache"].index_select(0, ids), w.dtype)
        vh = to_host(t["v_cache"].index_select(0, ids), w.dtype)
        with one_thread():
            c0 = time.perf_counter()
            oracle.store_kvcache(k_h[b:b + 1], v_h[b:b + 1], kh, vh,
                                 np.array([(nb - 1) * bs + (n - 1) % bs], np.int32))
            oracle.decode(q_h[b:b + 1], kh, vh, np.arange(nb, dtype=np.int32)[None], np.array([n], np.int32),
                          w.scale, w.dtype)
            spent += time.perf_counter() - c0
        done += 1
        done_bytes += n * 2 * w.num_kv_heads * w.head_dim * w.elem_bytes + \
            2 * w.num_q_heads * w.head_dim * w.elem_bytes + nb * 4 + 4
        if spent >= seconds:
            break
    del t
    info = host_info()
    return {
        "value": round(done_bytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the first {done} of the {w.num_seqs} sequences of {w.name} ({done_bytes / 1e9:.2f} GB of "
                  f"the step's {w.algorithmic_bytes() / 1e9:.2f} GB; fp64 NumPy store + decode, one sequence "
                  f"at a time on one thread), {spent:.1f} s of oracle compute",
        "host": info,
    }


def cpu_baseline_prefill(torch, wl, w, seconds):
    """fp64 oracle on the host over the prefill workload: the caches, queries
    and new rows are copied to the host and the oracle stores the chunk
    (untimed); then rows are computed sequence by sequence, a seeded sample
    of rows per sequence, until the time budget is spent. The flop count is
    the metric's (QK^T + PV over the unmasked pairs) for the rows done."""
    import numpy as np

    import oracle
    from tests.helpers import to_host

    t = wl.make_device_tensors(w)
    kc, vc = to_host(t["k_cache"], w.dtype), to_host(t["v_cache"], w.dtype)
    q_h, k_h, v_h = (to_host(t[x], w.dtype) for x in ("q", "k", "v"))
    del t
    oracle.store_kvcache(k_h, v_h, kc, vc, w.slot_mapping)
    rng = np.random.default_rng(7)
    done_rows, flops, spent = 0, 0.0, 0.0
    while spent < seconds:
        for i in range(w.num_seqs):
            q0, q1 = int(w.cu_seqlens_q[i]), int(w.cu_seqlens_q[i + 1])
            lq, lk = q1 - q0, int(w.cu_seqlens_k[i + 1] - w.cu_seqlens_k[i])
            if lq == 0:
                continue
            rows = sorted(set(int(x) for x in rng.integers(0, lq, 4)))
            with one_thread():
                c0 = time.perf_counter()
                oracle.prefill_varlen(q_h[q0:q1], kc, vc, np.array([0, lq], np.int32),
                                      np.array([0, lk], np.int32), w.block_tables[i:i + 1], w.scale, w.dtype,
                                      rows=rows)
                spent += time.perf_counter() - c0
            done_rows += len(rows)
            flops += sum(4.0 * w.head_dim * w.num_q_heads * (lk - lq + j + 1) for j in rows)
            if spent >= seconds:
                break
    return {
        "value": round(flops / spent / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done_rows} query rows of {w.name} (4 seeded rows per sequence per pass, all 32 heads; "
                  f"{flops / 1e9:.1f} GFLOP of the step's {w.flops() / 1e12:.3f} TFLOP; fp64 NumPy, one "
                  f"thread), {spent:.1f} s of oracle compute",
        "host": host_info(),
    }


def decode_roofline(res, traffic):
    fm = res["fused_ms"]["mean"]
    achieved = res["fused_bytes"] / (fm * 1e-3) / 1e9
    return {
        "bound": "hbm",
        "achieved": round(achieved, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "workload": res["workload"],
        "kernel": res["kernel"],
        "algorithmic_bytes_per_launch": res["fused_bytes"],
        "avg_launch_ms": round(fm, 5),
        "median_launch_ms": round(res["fused_ms"]["median"], 5),
        "p10_p90_launch_ms": [round(res["fused_ms"]["p10"], 5), round(res["fused_ms"]["p90"], 5)],
    }


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch

    from paged_kv_cache_66_amd import binding
    from paged_kv_cache_66_amd import workloads as wl

    binding.load()
    binding.check_source_hash()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    flush = not args.no_flush
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda") if flush else None
    steps, warm = args.steps, args.warmup

    w = wl.DECODE_CONFIGS[HEADLINE](0)
    log(f"[bench] {w.name}: warmup {warm}, steps {steps}")
    head = run_decode(torch, binding, wl, w, steps, warm, flush, scratch, args.partition)
    torch.cuda.empty_cache()
    log(f"[bench] {w.name}: fused {head['fused_ms']['mean'] * 1e3:.1f} us, {head['fused_GBps']:.0f} GB/s")

    wp = wl.PREFILL_CONFIGS[PREFILL](0)
    log(f"[bench] {wp.name}")
    pre = run_prefill(torch, binding, wl, wp, steps, warm, flush, scratch)
    torch.cuda.empty_cache()
    log(f"[bench] {wp.name}: prefill {pre['prefill_ms']['mean']:.3f} ms, {pre['prefill_TFLOPs']:.1f} TFLOP/s")

    secondary = {}
    if not args.quick:
        for name in ("8b-decode-bs256", "qwen3-0.6b-decode", "long-context-decode", "qwen3-0.6b-decode-fp8",
                     "long-context-decode-fp8"):
            log(f"[bench] {name}")
            r = run_decode(torch, binding, wl, wl.DECODE_CONFIGS[name](0), steps, warm, flush, scratch,
                           args.partition)
            torch.cuda.empty_cache()
            if name in ("8b-decode-bs256", "qwen3-0.6b-decode"):
                r["roofline"] = decode_roofline(r, stored_traffic(name, "decode"))
            secondary[name] = rounded(r, 4)
            log(f"[bench] {name}: fused {r['fused_ms']['mean']:.4f} ms, {r['fused_GBps_unique']:.0f} GB/s unique")
        log("[bench] graph replay, small batch")
        secondary["decode-graph-small"] = run_graph_small(torch, binding, wl)
        log(f"[bench] small batch: {secondary['decode-graph-small']}")
        name = "chunked-prefill-fp8"
        log(f"[bench] {name}")
        p = run_prefill(torch, binding, wl, wl.PREFILL_CONFIGS[name](0), steps, warm, flush, scratch)
        torch.cuda.empty_cache()
        secondary[name] = rounded(p, 4)
        log(f"[bench] {name}: prefill {p['prefill_ms']['mean']:.3f} ms, {p['prefill_TFLOPs']:.1f} TFLOP/s")

    cpu = cpu_pre = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle), decode")
        cpu = cpu_baseline_decode(torch, wl, w, args.cpu_seconds)
        log("[bench] cpu baseline (oracle), prefill")
        cpu_pre = cpu_baseline_prefill(torch, wl, wp, args.cpu_seconds)

    pm = pre["prefill_ms"]["mean"]
    rec = {
        "metric": METRIC,
        "value": round(head["fused_GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(head["fused_ms"]["mean"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/q generated on the device; random block placement)",
        "config": {
            "workload": w.name,
            "batch": w.num_seqs,
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "num_blocks": w.num_blocks,
            "context_lens": "round(exp(U(ln 512, ln 32768))), seed 0",
            "sum_context": int(w.context_lens.sum()),
            "step": "pa_store_decode: scatter of the 512 new K/V rows + decode, one launch (+ split-K merge)",
            "value_is": "decode algorithmic bytes / mean fused-call time",
            "cache": "cold (L2/MALL evicted before each call)" if flush else "warm",
            "parallelism": "none (1 GPU)",
        },
        "roofline": decode_roofline(head, stored_traffic(HEADLINE, "decode")),
        "roofline_prefill": {
            "bound": "mfma",
            "achieved": round(pre["prefill_TFLOPs"], 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre["prefill_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": stored_traffic(PREFILL, "prefill"),
            "workload": wp.name,
            "kernel": "pa_prefill_varlen (prefill_direct_kernel<128, 4, false>)",
            "algorithmic_flops_per_launch": pre["flops"],
            "avg_launch_ms": round(pm, 5),
            "median_launch_ms": round(pre["prefill_ms"]["median"], 5),
            "p10_p90_launch_ms": [round(pre["prefill_ms"]["p10"], 5), round(pre["prefill_ms"]["p90"], 5)],
        },
        "cpu_baseline": cpu,
        "cpu_baseline_prefill": cpu_pre,
        "components": {
            "decode": rounded(head, 5),
            "prefill": rounded(pre, 5),
        },
        "secondary": secondary,
        "library": binding.version(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
