"""Run one hot-path operation a few times, for rocprofv3.

    rocprofv3 --kernel-trace --stats --output-format csv -d OUT -o run -- \\
        python3 -m paged_kv_cache_66_amd.profile_ops decode qwen3-0.6b-decode

Operations:
  decode <workload>   pa_store_kvcache of the new tokens + pa_decode, inputs
                      resident, a 1 GiB read between calls (cold caches);
  store_decode <workload>  the same step as one pa_store_decode launch;
  prefill [workload]  pa_store_kvcache + pa_prefill_varlen on chunked-prefill
                      (or chunked-prefill-fp8: the _fp8 entry points);
  store_prefill [workload]  the same step as one pa_store_prefill call
                      (pa_store_prefill_fp8 over fp8 caches);
  copy                a 1 GiB device-to-device copy (counter calibration:
                      reads 1 GiB, writes 1 GiB).
Workloads are the seeded synthetic ones of ``workloads.py``; a workload over
fp8 caches (name ending in -fp8) runs the *_fp8 entry points.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("op", choices=["decode", "store_decode", "prefill", "store_prefill", "copy"])
    ap.add_argument("workload", nargs="?", default="qwen3-0.6b-decode")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--partition", type=int, default=0)
    args = ap.parse_args(argv)

    import torch

    from paged_kv_cache_66_amd import binding
    from paged_kv_cache_66_amd import workloads as wl

    binding.load()
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    if args.op == "copy":
        dst = torch.empty_like(scratch)
        for _ in range(args.reps):
            dst.copy_(scratch)
    elif args.op in ("prefill", "store_prefill"):
        name = args.workload if args.workload in wl.PREFILL_CONFIGS else "chunked-prefill"
        w = wl.PREFILL_CONFIGS[name](0)
        fp8 = w.cache_dtype == "fp8e4m3"
        t = wl.make_device_tensors(w)
        slots = torch.from_numpy(w.slot_mapping).cuda()
        cuq = torch.from_numpy(w.cu_seqlens_q).cuda()
        cuk = torch.from_numpy(w.cu_seqlens_k).cuda()
        tables = torch.from_numpy(w.block_tables).cuda()
        out = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        for _ in range(args.reps):
            scratch.amax()
            if args.op == "store_prefill":
                fused = binding.pa_store_prefill_fp8 if fp8 else binding.pa_store_prefill
                extra = (w.k_scale, w.v_scale) if fp8 else ()
                fused(t["q"], t["k"], t["v"], slots, t["k_cache"], t["v_cache"], cuq, cuk, w.max_seqlen_q,
                      w.max_seqlen_k, tables, w.scale, *extra, out=out)
                continue
            if fp8:
                binding.pa_store_kvcache_fp8(t["k"], t["v"], t["k_cache"], t["v_cache"], slots, w.k_scale,
                                             w.v_scale)
                binding.pa_prefill_varlen_fp8(t["q"], t["k_cache"], t["v_cache"], cuq, cuk, w.max_seqlen_q,
                                              w.max_seqlen_k, tables, w.scale, w.k_scale, w.v_scale, out=out)
                continue
            binding.pa_store_kvcache(t["k"], t["v"], t["k_cache"], t["v_cache"], slots)
            binding.pa_prefill_varlen(t["q"], t["k_cache"], t["v_cache"], cuq, cuk, w.max_seqlen_q,
                                      w.max_seqlen_k, tables, w.scale, out=out)
    else:
        w = wl.DECODE_CONFIGS[args.workload](0)
        fp8 = w.cache_dtype == "fp8e4m3"
        t = wl.make_device_tensors(w)
        slots = torch.from_numpy(w.slot_mapping).cuda()
        tables = torch.from_numpy(w.block_tables).cuda()
        ctx = torch.from_numpy(w.context_lens).cuda()
        out = torch.empty_like(t["q"].contiguous())
        for _ in range(args.reps):
            scratch.amax()
            if args.op == "store_decode" and fp8:
                binding.pa_store_decode_fp8(t["q"], t["k"], t["v"], slots, t["k_cache"], t["v_cache"],
                                            tables, ctx, w.scale, w.k_scale, w.v_scale, out=out,
                                            partition_size=args.partition)
            elif args.op == "store_decode":
                binding.pa_store_decode(t["q"], t["k"], t["v"], slots, t["k_cache"], t["v_cache"], tables,
                                        ctx, w.scale, out=out, partition_size=args.partition)
            elif fp8:
                binding.pa_store_kvcache_fp8(t["k"], t["v"], t["k_cache"], t["v_cache"], slots, w.k_scale,
                                             w.v_scale)
                binding.pa_decode_fp8(t["q"], t["k_cache"], t["v_cache"], tables, ctx, w.scale, w.k_scale,
                                      w.v_scale, out=out, partition_size=args.partition)
            else:
                binding.pa_store_kvcache(t["k"], t["v"], t["k_cache"], t["v_cache"], slots)
                binding.pa_decode(t["q"], t["k_cache"], t["v_cache"], tables, ctx, w.scale, out=out,
                                  partition_size=args.partition)
    torch.cuda.synchronize()
    print(f"profile_ops {args.op} {args.workload if args.op != 'copy' else ''} done", flush=True)


if __name__ == "__main__":
    main()
