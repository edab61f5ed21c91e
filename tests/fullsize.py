"""Full-size parity helpers: the benchmark's workloads in its launch
configuration, every sequence (decode) or one row of every query tile
(prefill) checked against the fp64 oracle.

Outputs are pre-filled with NaN, so the finiteness check of the whole output
also proves that every row was written. The oracle's inputs are host copies
of the device inputs taken before the HIP path runs (the pre-store cache
snapshot), never anything the HIP path wrote. The oracle runs per sequence
in a thread pool (NumPy releases the interpreter lock in its array work);
the oracle functions themselves are the plain ones.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from paged_kv_cache_66_amd import workloads as wl
from tests.helpers import to_host

WORKERS = max(1, min(16, os.cpu_count() or 1))


def nan_out(shape, dtype):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def cache_host(cache, ids, kv_dtype):
    """Host copy of the cache blocks `ids` (device index_select, then copy)."""
    import torch
    rows = cache.index_select(0, torch.from_numpy(np.asarray(ids, np.int64)).cuda())
    if kv_dtype == "fp8e4m3":
        return rows.contiguous().cpu().numpy().view(np.uint8)
    return to_host(rows, kv_dtype)


def decode_reference(w, snap_k, snap_v, q, key, value, seqs, chunk=32):
    """fp64 oracle output [B, H_q, D] (NaN outside `seqs`) of the decode step:
    the oracle's store of each sequence's new row (slot_mapping[b]) into a
    host copy of its blocks from the pre-store snapshot, then its decode.

    q, key, value: device tensors of the step; snap_k / snap_v: device copies
    of the caches before the HIP path ran."""
    bs = w.block_size
    fp8 = w.cache_dtype == "fp8e4m3"
    out = np.full((w.num_seqs, w.num_q_heads, w.head_dim), np.nan)
    q_h, k_h, v_h = to_host(q, w.dtype), to_host(key, w.dtype), to_host(value, w.dtype)

    def one(item):
        b, kh, vh = item
        n = int(w.context_lens[b])
        nb = wl.num_blocks_for(n, bs)
        table = np.arange(nb, dtype=np.int32)[None, :]
        s = int(w.slot_mapping[b])
        if s >= 0 and nb > 0:
            # the slot is position n - 1's: block nb - 1 of the local copy
            local = np.array([(nb - 1) * bs + s % bs], np.int32)
            if fp8:
                oracle.fp8.store_kvcache(oracle.widen(k_h[b:b + 1], "bf16"), oracle.widen(v_h[b:b + 1], "bf16"),
                                         kh, vh, local, w.k_scale, w.v_scale)
            else:
                oracle.store_kvcache(k_h[b:b + 1], v_h[b:b + 1], kh, vh, local)
        if fp8:
            return b, oracle.decode(q_h[b:b + 1], kh, vh, table, np.array([n], np.int32), w.scale, "bf16",
                                    kv_dtype="fp8e4m3", k_scale=w.k_scale, v_scale=w.v_scale)[0]
        return b, oracle.decode(q_h[b:b + 1], kh, vh, table, np.array([n], np.int32), w.scale, w.dtype)[0]

    with ThreadPoolExecutor(WORKERS) as pool:
        for c0 in range(0, len(seqs), chunk):
            items = []
            for b in seqs[c0:c0 + chunk]:
                n = int(w.context_lens[b])
                ids = w.block_tables[b, :wl.num_blocks_for(n, bs)]
                items.append((b, cache_host(snap_k, ids, w.cache_dtype), cache_host(snap_v, ids, w.cache_dtype)))
            for b, ref in pool.map(one, items):
                out[b] = ref
            print(f"[oracle] {w.name}: {min(c0 + chunk, len(seqs))}/{len(seqs)} sequences", flush=True)
    return out


def prefill_rows_per_tile(w, query_tile: int, full_seqs=(0,), extra_seed=4):
    """Query rows to check: every row of the sequences in `full_seqs`, and in
    every other sequence one row of every tile of `query_tile` queries (a
    seeded row inside the tile) plus the sequence's first and last rows."""
    rng = np.random.default_rng(extra_seed)
    rows = []
    for i in range(w.num_seqs):
        q0, q1 = int(w.cu_seqlens_q[i]), int(w.cu_seqlens_q[i + 1])
        if q1 == q0:
            continue
        if i in full_seqs:
            rows += list(range(q0, q1))
            continue
        rows += [q0, q1 - 1]
        for t0 in range(q0, q1, query_tile):
            rows.append(int(rng.integers(t0, min(t0 + query_tile, q1))))
    return sorted(set(rows))


def prefill_reference(w, q_h, kc_h, vc_h, rows):
    """fp64 oracle rows of the prefill over host caches that already hold the
    step's new rows (written by the oracle's store), one sequence per task."""
    fp8 = w.cache_dtype == "fp8e4m3"
    out = np.full((w.total_q, w.num_q_heads, w.head_dim), np.nan)
    want = np.asarray(rows)

    def one(i):
        q0, q1 = int(w.cu_seqlens_q[i]), int(w.cu_seqlens_q[i + 1])
        mine = want[(want >= q0) & (want < q1)]
        if not len(mine):
            return None
        cq = np.array([0, q1 - q0], np.int32)
        ck = np.array([0, int(w.cu_seqlens_k[i + 1] - w.cu_seqlens_k[i])], np.int32)
        kw = dict(kv_dtype="fp8e4m3", k_scale=w.k_scale, v_scale=w.v_scale) if fp8 else {}
        ref = oracle.prefill_varlen(q_h[q0:q1], kc_h, vc_h, cq, ck, w.block_tables[i:i + 1], w.scale, "bf16",
                                    rows=list(mine - q0), **kw)
        return mine, ref[mine - q0]

    with ThreadPoolExecutor(WORKERS) as pool:
        for i, res in enumerate(pool.map(one, range(w.num_seqs))):
            if res is not None:
                out[res[0]] = res[1]
            print(f"[oracle] {w.name}: sequence {i + 1}/{w.num_seqs}", flush=True)
    return out
