"""Decode step captured in a HIP graph and replayed, as a serving engine does
for decode ("nano-vLLM Part 2 ...", section 4.2: graphs captured per batch
bucket 1, 2, 4, 8, ...; before replay the runner copies the step's inputs into
static buffers, fills slot_mapping with -1 and zeroes context_lens for the
padding rows).

pa_store_kvcache + pa_decode (or the fused pa_store_decode) are captured
once per bucket with static buffers and replayed over several steps with
changing contents; buckets run from 1 to 512 (the large-batch decode
workload's head shapes for the smallest and largest). Every replay
is compared bit for bit with the same two calls run eagerly on a copy of the
cache state, and with the fp64 oracle; padding rows must leave the cache
untouched and produce zero output rows. Between replays the test runs its own
eager work and synchronises, and it replays several times.
"""
import numpy as np
import pytest

import oracle
from paged_kv_cache_66_amd import binding
from paged_kv_cache_66_amd import workloads as wl
from tests.helpers import assert_attention_close, gpu_available, to_device, to_host, widen_host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _step_inputs(rng, ctx, tables, bs, hq, hkv, d):
    """One decode step's host inputs for the real sequences: q and the new
    token's k/v rows, the slot of position ctx-1 and the context lengths."""
    b = len(ctx)
    q = wl.randn_storage(rng, (b, hq, d), "bf16")
    k = wl.randn_storage(rng, (b, hkv, d), "bf16")
    v = wl.randn_storage(rng, (b, hkv, d), "bf16")
    slots = np.array([wl.slot_of(tables[i], ctx[i] - 1, bs) for i in range(b)], np.int32)
    return q, k, v, slots, np.asarray(ctx, np.int32)


SMALL_HEADS = (8, 2)    # H_q, H_kv
HEADS_8B = (32, 8)      # the large-batch decode workload's heads


@pytest.mark.parametrize("bucket,real,heads,fused", [
    (8, 5, SMALL_HEADS, False), (4, 4, SMALL_HEADS, False), (16, 9, SMALL_HEADS, False),
    (1, 1, HEADS_8B, False), (1, 1, HEADS_8B, True),          # the smallest bucket
    (512, 300, HEADS_8B, False), (512, 300, HEADS_8B, True),  # the largest bucket, mostly real rows
    # the rest of the power-of-two ladder between them
    (2, 1, HEADS_8B, True), (32, 20, HEADS_8B, False), (64, 64, HEADS_8B, True),
    (128, 100, HEADS_8B, False), (256, 170, HEADS_8B, True),
])
def test_graph_replay_matches_eager(bucket, real, heads, fused):
    import torch
    hq, hkv = heads
    d, bs = 128, 16
    rng = np.random.default_rng(bucket * 100 + real + 7 * fused)
    steps = 3
    # sequences grow by one token per step; reserve blocks for every step
    ctx0 = [int(x) for x in rng.integers(20, 120, size=real)]
    need = [wl.num_blocks_for(c + steps, bs) for c in ctx0]
    n_blocks = sum(need) + 4
    free = [int(x) for x in rng.permutation(n_blocks)]
    tables = [wl.take_blocks(free, n) for n in need]
    width = max(need)
    # cache: history rows random, everything else NaN
    kc = np.full((n_blocks, bs, hkv, d), wl.BF16_NAN_BITS, np.uint16)
    vc = np.full_like(kc, wl.BF16_NAN_BITS)
    for t, c in zip(tables, ctx0):
        for p in range(c - 1):
            kc[t[p // bs], p % bs] = wl.randn_storage(rng, (hkv, d), "bf16")
            vc[t[p // bs], p % bs] = wl.randn_storage(rng, (hkv, d), "bf16")
    kc_d, vc_d = to_device(kc, "bf16"), to_device(vc, "bf16")

    # static buffers of the bucket; padding rows: slot -1, ctx 0, table -1
    q_s = torch.zeros((bucket, hq, d), dtype=torch.bfloat16, device="cuda")
    k_s = torch.zeros((bucket, hkv, d), dtype=torch.bfloat16, device="cuda")
    v_s = torch.zeros_like(k_s)
    slots_s = torch.full((bucket,), -1, dtype=torch.int32, device="cuda")
    ctx_s = torch.zeros((bucket,), dtype=torch.int32, device="cuda")
    tables_s = torch.full((bucket, width), -1, dtype=torch.int32, device="cuda")
    tables_s[:real] = torch.from_numpy(wl.pad_block_tables(tables, width)).cuda()
    out_s = torch.empty((bucket, hq, d), dtype=torch.bfloat16, device="cuda")
    need_ws = binding.pa_decode_workspace_size(bucket, hq, hkv, d, bs, width, 64)
    ws = torch.empty(max(need_ws, 16), dtype=torch.uint8, device="cuda")
    scale = 1.0 / np.sqrt(d)

    def fill(q, k, v, slots, ctx):
        q_s[:real].copy_(to_device(q, "bf16"))
        k_s[:real].copy_(to_device(k, "bf16"))
        v_s[:real].copy_(to_device(v, "bf16"))
        slots_s.fill_(-1)
        slots_s[:real].copy_(torch.from_numpy(slots).cuda())
        ctx_s.zero_()
        ctx_s[:real].copy_(torch.from_numpy(ctx).cuda())

    def step_calls(kcache, vcache, out):
        if fused:
            binding.pa_store_decode(q_s, k_s, v_s, slots_s, kcache, vcache, tables_s, ctx_s, scale, out=out,
                                    workspace=ws, partition_size=64)
            return
        binding.pa_store_kvcache(k_s, v_s, kcache, vcache, slots_s)
        binding.pa_decode(q_s, kcache, vcache, tables_s, ctx_s, scale, out=out, workspace=ws,
                          partition_size=64)

    # warm up on a side stream, then capture
    inputs = _step_inputs(rng, ctx0, tables, bs, hq, hkv, d)
    fill(*inputs)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kw, vw = kc_d.clone(), vc_d.clone()
        step_calls(kw, vw, torch.empty_like(out_s))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    print(f"[graph] capture bucket={bucket} real={real} heads={heads} fused={fused}", flush=True)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step_calls(kc_d, vc_d, out_s)
    torch.cuda.synchronize()

    ctx = list(ctx0)
    kc_h, vc_h = kc.copy(), vc.copy()
    for step in range(steps):
        if step > 0:
            inputs = _step_inputs(rng, ctx, tables, bs, hq, hkv, d)
        q, k, v, slots, ctx_arr = inputs
        fill(q, k, v, slots, ctx_arr)
        kc_before, vc_before = kc_d.clone(), vc_d.clone()
        torch.cuda.synchronize()
        print(f"[graph] replay step {step}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        got = out_s.clone()
        # eager run of the same calls on the pre-replay cache state
        eager_out = torch.empty_like(out_s)
        step_calls(kc_before, vc_before, eager_out)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager_out.view(torch.int16)), f"step {step}"
        assert torch.equal(kc_d.view(torch.int16), kc_before.view(torch.int16))
        assert torch.equal(vc_d.view(torch.int16), vc_before.view(torch.int16))
        # padding rows: zero output
        assert bool((got[real:].float() == 0).all())
        # oracle on the real rows
        oracle.store_kvcache(k, v, kc_h, vc_h, slots)
        ref = oracle.decode(q, kc_h, vc_h, wl.pad_block_tables(tables, width), ctx_arr, scale, "bf16")
        assert_attention_close(widen_host(to_host(got[:real], "bf16"), "bf16"), ref, "bf16",
                               f"graph step {step}")
        assert np.array_equal(to_host(kc_d, "bf16"), kc_h)
        ctx = [c + 1 for c in ctx]
