"""GPU edge cases of the entry points through the binding: empty batches
(no sequences, or sequences that compute no token) return empty / untouched
outputs without launching anything that could read past the inputs."""
import numpy as np
import pytest

from paged_kv_cache_66_amd import binding
from paged_kv_cache_66_amd import workloads as wl
from tests.helpers import gpu_available, to_device

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _caches(n=8, bs=16, hkv=2, d=128, dtype=None):
    import torch
    dtype = dtype or torch.bfloat16
    kc = torch.full((n, bs, hkv, d), 7.0, dtype=dtype, device="cuda")
    return kc, kc.clone()


@pytest.mark.parametrize("fused", [False, True])
def test_decode_empty_batch(fused):
    import torch
    kc, vc = _caches()
    before = kc.clone()
    q = torch.empty((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    tables = torch.empty((0, 4), dtype=torch.int32, device="cuda")
    ctx = torch.empty((0,), dtype=torch.int32, device="cuda")
    slots = torch.empty((0,), dtype=torch.int32, device="cuda")
    print(f"[edge] empty decode fused={fused}", flush=True)
    if fused:
        out = binding.pa_store_decode(q, kv, kv, slots, kc, vc, tables, ctx, 0.125)
    else:
        out = binding.pa_decode(q, kc, vc, tables, ctx, 0.125)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 4, 128)
    assert torch.equal(kc, before) and torch.equal(vc, before)


@pytest.mark.parametrize("fused", [False, True])
def test_prefill_no_query_tokens(fused):
    """Three sequences with cached history that compute nothing this step."""
    import torch
    w = wl.custom_prefill([10, 64, 300], [0, 0, 0], block_size=16, num_q_heads=8, num_kv_heads=2,
                          head_dim=128, dtype="bf16", seed=71)
    assert w.total_q == 0
    t = wl.make_host_tensors(w)
    kc, vc = to_device(t["k_cache"], "bf16"), to_device(t["v_cache"], "bf16")
    before = kc.clone()
    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    cuq = torch.from_numpy(w.cu_seqlens_q).cuda()
    cuk = torch.from_numpy(w.cu_seqlens_k).cuda()
    tables = torch.from_numpy(w.block_tables).cuda()
    print(f"[edge] prefill without query tokens fused={fused}", flush=True)
    if fused:
        out = binding.pa_store_prefill(q, kv, kv, torch.empty((0,), dtype=torch.int32, device="cuda"), kc, vc,
                                       cuq, cuk, w.max_seqlen_q, w.max_seqlen_k, tables, w.scale)
    else:
        out = binding.pa_prefill_varlen(q, kc, vc, cuq, cuk, w.max_seqlen_q, w.max_seqlen_k, tables, w.scale)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 8, 128)
    assert torch.equal(kc.view(torch.int16), before.view(torch.int16))
    assert np.array_equal(w.cu_seqlens_q, np.zeros(4, dtype=np.int32))
