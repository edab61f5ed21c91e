"""Seeded random shape sweep against the fp64 oracle: decode (two calls and
fused), prefill (two calls and fused) and the fp8 variants over random
batch sizes, context and chunk lengths (zero included), block sizes 1-1024,
group sizes 1-16, both head dims, both dtypes and explicit partitions. Each
case reuses the parity runner of its entry point; the case index seeds
everything, and the shapes are printed before each case runs."""
import numpy as np
import pytest

from paged_kv_cache_66_amd import workloads as wl
from tests import test_gpu_decode as dec
from tests import test_gpu_fp8 as fp8
from tests import test_gpu_store_prefill as spf
from tests.helpers import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

GROUPS = [1, 2, 4, 8, 16]


def _heads(rng):
    g = int(rng.choice(GROUPS))
    hkv = int(rng.choice([1, 2, 4])) if g <= 8 else int(rng.choice([1, 2]))
    return g * hkv, hkv, g


def _decode_case(i):
    rng = np.random.default_rng(7000 + i)
    hq, hkv, g = _heads(rng)
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    bs = int(2 ** rng.integers(0, 11))                      # 1 .. 1024
    b = int(rng.integers(1, 13))
    ctx = [int(c) for c in rng.integers(1, 700, size=b)]
    if b > 2:
        ctx[int(rng.integers(0, b))] = 0                    # an idle padding row
    parts = [p for p in (0, 64, 128, 256, 512, 1024) if p == 0 or g * p <= 8192]
    part = int(rng.choice(parts))
    w = wl.custom_decode(ctx, block_size=bs, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                         seed=7000 + i, name=f"random-decode-{i}")
    return w, part, bool(rng.integers(0, 2))


def _prefill_case(i):
    rng = np.random.default_rng(8000 + i)
    hq, hkv, g = _heads(rng)
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([4, 16, 32, 64, 128, 256]))
    b = int(rng.integers(1, 7))
    cached = [int(c) for c in rng.integers(0, 700, size=b)]
    sched = [int(s) for s in rng.integers(1, 300, size=b)]
    if b > 2:
        sched[int(rng.integers(0, b))] = 0                  # a sequence with nothing to compute
    w = wl.custom_prefill(cached, sched, block_size=bs, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                          dtype="bf16", seed=8000 + i, name=f"random-prefill-{i}")
    return w


@pytest.mark.parametrize("i", range(48))
def test_random_decode(i):
    w, part, fused = _decode_case(i)
    if fused:
        t = wl.make_host_tensors(w)
        dev = dec._device_inputs(w, t)
        out = dec._fused_vs_separate(w, {x: dev[x] for x in ("q", "k", "v", "k_cache", "v_cache")}, part)
        kc, vc = t["k_cache"].copy(), t["v_cache"].copy()
        dec.oracle.store_kvcache(t["k"], t["v"], kc, vc, w.slot_mapping)
        ref = dec.oracle.decode(t["q"], kc, vc, w.block_tables, w.context_lens, w.scale, w.dtype)
        dec.assert_attention_close(dec.widen_host(dec.to_host(out, w.dtype), w.dtype), ref, w.dtype, w.name)
    else:
        dec.run_small(w, partition=part)


@pytest.mark.parametrize("i", range(48))
def test_random_prefill(i):
    w = _prefill_case(i)
    spf.run_small(w)                # fused and two-call paths, bitwise, plus the oracle


@pytest.mark.parametrize("i", range(24))
def test_random_fp8(i):
    rng = np.random.default_rng(9000 + i)
    ks, vs = (float(x) for x in rng.choice([0.004, 0.0125, 0.02, 0.1, 1.0], size=2))
    if i % 2 == 0:
        w, part, _ = _decode_case(100 + i)
        if w.dtype != "bf16":
            w = wl.custom_decode(w.context_lens.tolist(), block_size=w.block_size, num_q_heads=w.num_q_heads,
                                 num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, dtype="bf16",
                                 seed=9000 + i, name=f"random-decode-fp8-{i}")
        fp8.run_decode_fp8(wl.with_fp8_cache(w, ks, vs), part)
    else:
        spf.run_small(wl.with_fp8_cache(_prefill_case(100 + i), ks, vs), fp8=True)
