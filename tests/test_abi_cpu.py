"""Host-only checks of the C ABI: the library loads, exports every function
include/pa.h declares, and rejects bad arguments with the documented status
codes before touching the GPU (no kernel is ever launched here)."""
import ctypes
import os
import subprocess

import pytest

from paged_kv_cache_66_amd import binding

# pa_status codes, fixed by include/pa.h (test_status_codes_match_header)
OK, NULL, SHAPE, UNSUP, WS, HIP, ALIGN = 0, 1, 2, 3, 4, 5, 6
F32, BF16 = 0, 1
A = 1 << 20  # a 16-byte aligned fake device address: never dereferenced on these paths


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from paged_kv_cache_66_amd import build
        build.build()
    return binding.load()


def test_exports_every_header_symbol(lib):
    names = binding.header_symbols()
    assert set(names) == {"pa_status_string", "pa_version", "pa_store_kvcache",
                          "pa_decode_workspace_size", "pa_decode", "pa_store_decode",
                          "pa_prefill_varlen", "pa_store_kvcache_fp8", "pa_decode_fp8",
                          "pa_store_decode_fp8", "pa_prefill_varlen_fp8", "pa_store_prefill",
                          "pa_store_prefill_fp8", "pa_store_decode_noalloc"}
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_codes_match_header(lib):
    import re
    with open(binding.HEADER) as f:
        text = f.read()
    enum = re.search(r"typedef enum pa_status \{(.*?)\} pa_status;", text, re.S).group(1)
    codes = {m.group(1): int(m.group(2)) for m in re.finditer(r"(PA_\w+)\s*=\s*(\d+)", enum)}
    assert codes == {"PA_OK": OK, "PA_ERR_NULL": NULL, "PA_ERR_SHAPE": SHAPE,
                     "PA_ERR_UNSUPPORTED": UNSUP, "PA_ERR_WORKSPACE": WS, "PA_ERR_HIP": HIP,
                     "PA_ERR_ALIGN": ALIGN}
    assert {v: k for k, v in codes.items()} == binding.STATUS


def test_status_strings(lib):
    expect = {OK: b"ok", NULL: b"null", SHAPE: b"size", UNSUP: b"unsupported", WS: b"workspace",
              HIP: b"HIP", ALIGN: b"aligned"}
    for code, word in expect.items():
        assert word in lib.pa_status_string(code), code
    assert b"unknown" in lib.pa_status_string(99)
    assert b"unknown" in lib.pa_status_string(-1)
    assert b"gfx950" in lib.pa_version()


def test_library_built_from_this_tree(lib):
    """pa_version() carries the SHA-256 of the sources the library was built
    from; it must be this tree's."""
    from paged_kv_cache_66_amd import srchash
    got = binding.library_source_sha256()
    assert len(got) == 64 and got == srchash.source_sha256(), (got, srchash.source_sha256())
    assert binding.check_source_hash() == got
    files = srchash.source_files()
    assert files[0] == "include/pa.h" and files == sorted(files)
    assert any(f.endswith("decode.hip") for f in files) and any(f.endswith("pa_api.cpp") for f in files)


def store(lib, **kw):
    a = dict(key=A, ks=128, value=A, vs=128, kc=A, vc=A, slots=A, t=4, n=32, bs=16, hkv=2, d=64,
             dtype=F32)
    a.update(kw)
    return lib.pa_store_kvcache(a["key"], a["ks"], a["value"], a["vs"], a["kc"], a["vc"], a["slots"],
                                a["t"], a["n"], a["bs"], a["hkv"], a["d"], a["dtype"], None)


def test_store_validation(lib):
    assert store(lib, t=0, key=None, value=None, slots=None) == OK  # no-op
    assert store(lib, kc=None) == NULL
    assert store(lib, slots=None) == NULL
    assert store(lib, t=-1) == SHAPE
    assert store(lib, d=96) == UNSUP
    assert store(lib, bs=24) == UNSUP
    assert store(lib, bs=2048) == UNSUP
    assert store(lib, dtype=7) == UNSUP
    assert store(lib, n=0) == SHAPE
    assert store(lib, ks=100) == SHAPE          # stride shorter than a row
    assert store(lib, ks=130) == ALIGN          # 520-byte rows are not 16-byte multiples
    assert store(lib, key=A + 4) == ALIGN
    assert store(lib, kc=A + 8) == ALIGN
    assert store(lib, n=1 << 28, bs=1024) == SHAPE  # slots would overflow int32


def decode(lib, **kw):
    a = dict(out=A, q=A, qs=256, kc=A, vc=A, bt=A, w=4, ctx=A, b=4, hq=4, hkv=2, d=64, bs=16, n=32,
             scale=0.125, part=0, dtype=F32, ws=None, wsn=0)
    a.update(kw)
    return lib.pa_decode(a["out"], a["q"], a["qs"], a["kc"], a["vc"], a["bt"], a["w"], a["ctx"], a["b"],
                         a["hq"], a["hkv"], a["d"], a["bs"], a["n"], a["scale"], a["part"], a["dtype"],
                         a["ws"], a["wsn"], None)


def test_decode_validation(lib):
    assert decode(lib, b=0, out=None, q=None) == OK
    assert decode(lib, out=None) == NULL
    assert decode(lib, bt=None) == NULL
    assert decode(lib, hq=3) == SHAPE
    assert decode(lib, hq=6, hkv=2) == UNSUP     # group size 3
    assert decode(lib, hq=64, hkv=2) == UNSUP    # group size 32
    assert decode(lib, d=80) == UNSUP
    assert decode(lib, bs=12) == UNSUP
    assert decode(lib, w=0) == SHAPE
    assert decode(lib, qs=100) == SHAPE
    assert decode(lib, q=A + 4) == ALIGN
    assert decode(lib, part=100) == UNSUP
    assert decode(lib, part=8192) == UNSUP
    assert decode(lib, part=4096, hq=16, hkv=2) == UNSUP  # 8 * 4096 scores exceed LDS
    assert decode(lib, scale=float("inf")) == SHAPE
    assert decode(lib, scale=0.0) == SHAPE
    assert decode(lib, scale=-0.5) == SHAPE
    # W * bs = 64 fits the default partition: single pass, no workspace needed
    assert lib.pa_decode_workspace_size(4, 4, 2, 64, 16, 4, 0) == 0
    # W * bs = 2048 over a grid of 8 (sequence, kv head) pairs: the default
    # cuts it into 64-token partitions (about 512 workgroups): 32 partials
    need = lib.pa_decode_workspace_size(4, 4, 2, 64, 16, 128, 0)
    assert need == 4 * 4 * 32 * (64 + 2) * 4
    # an explicit partition of 512 -> 4 partials
    assert lib.pa_decode_workspace_size(4, 4, 2, 64, 16, 128, 512) == 4 * 4 * 4 * (64 + 2) * 4
    assert lib.pa_decode_workspace_size(4, 4, 3, 64, 16, 128, 0) == 0  # invalid group
    assert decode(lib, w=128) == WS
    assert decode(lib, w=128, ws=A, wsn=need - 1) == WS
    assert decode(lib, w=128, ws=A + 4, wsn=need) == ALIGN
    assert lib.pa_decode_workspace_size(4, 4, 2, 64, 16, 4, 64) == 0  # one partition of 64


def store_decode(lib, **kw):
    a = dict(out=A, q=A, qs=256, key=A, ks=128, value=A, vs=128, slots=A, kc=A, vc=A, bt=A, w=4, ctx=A,
             b=4, hq=4, hkv=2, d=64, bs=16, n=32, scale=0.125, part=0, dtype=F32, ws=None, wsn=0)
    a.update(kw)
    return lib.pa_store_decode(a["out"], a["q"], a["qs"], a["key"], a["ks"], a["value"], a["vs"],
                               a["slots"], a["kc"], a["vc"], a["bt"], a["w"], a["ctx"], a["b"], a["hq"],
                               a["hkv"], a["d"], a["bs"], a["n"], a["scale"], a["part"], a["dtype"],
                               a["ws"], a["wsn"], None)


def test_store_decode_validation(lib):
    assert store_decode(lib, b=0, out=None, key=None) == OK
    assert store_decode(lib, key=None) == NULL
    assert store_decode(lib, slots=None) == NULL
    assert store_decode(lib, out=None) == NULL
    assert store_decode(lib, ks=100) == SHAPE
    assert store_decode(lib, vs=130) == ALIGN
    assert store_decode(lib, value=A + 4) == ALIGN
    assert store_decode(lib, hq=6, hkv=2) == UNSUP
    assert store_decode(lib, w=128) == WS


def prefill(lib, **kw):
    a = dict(out=A, q=A, qs=512, tq=8, k=A, ks=0, v=A, vs=0, cuq=A, cuk=A, mq=8, mk=8, bt=A, w=4, b=1,
             hq=4, hkv=2, d=128, bs=16, n=32, scale=0.1, dtype=BF16)
    a.update(kw)
    return lib.pa_prefill_varlen(a["out"], a["q"], a["qs"], a["tq"], a["k"], a["ks"], a["v"], a["vs"],
                                 a["cuq"], a["cuk"], a["mq"], a["mk"], a["bt"], a["w"], a["b"], a["hq"],
                                 a["hkv"], a["d"], a["bs"], a["n"], a["scale"], a["dtype"], None)


def test_prefill_validation(lib):
    assert prefill(lib, b=0) == OK
    assert prefill(lib, tq=0) == OK
    assert prefill(lib, dtype=F32) == UNSUP      # only bf16 MFMA path is built
    assert prefill(lib, cuq=None) == NULL
    assert prefill(lib, hq=5) == SHAPE
    assert prefill(lib, d=32) == UNSUP
    assert prefill(lib, qs=256) == SHAPE
    assert prefill(lib, out=A + 2) == ALIGN
    assert prefill(lib, mq=-1) == SHAPE
    assert prefill(lib, scale=0.0) == SHAPE
    assert prefill(lib, scale=float("nan")) == SHAPE
    # paged mode: the caches are contiguous, a row stride must say so
    assert prefill(lib, ks=300) == SHAPE
    assert prefill(lib, bs=24) == UNSUP
    # packed mode (no block table): row strides required, block size ignored
    packed = dict(bt=None, w=0, bs=0, n=0, ks=256, vs=256)
    assert prefill(lib, **{**packed, "tq": 0}) == OK
    assert prefill(lib, **{**packed, "ks": 0}) == SHAPE
    assert prefill(lib, **{**packed, "vs": 100}) == SHAPE
    assert prefill(lib, **{**packed, "ks": 260}) == ALIGN
    assert prefill(lib, **{**packed, "k": A + 8}) == ALIGN
    assert prefill(lib, **{**packed, "ks": 1 << 26}) == SHAPE


# ---- fp8 (E4M3) cache entry points: bf16 rows, one-byte caches, two scales ----

def store_fp8(lib, **kw):
    a = dict(key=A, ks=128, value=A, vs=128, kc=A, vc=A, slots=A, t=4, n=32, bs=16, hkv=2, d=64,
             kscale=0.02, vscale=0.03, dtype=BF16)
    a.update(kw)
    return lib.pa_store_kvcache_fp8(a["key"], a["ks"], a["value"], a["vs"], a["kc"], a["vc"], a["slots"],
                                    a["t"], a["n"], a["bs"], a["hkv"], a["d"], a["kscale"], a["vscale"],
                                    a["dtype"], None)


def test_store_fp8_validation(lib):
    assert store_fp8(lib, t=0, key=None, value=None, slots=None) == OK
    assert store_fp8(lib, dtype=F32) == UNSUP       # bf16 rows only
    assert store_fp8(lib, kscale=0.0) == SHAPE
    assert store_fp8(lib, vscale=float("inf")) == SHAPE
    assert store_fp8(lib, kscale=-1.0) == SHAPE
    assert store_fp8(lib, kc=None) == NULL
    assert store_fp8(lib, slots=None) == NULL
    assert store_fp8(lib, d=96) == UNSUP
    assert store_fp8(lib, ks=100) == SHAPE
    assert store_fp8(lib, ks=132) == ALIGN          # 264-byte bf16 rows
    assert store_fp8(lib, vc=A + 8) == ALIGN


def decode_fp8(lib, fused=False, **kw):
    a = dict(out=A, q=A, qs=256, key=A, ks=128, value=A, vs=128, slots=A, kc=A, vc=A, bt=A, w=4, ctx=A,
             b=4, hq=4, hkv=2, d=64, bs=16, n=32, scale=0.125, kscale=0.02, vscale=0.03, part=0,
             dtype=BF16, ws=None, wsn=0)
    a.update(kw)
    if fused:
        return lib.pa_store_decode_fp8(a["out"], a["q"], a["qs"], a["key"], a["ks"], a["value"], a["vs"],
                                       a["slots"], a["kc"], a["vc"], a["bt"], a["w"], a["ctx"], a["b"],
                                       a["hq"], a["hkv"], a["d"], a["bs"], a["n"], a["scale"], a["kscale"],
                                       a["vscale"], a["part"], a["dtype"], a["ws"], a["wsn"], None)
    return lib.pa_decode_fp8(a["out"], a["q"], a["qs"], a["kc"], a["vc"], a["bt"], a["w"], a["ctx"], a["b"],
                             a["hq"], a["hkv"], a["d"], a["bs"], a["n"], a["scale"], a["kscale"],
                             a["vscale"], a["part"], a["dtype"], a["ws"], a["wsn"], None)


@pytest.mark.parametrize("fused", [False, True])
def test_decode_fp8_validation(lib, fused):
    assert decode_fp8(lib, fused, b=0, out=None, q=None) == OK
    assert decode_fp8(lib, fused, dtype=F32) == UNSUP
    assert decode_fp8(lib, fused, kscale=0.0) == SHAPE
    assert decode_fp8(lib, fused, vscale=float("nan")) == SHAPE
    assert decode_fp8(lib, fused, scale=0.0) == SHAPE
    assert decode_fp8(lib, fused, out=None) == NULL
    assert decode_fp8(lib, fused, hq=6, hkv=2) == UNSUP
    assert decode_fp8(lib, fused, qs=100) == SHAPE
    assert decode_fp8(lib, fused, w=128) == WS
    if fused:
        assert decode_fp8(lib, fused, key=None) == NULL
        assert decode_fp8(lib, fused, vs=130) == ALIGN


def prefill_fp8(lib, **kw):
    a = dict(out=A, q=A, qs=512, tq=8, kc=A, vc=A, cuq=A, cuk=A, mq=8, mk=8, bt=A, w=4, b=1,
             hq=4, hkv=2, d=128, bs=16, n=32, scale=0.1, kscale=0.02, vscale=0.03, dtype=BF16)
    a.update(kw)
    return lib.pa_prefill_varlen_fp8(a["out"], a["q"], a["qs"], a["tq"], a["kc"], a["vc"], a["cuq"],
                                     a["cuk"], a["mq"], a["mk"], a["bt"], a["w"], a["b"], a["hq"],
                                     a["hkv"], a["d"], a["bs"], a["n"], a["scale"], a["kscale"],
                                     a["vscale"], a["dtype"], None)


def test_prefill_fp8_validation(lib):
    assert prefill_fp8(lib, b=0) == OK
    assert prefill_fp8(lib, bt=None) == NULL    # fp8 data lives only in the paged caches
    assert prefill_fp8(lib, dtype=F32) == UNSUP
    assert prefill_fp8(lib, kscale=0.0) == SHAPE
    assert prefill_fp8(lib, vscale=-2.0) == SHAPE
    assert prefill_fp8(lib, cuq=None) == NULL
    assert prefill_fp8(lib, d=32) == UNSUP
    assert prefill_fp8(lib, bs=24) == UNSUP
    assert prefill_fp8(lib, kc=A + 8) == ALIGN


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.import_module("paged_kv_cache_66_amd.binding")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            mod.load(str(tmp_path / "missing.so"))
    finally:
        mod._lib = saved


# ---- fused scatter + prefill: paged mode only, new rows packed like q ----

def store_prefill(lib, fp8=False, **kw):
    a = dict(out=A, q=A, qs=512, tq=8, key=A, ks=256, value=A, vs=256, slots=A, kc=A, vc=A, cuq=A, cuk=A,
             mq=8, mk=8, bt=A, w=4, b=1, hq=4, hkv=2, d=128, bs=16, n=32, scale=0.1, kscale=0.02,
             vscale=0.03, dtype=BF16)
    a.update(kw)
    head = (a["out"], a["q"], a["qs"], a["tq"], a["key"], a["ks"], a["value"], a["vs"], a["slots"], a["kc"],
            a["vc"], a["cuq"], a["cuk"], a["mq"], a["mk"], a["bt"], a["w"], a["b"], a["hq"], a["hkv"], a["d"],
            a["bs"], a["n"], a["scale"])
    if fp8:
        return lib.pa_store_prefill_fp8(*head, a["kscale"], a["vscale"], a["dtype"], None)
    return lib.pa_store_prefill(*head, a["dtype"], None)


@pytest.mark.parametrize("fp8", [False, True])
def test_store_prefill_validation(lib, fp8):
    assert store_prefill(lib, fp8, b=0) == OK
    assert store_prefill(lib, fp8, tq=0) == OK
    assert store_prefill(lib, fp8, dtype=F32) == UNSUP
    assert store_prefill(lib, fp8, bt=None) == NULL      # the fused call is paged only
    assert store_prefill(lib, fp8, slots=None) == NULL
    assert store_prefill(lib, fp8, slots=None, key=None, value=None, tq=0) == OK  # empty step
    assert store_prefill(lib, fp8, key=None) == NULL
    assert store_prefill(lib, fp8, value=None) == NULL
    assert store_prefill(lib, fp8, ks=100) == SHAPE       # stride shorter than a K row
    assert store_prefill(lib, fp8, vs=260) == ALIGN       # 520-byte rows
    assert store_prefill(lib, fp8, key=A + 2) == ALIGN
    assert store_prefill(lib, fp8, ks=1 << 24) == SHAPE     # 64-row tiles use 32-bit offsets
    assert store_prefill(lib, fp8, hq=5) == SHAPE
    assert store_prefill(lib, fp8, d=32) == UNSUP
    assert store_prefill(lib, fp8, bs=24) == UNSUP
    assert store_prefill(lib, fp8, scale=0.0) == SHAPE
    if fp8:
        assert store_prefill(lib, fp8, kscale=0.0) == SHAPE
        assert store_prefill(lib, fp8, vscale=float("inf")) == SHAPE


def test_noalloc_rejects_workspace_beyond_the_array(lib):
    """pa_store_decode_noalloc refuses, before any HIP call or launch, a call
    whose split-K workspace exceeds the fixed array (64 MiB), and validates
    like pa_store_decode otherwise."""
    import re
    with open(binding.HEADER) as f:
        cap = eval(re.search(r"#define PA_NOALLOC_WORKSPACE_BYTES \((.*?)\)", f.read()).group(1).replace("u", ""))
    assert cap == 64 << 20

    def call(**kw):
        a = dict(b=512, hq=32, hkv=8, d=128, bs=16, w=2048, n=300000, part=0, dtype=BF16, out=A, slots=A)
        a.update(kw)
        return lib.pa_store_decode_noalloc(a["out"], A, a["hq"] * a["d"], A, a["hkv"] * a["d"], A,
                                           a["hkv"] * a["d"], a["slots"], A, A, A, a["w"], A, a["b"], a["hq"],
                                           a["hkv"], a["d"], a["bs"], a["n"], 0.088, a["part"], a["dtype"], None)
    # the 8B-shaped batch at block size 16 needs 272 MiB of partials: refused
    need = lib.pa_decode_workspace_size(512, 32, 8, 128, 16, 2048, 0)
    assert need > cap
    assert call() == WS
    # half the batch in 4096-token partitions needs 34 MiB: it passes the size
    # check and fails only on what follows (an unsupported group size here,
    # so nothing runs)
    assert lib.pa_decode_workspace_size(256, 32, 8, 128, 16, 2048, 4096) <= cap
    assert call(b=256, hq=24, part=4096) == UNSUP
    assert call(out=None, b=4, w=4) == NULL
    assert call(slots=None, b=4, w=4) == NULL
    assert call(b=4, w=4, d=96) == UNSUP
