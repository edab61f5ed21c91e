"""Thin Python binding over the C ABI in ``libpa.so`` (see include/pa.h).

Argument marshalling only: tensors are checked for device, dtype and shape,
their data pointers and the current torch stream are handed to the C entry
point of the same name, and a non-zero status raises :class:`PaError`. Every
step of the computation runs in the HIP kernels; there is no fallback. If the
library is missing the first call raises instead of computing anything.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "pa.h")

PA_F32, PA_BF16 = 0, 1
STATUS = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED",
          4: "PA_ERR_WORKSPACE", 5: "PA_ERR_HIP", 6: "PA_ERR_ALIGN"}


class PaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


_lib = None

_i32, _i64, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

_SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_version": (ctypes.c_char_p, []),
    "pa_store_kvcache": (ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                        _i32, ctypes.c_int, _vp]),
    "pa_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                 _i32, _i32, _f32, _i32, ctypes.c_int, _vp, _sz, _vp]),
    "pa_store_decode": (ctypes.c_int, [_vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i32,
                                       _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                       ctypes.c_int, _vp, _sz, _vp]),
    "pa_store_decode_noalloc": (ctypes.c_int, [_vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp,
                                               _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                               ctypes.c_int, _vp]),
    "pa_prefill_varlen": (ctypes.c_int, [_vp, _vp, _i64, _i32, _vp, _i64, _vp, _i64, _vp, _vp, _i32,
                                         _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                         _f32, ctypes.c_int, _vp]),
    "pa_store_kvcache_fp8": (ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                            _i32, _f32, _f32, ctypes.c_int, _vp]),
    "pa_decode_fp8": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                     _i32, _i32, _f32, _f32, _f32, _i32, ctypes.c_int, _vp, _sz, _vp]),
    "pa_store_decode_fp8": (ctypes.c_int, [_vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp,
                                           _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _f32,
                                           _f32, _i32, ctypes.c_int, _vp, _sz, _vp]),
    "pa_prefill_varlen_fp8": (ctypes.c_int, [_vp, _vp, _i64, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _vp,
                                             _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _f32,
                                             _f32, ctypes.c_int, _vp]),
    "pa_store_prefill": (ctypes.c_int, [_vp, _vp, _i64, _i32, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp,
                                        _vp, _i32, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                        _f32, ctypes.c_int, _vp]),
    "pa_store_prefill_fp8": (ctypes.c_int, [_vp, _vp, _i64, _i32, _vp, _i64, _vp, _i64, _vp, _vp, _vp,
                                            _vp, _vp, _i32, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                            _i32, _f32, _f32, _f32, ctypes.c_int, _vp]),
}


def header_symbols(path: str = HEADER) -> list[str]:
    """Names of the functions include/pa.h declares."""
    with open(path) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(pa_\w+)\s*\(", text, re.M)))


def load(path: str = LIB_PATH):
    """Load (once) and return the ctypes handle of libpa.so."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run python -m paged_kv_cache_66_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def version() -> str:
    """pa_version(): package version, target and src-sha256 of the library."""
    return load().pa_version().decode()


def library_source_sha256() -> str:
    """The source hash baked into the loaded library (after "src-sha256:")."""
    v = version()
    key = "src-sha256:"
    return v.split(key, 1)[1].strip() if key in v else ""


def check_source_hash() -> str:
    """Raise unless the loaded library was built from the sources in this
    tree (include/pa.h and csrc/, hashed as srchash.source_sha256 does);
    returns the hash."""
    from .srchash import source_sha256
    want = source_sha256()
    got = library_source_sha256()
    if got != want:
        raise RuntimeError(f"libpa.so was built from other sources (src-sha256:{got}) than this tree "
                           f"({want}); rebuild with python -m paged_kv_cache_66_amd.build")
    return got


def _check(fn: str, status: int):
    if status != 0:
        msg = load().pa_status_string(status).decode()
        raise PaError(fn, status, msg)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _require(cond: bool, what: str):
    if not cond:
        raise ValueError(what)


def _rows(t, name: str):
    """(pointer, row stride in elements) of a [T, heads, head_dim] tensor
    whose inner two dimensions are contiguous."""
    _require(t.dim() == 3, f"{name} must be 3-D")
    _require(t.stride(2) == 1 and t.stride(1) == t.shape[2], f"{name}: inner dims must be contiguous")
    return t.data_ptr(), t.stride(0)


def _int32(t, name):
    import torch
    _require(t.dtype == torch.int32, f"{name} must be int32")
    _require(t.is_contiguous(), f"{name} must be contiguous")


def _cache_dims(k_cache, v_cache):
    _require(k_cache.dim() == 4 and k_cache.is_contiguous(), "k_cache must be contiguous [N, bs, H_kv, D]")
    _require(v_cache.shape == k_cache.shape and v_cache.is_contiguous(), "v_cache must match k_cache")
    _require(v_cache.dtype == k_cache.dtype, "k_cache and v_cache dtypes differ")
    return tuple(int(x) for x in k_cache.shape)


def _fp8_cache_dims(k_cache, v_cache):
    """Dims of E4M3 caches held as uint8 (or torch.float8_e4m3fn) tensors."""
    import torch
    _require(k_cache.dtype in (torch.uint8, torch.float8_e4m3fn), "fp8 caches must be uint8 / float8_e4m3fn")
    return _cache_dims(k_cache, v_cache)


def _workspace(workspace, b, hq, hkv, d, bs, w, partition_size, device):
    import torch
    need = pa_decode_workspace_size(b, hq, hkv, d, bs, w, partition_size) if b > 0 else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    wp = workspace.data_ptr() if workspace is not None else None
    wn = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return wp, wn


def pa_store_kvcache(key, value, k_cache, v_cache, slot_mapping) -> None:
    """Scatter key/value rows [T, H_kv, D] into the caches at slot_mapping."""
    lib = load()
    n, bs, hkv, d = _cache_dims(k_cache, v_cache)
    _int32(slot_mapping, "slot_mapping")
    t = int(slot_mapping.shape[0])
    kp, ks = _rows(key, "key")
    vp, vs = _rows(value, "value")
    _require(key.shape[0] == t and value.shape[0] == t, "key/value rows != len(slot_mapping)")
    _require(tuple(key.shape[1:]) == (hkv, d) and tuple(value.shape[1:]) == (hkv, d), "key/value head shape")
    _require(key.dtype == k_cache.dtype == value.dtype, "dtype mismatch")
    st = lib.pa_store_kvcache(kp, ks, vp, vs, k_cache.data_ptr(), v_cache.data_ptr(),
                              slot_mapping.data_ptr(), t, n, bs, hkv, d, _dtype_code(k_cache),
                              _stream(k_cache))
    _check("pa_store_kvcache", st)


def pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             max_blocks_per_seq, partition_size=0) -> int:
    return int(load().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                block_size, max_blocks_per_seq, partition_size))


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out=None, workspace=None,
              partition_size=0):
    """Paged GQA decode. q [B, H_q, D]; returns out [B, H_q, D]."""
    import torch
    lib = load()
    n, bs, hkv, d = _cache_dims(k_cache, v_cache)
    _int32(block_tables, "block_tables")
    _int32(context_lens, "context_lens")
    qp, qs = _rows(q, "q")
    b, hq = int(q.shape[0]), int(q.shape[1])
    _require(q.shape[2] == d and q.dtype == k_cache.dtype, "q shape/dtype")
    _require(block_tables.dim() == 2 and block_tables.shape[0] == b, "block_tables must be [B, W]")
    _require(context_lens.shape == (b,), "context_lens must be [B]")
    w = int(block_tables.shape[1])
    if out is None:
        out = torch.empty((b, hq, d), dtype=q.dtype, device=q.device)
    _require(out.is_contiguous() and tuple(out.shape) == (b, hq, d) and out.dtype == q.dtype, "out")
    wp, wn = _workspace(workspace, b, hq, hkv, d, bs, w, partition_size, q.device)
    st = lib.pa_decode(out.data_ptr(), qp, qs, k_cache.data_ptr(), v_cache.data_ptr(),
                       block_tables.data_ptr(), w, context_lens.data_ptr(), b, hq, hkv, d, bs, n,
                       float(scale), int(partition_size), _dtype_code(q), wp, wn, _stream(q))
    _check("pa_decode", st)
    return out


def pa_store_decode(q, key, value, slot_mapping, k_cache, v_cache, block_tables, context_lens, scale,
                    out=None, workspace=None, partition_size=0):
    """pa_store_kvcache + pa_decode in one launch. q [B, H_q, D]; key/value
    [B, H_kv, D]; slot_mapping[b] is -1 or the slot of position
    context_lens[b] - 1."""
    import torch
    lib = load()
    n, bs, hkv, d = _cache_dims(k_cache, v_cache)
    _int32(block_tables, "block_tables")
    _int32(context_lens, "context_lens")
    _int32(slot_mapping, "slot_mapping")
    qp, qs = _rows(q, "q")
    kp, ks = _rows(key, "key")
    vp, vs = _rows(value, "value")
    b, hq = int(q.shape[0]), int(q.shape[1])
    _require(q.shape[2] == d and q.dtype == k_cache.dtype, "q shape/dtype")
    _require(tuple(key.shape) == (b, hkv, d) and tuple(value.shape) == (b, hkv, d), "key/value shape")
    _require(key.dtype == value.dtype == k_cache.dtype, "key/value dtype")
    _require(slot_mapping.shape == (b,), "slot_mapping must be [B]")
    _require(block_tables.dim() == 2 and block_tables.shape[0] == b, "block_tables must be [B, W]")
    _require(context_lens.shape == (b,), "context_lens must be [B]")
    w = int(block_tables.shape[1])
    if out is None:
        out = torch.empty((b, hq, d), dtype=q.dtype, device=q.device)
    _require(out.is_contiguous() and tuple(out.shape) == (b, hq, d) and out.dtype == q.dtype, "out")
    wp, wn = _workspace(workspace, b, hq, hkv, d, bs, w, partition_size, q.device)
    st = lib.pa_store_decode(out.data_ptr(), qp, qs, kp, ks, vp, vs, slot_mapping.data_ptr(),
                             k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), w,
                             context_lens.data_ptr(), b, hq, hkv, d, bs, n, float(scale),
                             int(partition_size), _dtype_code(q), wp, wn, _stream(q))
    _check("pa_store_decode", st)
    return out


def pa_store_decode_noalloc(q, key, value, slot_mapping, k_cache, v_cache, block_tables, context_lens,
                            scale, out, partition_size=0):
    """pa_store_decode with the split-K workspace in the library's fixed
    device array (PA_NOALLOC_WORKSPACE_BYTES per GPU): nothing is allocated,
    so ``out`` [B, H_q, D] must be given."""
    lib = load()
    n, bs, hkv, d = _cache_dims(k_cache, v_cache)
    _int32(block_tables, "block_tables")
    _int32(context_lens, "context_lens")
    _int32(slot_mapping, "slot_mapping")
    qp, qs = _rows(q, "q")
    kp, ks = _rows(key, "key")
    vp, vs = _rows(value, "value")
    b, hq = int(q.shape[0]), int(q.shape[1])
    _require(q.shape[2] == d and q.dtype == k_cache.dtype, "q shape/dtype")
    _require(tuple(key.shape) == (b, hkv, d) and tuple(value.shape) == (b, hkv, d), "key/value shape")
    _require(key.dtype == value.dtype == k_cache.dtype, "key/value dtype")
    _require(slot_mapping.shape == (b,), "slot_mapping must be [B]")
    _require(block_tables.dim() == 2 and block_tables.shape[0] == b, "block_tables must be [B, W]")
    _require(context_lens.shape == (b,), "context_lens must be [B]")
    _require(out is not None and out.is_contiguous() and tuple(out.shape) == (b, hq, d) and
             out.dtype == q.dtype, "out [B, H_q, D] must be given (this call allocates nothing)")
    st = lib.pa_store_decode_noalloc(out.data_ptr(), qp, qs, kp, ks, vp, vs, slot_mapping.data_ptr(),
                                     k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                                     int(block_tables.shape[1]), context_lens.data_ptr(), b, hq, hkv, d, bs, n,
                                     float(scale), int(partition_size), _dtype_code(q), _stream(q))
    _check("pa_store_decode_noalloc", st)
    return out


def pa_prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                      block_tables, scale, out=None):
    """Packed varlen causal prefill. q [Tq, H_q, D].

    With block_tables ([B, W] int32) k and v are the paged caches
    [N, bs, H_kv, D]; with block_tables=None they are packed [Tk, H_kv, D]
    (row-strided views are fine) and key t of sequence i is row
    cu_seqlens_k[i] + t."""
    import torch
    lib = load()
    _int32(cu_seqlens_q, "cu_seqlens_q")
    _int32(cu_seqlens_k, "cu_seqlens_k")
    qp, qs = _rows(q, "q")
    tq, hq = int(q.shape[0]), int(q.shape[1])
    bsq = int(cu_seqlens_q.shape[0]) - 1
    _require(cu_seqlens_k.shape == cu_seqlens_q.shape, "cu_seqlens_k must match cu_seqlens_q")
    if block_tables is not None:
        n, bs, hkv, d = _cache_dims(k, v)
        _int32(block_tables, "block_tables")
        _require(block_tables.dim() == 2 and block_tables.shape[0] == bsq, "block_tables must be [B, W]")
        bt_ptr, w = block_tables.data_ptr(), int(block_tables.shape[1])
        kp, ks, vp, vs = k.data_ptr(), 0, v.data_ptr(), 0
    else:
        kp, ks = _rows(k, "k")
        vp, vs = _rows(v, "v")
        hkv, d = int(k.shape[1]), int(k.shape[2])
        _require(tuple(v.shape[1:]) == (hkv, d) and v.dtype == k.dtype, "k/v shapes")
        n, bs, bt_ptr, w = 0, 0, None, 0
    _require(q.shape[2] == d and q.dtype == k.dtype, "q shape/dtype")
    if out is None:
        out = torch.empty((tq, hq, d), dtype=q.dtype, device=q.device)
    _require(out.is_contiguous() and tuple(out.shape) == (tq, hq, d) and out.dtype == q.dtype, "out")
    st = lib.pa_prefill_varlen(out.data_ptr(), qp, qs, tq, kp, ks, vp, vs, cu_seqlens_q.data_ptr(),
                               cu_seqlens_k.data_ptr(), int(max_seqlen_q), int(max_seqlen_k), bt_ptr, w,
                               bsq, hq, hkv, d, bs, n, float(scale), _dtype_code(q), _stream(q))
    _check("pa_prefill_varlen", st)
    return out


# ---------------------------------------------------------------------------
# E4M3 (fp8) caches: one-byte codes with a per-tensor scale for K and for V;
# queries, new key/value rows and outputs are bf16.
# ---------------------------------------------------------------------------

def pa_store_kvcache_fp8(key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale) -> None:
    """Quantise bf16 key/value rows [T, H_kv, D] (x / scale, nearest E4M3
    code) and scatter them into the fp8 caches at slot_mapping."""
    import torch
    lib = load()
    n, bs, hkv, d = _fp8_cache_dims(k_cache, v_cache)
    _int32(slot_mapping, "slot_mapping")
    t = int(slot_mapping.shape[0])
    kp, ks = _rows(key, "key")
    vp, vs = _rows(value, "value")
    _require(key.shape[0] == t and value.shape[0] == t, "key/value rows != len(slot_mapping)")
    _require(tuple(key.shape[1:]) == (hkv, d) and tuple(value.shape[1:]) == (hkv, d), "key/value head shape")
    _require(key.dtype == value.dtype == torch.bfloat16, "key/value must be bf16")
    st = lib.pa_store_kvcache_fp8(kp, ks, vp, vs, k_cache.data_ptr(), v_cache.data_ptr(),
                                  slot_mapping.data_ptr(), t, n, bs, hkv, d, float(k_scale),
                                  float(v_scale), PA_BF16, _stream(k_cache))
    _check("pa_store_kvcache_fp8", st)


def pa_decode_fp8(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale, out=None,
                  workspace=None, partition_size=0):
    """Paged GQA decode over fp8 caches. q [B, H_q, D] bf16; returns bf16 out."""
    import torch
    lib = load()
    n, bs, hkv, d = _fp8_cache_dims(k_cache, v_cache)
    _int32(block_tables, "block_tables")
    _int32(context_lens, "context_lens")
    qp, qs = _rows(q, "q")
    b, hq = int(q.shape[0]), int(q.shape[1])
    _require(q.shape[2] == d and q.dtype == torch.bfloat16, "q shape/dtype")
    _require(block_tables.dim() == 2 and block_tables.shape[0] == b, "block_tables must be [B, W]")
    _require(context_lens.shape == (b,), "context_lens must be [B]")
    w = int(block_tables.shape[1])
    if out is None:
        out = torch.empty((b, hq, d), dtype=q.dtype, device=q.device)
    _require(out.is_contiguous() and tuple(out.shape) == (b, hq, d) and out.dtype == q.dtype, "out")
    wp, wn = _workspace(workspace, b, hq, hkv, d, bs, w, partition_size, q.device)
    st = lib.pa_decode_fp8(out.data_ptr(), qp, qs, k_cache.data_ptr(), v_cache.data_ptr(),
                           block_tables.data_ptr(), w, context_lens.data_ptr(), b, hq, hkv, d, bs, n,
                           float(scale), float(k_scale), float(v_scale), int(partition_size), PA_BF16,
                           wp, wn, _stream(q))
    _check("pa_decode_fp8", st)
    return out


def pa_store_decode_fp8(q, key, value, slot_mapping, k_cache, v_cache, block_tables, context_lens,
                        scale, k_scale, v_scale, out=None, workspace=None, partition_size=0):
    """pa_store_kvcache_fp8 + pa_decode_fp8 in one launch (slot_mapping[b]
    is -1 or the slot of position context_lens[b] - 1)."""
    import torch
    lib = load()
    n, bs, hkv, d = _fp8_cache_dims(k_cache, v_cache)
    _int32(block_tables, "block_tables")
    _int32(context_lens, "context_lens")
    _int32(slot_mapping, "slot_mapping")
    qp, qs = _rows(q, "q")
    kp, ks = _rows(key, "key")
    vp, vs = _rows(value, "value")
    b, hq = int(q.shape[0]), int(q.shape[1])
    _require(q.shape[2] == d and q.dtype == torch.bfloat16, "q shape/dtype")
    _require(tuple(key.shape) == (b, hkv, d) and tuple(value.shape) == (b, hkv, d), "key/value shape")
    _require(key.dtype == value.dtype == torch.bfloat16, "key/value must be bf16")
    _require(slot_mapping.shape == (b,), "slot_mapping must be [B]")
    _require(block_tables.dim() == 2 and block_tables.shape[0] == b, "block_tables must be [B, W]")
    _require(context_lens.shape == (b,), "context_lens must be [B]")
    w = int(block_tables.shape[1])
    if out is None:
        out = torch.empty((b, hq, d), dtype=q.dtype, device=q.device)
    _require(out.is_contiguous() and tuple(out.shape) == (b, hq, d) and out.dtype == q.dtype, "out")
    wp, wn = _workspace(workspace, b, hq, hkv, d, bs, w, partition_size, q.device)
    st = lib.pa_store_decode_fp8(out.data_ptr(), qp, qs, kp, ks, vp, vs, slot_mapping.data_ptr(),
                                 k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), w,
                                 context_lens.data_ptr(), b, hq, hkv, d, bs, n, float(scale),
                                 float(k_scale), float(v_scale), int(partition_size), PA_BF16, wp, wn,
                                 _stream(q))
    _check("pa_store_decode_fp8", st)
    return out


def pa_prefill_varlen_fp8(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                          block_tables, scale, k_scale, v_scale, out=None):
    """Packed varlen causal prefill whose keys and values are read from fp8
    paged caches through block_tables. q [Tq, H_q, D] bf16."""
    import torch
    lib = load()
    _int32(cu_seqlens_q, "cu_seqlens_q")
    _int32(cu_seqlens_k, "cu_seqlens_k")
    _int32(block_tables, "block_tables")
    qp, qs = _rows(q, "q")
    tq, hq = int(q.shape[0]), int(q.shape[1])
    bsq = int(cu_seqlens_q.shape[0]) - 1
    _require(cu_seqlens_k.shape == cu_seqlens_q.shape, "cu_seqlens_k must match cu_seqlens_q")
    n, bs, hkv, d = _fp8_cache_dims(k_cache, v_cache)
    _require(block_tables.dim() == 2 and block_tables.shape[0] == bsq, "block_tables must be [B, W]")
    _require(q.shape[2] == d and q.dtype == torch.bfloat16, "q shape/dtype")
    if out is None:
        out = torch.empty((tq, hq, d), dtype=q.dtype, device=q.device)
    _require(out.is_contiguous() and tuple(out.shape) == (tq, hq, d) and out.dtype == q.dtype, "out")
    st = lib.pa_prefill_varlen_fp8(out.data_ptr(), qp, qs, tq, k_cache.data_ptr(), v_cache.data_ptr(),
                                   cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), int(max_seqlen_q),
                                   int(max_seqlen_k), block_tables.data_ptr(), int(block_tables.shape[1]),
                                   bsq, hq, hkv, d, bs, n, float(scale), float(k_scale), float(v_scale),
                                   PA_BF16, _stream(q))
    _check("pa_prefill_varlen_fp8", st)
    return out


def _store_prefill_args(q, key, value, slot_mapping, cu_seqlens_q, cu_seqlens_k, block_tables, dims, out):
    import torch
    n, bs, hkv, d = dims
    for t, name in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k"),
                    (block_tables, "block_tables"), (slot_mapping, "slot_mapping")):
        _int32(t, name)
    qp, qs = _rows(q, "q")
    kp, ks = _rows(key, "key")
    vp, vs = _rows(value, "value")
    tq, hq = int(q.shape[0]), int(q.shape[1])
    bsq = int(cu_seqlens_q.shape[0]) - 1
    _require(cu_seqlens_k.shape == cu_seqlens_q.shape, "cu_seqlens_k must match cu_seqlens_q")
    _require(block_tables.dim() == 2 and block_tables.shape[0] == bsq, "block_tables must be [B, W]")
    _require(q.shape[2] == d and q.dtype == torch.bfloat16, "q shape/dtype")
    _require(tuple(key.shape) == (tq, hkv, d) and tuple(value.shape) == (tq, hkv, d), "key/value shape")
    _require(key.dtype == value.dtype == torch.bfloat16, "key/value must be bf16")
    _require(slot_mapping.shape == (tq,), "slot_mapping must be [Tq]")
    if out is None:
        out = torch.empty((tq, hq, d), dtype=q.dtype, device=q.device)
    _require(out.is_contiguous() and tuple(out.shape) == (tq, hq, d) and out.dtype == q.dtype, "out")
    return out, [out.data_ptr(), qp, qs, tq, kp, ks, vp, vs, slot_mapping.data_ptr()], \
        [cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr()], \
        [block_tables.data_ptr(), int(block_tables.shape[1]), bsq, hq, hkv, d, bs, n]


def pa_store_prefill(q, key, value, slot_mapping, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k,
                     max_seqlen_q, max_seqlen_k, block_tables, scale, out=None):
    """pa_store_kvcache + paged pa_prefill_varlen in one launch. q [Tq, H_q, D];
    key/value [Tq, H_kv, D] are this step's rows, packed like q;
    slot_mapping[r] is the slot of query row r's position."""
    lib = load()
    dims = _cache_dims(k_cache, v_cache)
    _require(k_cache.dtype == q.dtype, "caches must be bf16 like q")
    out, a, cu, t = _store_prefill_args(q, key, value, slot_mapping, cu_seqlens_q, cu_seqlens_k,
                                        block_tables, dims, out)
    st = lib.pa_store_prefill(*a, k_cache.data_ptr(), v_cache.data_ptr(), *cu, int(max_seqlen_q),
                              int(max_seqlen_k), *t, float(scale), PA_BF16, _stream(q))
    _check("pa_store_prefill", st)
    return out


def pa_store_prefill_fp8(q, key, value, slot_mapping, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k,
                         max_seqlen_q, max_seqlen_k, block_tables, scale, k_scale, v_scale, out=None):
    """pa_store_kvcache_fp8 + pa_prefill_varlen_fp8 in one launch (same
    arguments as pa_store_prefill plus the two cache scales)."""
    lib = load()
    dims = _fp8_cache_dims(k_cache, v_cache)
    out, a, cu, t = _store_prefill_args(q, key, value, slot_mapping, cu_seqlens_q, cu_seqlens_k,
                                        block_tables, dims, out)
    st = lib.pa_store_prefill_fp8(*a, k_cache.data_ptr(), v_cache.data_ptr(), *cu, int(max_seqlen_q),
                                  int(max_seqlen_k), *t, float(scale), float(k_scale), float(v_scale),
                                  PA_BF16, _stream(q))
    _check("pa_store_prefill_fp8", st)
    return out
