"""Plain, slow, fp64 CPU oracle for paged attention over a block-table cache.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The library's product path never does, and this module imports
nothing from the library.

Every function is the textbook definition written out, with no blocking,
fusion or reordering: the paged methods reach exactly (up to rounding order)
the result of ordinary attention over a contiguous copy of each sequence's
history, because paging only changes where bytes live ("How vLLM Works":
paging is lossless bookkeeping). So each attention function first copies the
sequence's blocks, in logical order, into a contiguous buffer and then runs
softmax(scale * q K^T) V in fp64.

Storage formats: fp32 tensors are numpy float32; bf16 tensors are numpy
uint16 arrays holding the bf16 bit patterns, widened exactly to fp64 here.
An fp8 cache ("fp8e4m3") is a numpy uint8 array of E4M3 codes with one scale
per tensor; its rows widen to value(code) * scale (``oracle.fp8``), and the
queries and outputs keep the 16-bit type.

Readings of points the pages leave open (each is also listed in the design
notes of the repository):
* GQA: query head h reads kv head h // (H_q / H_kv) (contiguous groups),
  the only mapping consistent with the tensor-parallel head split on
  "From nano-vLLM to vLLM ...", section 16.3.
* decode: context_lens includes the token being decoded, which has already
  been stored ("nano-vLLM Part 2 ...", section 3.1: position 11 with
  context_lens [12]; store runs before attention in Attention.forward).
* prefill with a cached prefix: query j of a sequence with Lq queries and Lk
  visible keys sits at absolute position Lk - Lq + j and sees keys
  0 .. Lk - Lq + j (bottom-right causal alignment; "Inference Engine
  Inside nano-vLLM", "Prepare Prefill": positions = range(start, end) and
  seqlen_k = end).
* context_len == 0 gives an all-zero output row and reads nothing.
* table entries at or past ceil(context_len / block_size) are never read.
* any negative slot is skipped by the store (the pages use -1).
"""
from __future__ import annotations

import numpy as np

from . import fp8


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of stored values to float64."""
    if dtype == "bf16":
        return (np.asarray(x).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def store_kvcache(key, value, k_cache, v_cache, slot_mapping) -> None:
    """KV scatter, in place.

    For token t with slot s = slot_mapping[t] >= 0, copy key[t] into the
    cache row (s // block_size, s % block_size) and value[t] likewise; a
    negative slot is skipped. Follows the store kernel described in
    "Inference Engine Inside nano-vLLM", "Attention in nano-vLLM" (one
    program per token, skip on -1, row copy to slot * D) and the slot
    definition of "nano-vLLM Part 2 ...", section 2.2.

    key, value: [T, H_kv, D]; k_cache, v_cache: [N, block_size, H_kv, D], same
    storage dtype. Values are copied bit for bit.
    """
    block_size = k_cache.shape[1]
    for t in range(len(slot_mapping)):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        block, offset = divmod(s, block_size)
        k_cache[block, offset] = key[t]
        v_cache[block, offset] = value[t]


def widen_kv(x: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Exact fp64 values of stored cache elements: ``widen`` for fp32 / bf16,
    value(code) * scale for an fp8 cache."""
    if dtype == "fp8e4m3":
        return fp8.dequantize(x, scale)
    return widen(x, dtype)


def gather_history(cache, table_row, n: int, kv_head: int, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Copy the first ``n`` logical rows of one kv head of one sequence into a
    contiguous fp64 [n, D] buffer by walking its block table ("nano-vLLM
    Part 2 ...", section 2.2: logical page p // bs lives in physical block
    table[p // bs] at offset p % bs). ``scale`` is the per-tensor scale of an
    fp8 cache."""
    block_size = cache.shape[1]
    n_pages = -(-n // block_size)
    pages = [cache[int(table_row[j]), :, kv_head, :] for j in range(n_pages)]
    rows = np.concatenate(pages, axis=0)[:n] if pages else cache[:0, :, kv_head, :].reshape(0, cache.shape[-1])
    return widen_kv(rows, dtype, scale)


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q . K^T) V for one query vector q [D] over K, V [n, D]."""
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    w /= w.sum()
    return w @ V


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, dtype: str,
           seqs=None, kv_dtype=None, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Paged decode attention: one query per sequence over its whole cached
    history ("Inference Engine Inside nano-vLLM", "Attention in nano-vLLM",
    the flash_attn_with_kvcache branch; "From nano-vLLM to vLLM ...",
    section 11.2).

    q: [B, H_q, D] storage dtype; caches [N, bs, H_kv, D]; block_tables int
    [B, W]; context_lens int [B]. Returns fp64 [B, H_q, D]. With ``seqs`` (a
    list of sequence indices) only those rows are computed; the others are
    NaN. ``kv_dtype`` (default: ``dtype``) is the caches' storage type; for
    "fp8e4m3" the caches hold codes scaled by ``k_scale`` / ``v_scale``.
    """
    B, H_q, D = q.shape
    H_kv = k_cache.shape[2]
    G = H_q // H_kv
    out = np.full((B, H_q, D), np.nan)
    for b in (range(B) if seqs is None else seqs):
        n = int(context_lens[b])
        if n == 0:
            out[b] = 0.0
            continue
        qb = widen(q[b], dtype)
        for g in range(H_kv):
            K = gather_history(k_cache, block_tables[b], n, g, kv_dtype or dtype, k_scale)
            V = gather_history(v_cache, block_tables[b], n, g, kv_dtype or dtype, v_scale)
            for h in range(g * G, (g + 1) * G):  # query heads of kv head g: h // G == g
                out[b, h] = softmax_attention(qb[h], K, V, scale)
    return out


def prefill_varlen(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_tables, scale: float,
                   dtype: str, rows=None, k=None, v=None, kv_dtype=None, k_scale: float = 1.0,
                   v_scale: float = 1.0) -> np.ndarray:
    """Packed variable-length causal prefill ("Inference Engine Inside
    nano-vLLM", "Attention in nano-vLLM", the flash_attn_varlen_func branch;
    "nano-vLLM Part 2 ...", sections 2.5 and 4.1).

    Sequence i owns query rows cu_seqlens_q[i] .. cu_seqlens_q[i+1] - 1 and
    sees Lk = cu_seqlens_k[i+1] - cu_seqlens_k[i] keys. With a block table the
    keys are the first Lk logical rows of the paged cache; without one
    (``block_tables is None``) they are rows cu_seqlens_k[i] .. of the packed
    ``k``/``v`` [Tk, H_kv, D]. Query j (0-based within the sequence) sees keys
    0 .. (Lk - Lq) + j inclusive.

    q: [Tq, H_q, D]. Returns fp64 [Tq, H_q, D]; with ``rows`` (global query
    row indices) only those rows are computed and the others are NaN.
    ``kv_dtype`` / ``k_scale`` / ``v_scale`` describe a paged fp8 cache as in
    ``decode``.
    """
    Tq, H_q, D = q.shape
    H_kv = (k_cache if block_tables is not None else k).shape[-2]
    G = H_q // H_kv
    out = np.full((Tq, H_q, D), np.nan)
    want = None if rows is None else set(int(r) for r in rows)
    B = len(cu_seqlens_q) - 1
    for i in range(B):
        q0, q1 = int(cu_seqlens_q[i]), int(cu_seqlens_q[i + 1])
        Lq = q1 - q0
        Lk = int(cu_seqlens_k[i + 1]) - int(cu_seqlens_k[i])
        start = Lk - Lq
        js = [j for j in range(Lq) if want is None or (q0 + j) in want]
        if not js:
            continue
        for g in range(H_kv):
            if block_tables is not None:
                K = gather_history(k_cache, block_tables[i], Lk, g, kv_dtype or dtype, k_scale)
                V = gather_history(v_cache, block_tables[i], Lk, g, kv_dtype or dtype, v_scale)
            else:
                k0 = int(cu_seqlens_k[i])
                K = widen(k[k0:k0 + Lk, g, :], dtype)
                V = widen(v[k0:k0 + Lk, g, :], dtype)
            for h in range(g * G, (g + 1) * G):
                for j in js:
                    visible = start + j + 1
                    qv = widen(q[q0 + j, h], dtype)
                    out[q0 + j, h] = softmax_attention(qv, K[:visible], V[:visible], scale)
    return out
