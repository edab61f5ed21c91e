"""Seeded synthetic workloads for the paged-attention hot path.

This module builds the *inputs* of the three library calls: block tables,
context lengths, slot mappings, cumulative sequence lengths and the random
q/k/v/cache contents. It is shared by the tests, the benchmark and the
oracle-side checks, and on purpose holds none of the attention arithmetic
(no scatter, no gather, no softmax): it only produces the metadata a serving
engine's model runner would hand to the kernels, and random tensors.

The metadata rules follow the control-plane description on the pages:

* position -> slot: "nano-vLLM Part 2: Block Tables, KV Cache, and the Path
  to the GPU", section 2.2 (logical page = p // block_size, offset =
  p % block_size, slot = physical id * block_size + offset).
* the prefill slot loop with its first-page offset and last-page boundary:
  same page, section 2.2, and "From nano-vLLM to vLLM ...", section 8.2.
* cu_seqlens_q / cu_seqlens_k and positions for packed prefill: "Inference
  Engine Inside nano-vLLM" (junupark notes), "Prepare Prefill"; Part 2
  section 4.1.
* decode metadata (position len-1, context_len = len, slot in the last
  block): junupark notes "Prepare Decode"; Part 2 section 3.1.
* -1 padding of batched block tables: Part 2 section 3.2.
* a new block is claimed when len % block_size == 1: Part 2 section 3.1;
  "How vLLM Works" (the 17th token at block size 16).

Random values are N(0, 1) drawn in fp32 and rounded to the storage dtype
(round to nearest even for bf16). Rows of the pool that no sequence may read
hold NaN, so any over-read shows up as a non-finite output.

fp8 caches (``kv_dtype="fp8e4m3"``, next to bf16 queries and new rows) hold
one-byte E4M3 codes with a per-tensor scale for K and V: the history rows are
N(0, 1) / scale drawn in fp32, clamped to +-448 (torch's cast would turn the
rare tail beyond it into NaN) and cast to torch.float8_e4m3fn, so the
dequantised history again looks like N(0, 1); the NaN code 0x7F poisons the
rows nobody may read.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np

# bf16 quiet NaN bit pattern
BF16_NAN_BITS = np.uint16(0x7FC0)

DTYPES = ("f32", "bf16")


# ---------------------------------------------------------------------------
# Control-plane metadata (what the model runner serialises for the kernels)
# ---------------------------------------------------------------------------

def slot_of(block_table, pos: int, block_size: int) -> int:
    """Flattened cache slot of logical position ``pos`` of one sequence."""
    logical_page = pos // block_size
    offset = pos % block_size
    return int(block_table[logical_page]) * block_size + offset


def slots_for_range(block_table, start: int, end: int, block_size: int) -> list[int]:
    """Slots of positions [start, end), built page by page as the prefill
    runner does: the first page starts at ``start % block_size`` and the last
    page stops at ``end``."""
    out: list[int] = []
    if end <= start:
        return out
    start_block = start // block_size
    end_block = (end + block_size - 1) // block_size
    for i in range(start_block, end_block):
        base = int(block_table[i]) * block_size
        lo = base + (start % block_size if i == start_block else 0)
        hi = base + (end - i * block_size if i == end_block - 1 else block_size)
        out.extend(range(lo, hi))
    return out


def decode_slot(block_table, seq_len: int, block_size: int) -> int:
    """Slot of the token being decoded (position seq_len - 1), which lives in
    the last block of the table."""
    return int(block_table[-1]) * block_size + (seq_len - 1) % block_size


def needs_new_block(seq_len: int, block_size: int) -> bool:
    """True when the last token of a sequence of length ``seq_len`` is the
    first token of a fresh page."""
    return seq_len % block_size == 1 or block_size == 1


def cu_seqlens(lengths) -> np.ndarray:
    """Exclusive prefix sums [0, l0, l0+l1, ...] as int32."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out.astype(np.int32)


def prefill_layout(num_cached, num_scheduled):
    """Packed-prefill metadata for sequences with ``num_cached[i]`` cached
    tokens and ``num_scheduled[i]`` tokens computed this step.

    Returns (positions, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k).
    The visible key length of a sequence is cached + scheduled.
    """
    positions: list[int] = []
    lq, lk = [], []
    for c, s in zip(num_cached, num_scheduled):
        c, s = int(c), int(s)
        positions.extend(range(c, c + s))
        lq.append(s)
        lk.append(c + s)
    return (np.asarray(positions, dtype=np.int64), cu_seqlens(lq), cu_seqlens(lk),
            max(lq, default=0), max(lk, default=0))


def pad_block_tables(tables, width: int | None = None) -> np.ndarray:
    """Batch per-sequence block tables into an int32 [B, W] array, short rows
    padded with -1."""
    w = max((len(t) for t in tables), default=0) if width is None else width
    out = np.full((len(tables), max(w, 1)), -1, dtype=np.int32)
    for i, t in enumerate(tables):
        out[i, : len(t)] = np.asarray(t, dtype=np.int32)
    return out


def take_blocks(free_ids: list[int], n: int) -> list[int]:
    """Claim ``n`` ids from the front of a free list (in place)."""
    got = free_ids[:n]
    del free_ids[:n]
    return got


def num_blocks_for(n_tokens: int, block_size: int) -> int:
    return -(-int(n_tokens) // block_size)


# ---------------------------------------------------------------------------
# Storage-dtype helpers (input rounding only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); return the
    16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def nan_value(dtype: str):
    return BF16_NAN_BITS if dtype == "bf16" else np.float32(np.nan)


def storage_np_dtype(dtype: str):
    return {"bf16": np.uint16, "f32": np.float32, "fp8e4m3": np.uint8}[dtype]


FP8_NAN_CODE = np.uint8(0x7F)
# per-tensor scale of the fp8 workloads: N(0, 1) history maps to codes of
# N(0, 80^2), whose 5.6-sigma tail reaches the largest code (448)
FP8_SCALE = 0.0125


def fp8_codes(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    """E4M3 codes of N(0, 1) / scale samples, clamped to +-448 (torch's
    float8_e4m3fn cast)."""
    import torch
    x = np.clip(rng.standard_normal(shape, dtype=np.float32) / np.float32(scale), -448.0, 448.0)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def randn_storage(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------

@dataclass
class DecodeWorkload:
    """One decode step: every sequence scatters one new token then attends
    over its whole history (context_lens includes the new token)."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    num_blocks: int
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int32 [B, W], -1 padded
    slot_mapping: np.ndarray  # int32 [B], slot of position ctx-1
    scale: float
    seed: int = 0
    note: str = ""
    kv_dtype: str | None = None  # cache storage type when it differs from dtype ("fp8e4m3")
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elem_bytes(self) -> int:
        """Bytes per query / new-row / output element."""
        return 2 if self.dtype == "bf16" else 4

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def kv_elem_bytes(self) -> int:
        """Bytes per cache element."""
        return 1 if self.cache_dtype == "fp8e4m3" else self.elem_bytes

    def readable_positions(self, b: int) -> int:
        """Rows that hold history before the step (positions 0 .. ctx-2)."""
        return max(int(self.context_lens[b]) - 1, 0)

    def kv_bytes_logical(self) -> int:
        return int(self.context_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * self.head_dim * self.kv_elem_bytes

    def kv_bytes_unique(self) -> int:
        """K/V bytes counted once per distinct (physical block, offset) row."""
        rows = set()
        bs = self.block_size
        for b in range(self.num_seqs):
            n = int(self.context_lens[b])
            for j in range(num_blocks_for(n, bs)):
                bid = int(self.block_tables[b, j])
                hi = min(bs, n - j * bs)
                rows.add((bid, hi))
        # count each physical block once with the largest row count used
        best: dict[int, int] = {}
        for bid, hi in rows:
            best[bid] = max(best.get(bid, 0), hi)
        return sum(best.values()) * 2 * self.num_kv_heads * self.head_dim * self.kv_elem_bytes

    def algorithmic_bytes(self, unique: bool = False) -> int:
        """Bytes the decode step must move: K/V rows once per kv head, q in,
        o out, the table entries actually used and the context lengths."""
        kv = self.kv_bytes_unique() if unique else self.kv_bytes_logical()
        qo = 2 * self.num_seqs * self.num_q_heads * self.head_dim * self.elem_bytes
        tables = sum(num_blocks_for(int(n), self.block_size) for n in self.context_lens) * 4
        return kv + qo + tables + 4 * self.num_seqs

    def flops(self) -> int:
        ctx = int(self.context_lens.astype(np.int64).sum())
        return 4 * ctx * self.num_q_heads * self.head_dim

    def store_bytes(self) -> int:
        """K and V rows read from the inputs and written to the caches."""
        t = int((self.slot_mapping >= 0).sum())
        return (t * 2 * self.num_kv_heads * self.head_dim * (self.elem_bytes + self.kv_elem_bytes)
                + 4 * len(self.slot_mapping))


@dataclass
class PrefillWorkload:
    """One packed prefill step over prefix-cached sequences: the step's
    tokens are scattered first, then every query attends causally over the
    cached prefix plus the chunk, all read through the block tables."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    num_blocks: int
    num_cached: np.ndarray     # int64 [B]
    num_scheduled: np.ndarray  # int64 [B]
    block_tables: np.ndarray   # int32 [B, W]
    slot_mapping: np.ndarray   # int32 [Tq]
    positions: np.ndarray
    cu_seqlens_q: np.ndarray   # int32 [B+1]
    cu_seqlens_k: np.ndarray   # int32 [B+1]
    max_seqlen_q: int
    max_seqlen_k: int
    scale: float
    seed: int = 0
    shared_groups: list = field(default_factory=list)
    note: str = ""
    kv_dtype: str | None = None
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def num_seqs(self) -> int:
        return int(self.num_cached.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elem_bytes(self) -> int:
        """Bytes per query / new-row / output element."""
        return 2 if self.dtype == "bf16" else 4

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def kv_elem_bytes(self) -> int:
        """Bytes per cache element."""
        return 1 if self.cache_dtype == "fp8e4m3" else self.elem_bytes

    def flops(self) -> int:
        """QK^T + PV multiply-adds (2 flops each) over unmasked pairs only."""
        tot = 0
        for c, s in zip(self.num_cached, self.num_scheduled):
            c, s = int(c), int(s)
            tot += s * c + s * (s + 1) // 2
        return 4 * self.head_dim * self.num_q_heads * tot

    def store_bytes(self) -> int:
        """K and V rows read from the inputs and written to the caches."""
        t = int((self.slot_mapping >= 0).sum())
        return (t * 2 * self.num_kv_heads * self.head_dim * (self.elem_bytes + self.kv_elem_bytes)
                + 4 * len(self.slot_mapping))


# ---------------------------------------------------------------------------
# Named configurations
# ---------------------------------------------------------------------------

def _assign_tables(ctx_blocks, free_ids):
    return [take_blocks(free_ids, n) for n in ctx_blocks]


def _decode_from_tables(name, tables, ctx, bs, n_blocks, hq, hkv, d, dtype, width, seed, note=""):
    ctx = np.asarray(ctx, dtype=np.int32)
    bt = pad_block_tables(tables, width)
    slots = np.asarray([decode_slot(t, int(n), bs) if n > 0 else -1 for t, n in zip(tables, ctx)],
                       dtype=np.int32)
    return DecodeWorkload(name=name, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                          block_size=bs, num_blocks=n_blocks, context_lens=ctx, block_tables=bt,
                          slot_mapping=slots, scale=1.0 / math.sqrt(d), seed=seed, note=note)


def tiny_decode(seed: int = 0) -> DecodeWorkload:
    """4 sequences, context lengths 5/17/33/64 at block size 16 in a pool of
    32 blocks; tables are consecutive slices of a seeded permutation;
    H_q=4, H_kv=2, D=64, fp32."""
    rng = np.random.default_rng(seed)
    bs, n_blocks = 16, 32
    ctx = [5, 17, 33, 64]
    free = [int(x) for x in rng.permutation(n_blocks)]
    tables = _assign_tables([num_blocks_for(c, bs) for c in ctx], free)
    return _decode_from_tables("tiny-decode", tables, ctx, bs, n_blocks, 4, 2, 64, "f32", 4, seed,
                               note="fp32, scale 1/8")


def qwen3_0p6b_decode(seed: int = 0) -> DecodeWorkload:
    """Batch 64, H_q=16, H_kv=8, D=128, bf16, block size 256, shuffled pool
    of 4096 blocks, context lengths uniform in [128, 4096]."""
    rng = np.random.default_rng(seed)
    bs, n_blocks, B = 256, 4096, 64
    ctx = rng.integers(128, 4096, size=B, endpoint=True)
    free = [int(x) for x in rng.permutation(n_blocks)]
    tables = _assign_tables([num_blocks_for(c, bs) for c in ctx], free)
    return _decode_from_tables("qwen3-0.6b-decode", tables, ctx, bs, n_blocks, 16, 8, 128, "bf16",
                               16, seed)


def large_batch_decode(block_size: int = 16, seed: int = 0) -> DecodeWorkload:
    """Batch 512, H_q=32, H_kv=8, D=128, bf16, context lengths log-uniform in
    [512, 32768]; pool = needed blocks + 10 %, random placement."""
    rng = np.random.default_rng(seed)
    B = 512
    ctx = np.rint(np.exp(rng.uniform(math.log(512), math.log(32768), size=B))).astype(np.int64)
    ctx = np.clip(ctx, 512, 32768)
    need = [num_blocks_for(c, block_size) for c in ctx]
    n_blocks = int(math.ceil(1.1 * sum(need)))
    free = [int(x) for x in rng.permutation(n_blocks)]
    tables = _assign_tables(need, free)
    return _decode_from_tables(f"8b-decode-bs{block_size}", tables, ctx, block_size, n_blocks,
                               32, 8, 128, "bf16", 32768 // block_size, seed)


def long_context_decode(seed: int = 0) -> DecodeWorkload:
    """8 sequences at context 131072 (512 blocks of 256) whose first 64
    blocks (16384 tokens) are the same physical ids; H_q=64, H_kv=8,
    D=128, bf16."""
    rng = np.random.default_rng(seed)
    bs, B, ctx, shared = 256, 8, 131072, 64
    per_seq = ctx // bs
    n_blocks = shared + B * (per_seq - shared)
    free = [int(x) for x in rng.permutation(n_blocks)]
    prefix = take_blocks(free, shared)
    tables = [prefix + take_blocks(free, per_seq - shared) for _ in range(B)]
    return _decode_from_tables("long-context-decode", tables, [ctx] * B, bs, n_blocks, 64, 8, 128,
                               "bf16", per_seq, seed, note="16384-token shared prefix")


def custom_decode(ctx, *, block_size, num_q_heads, num_kv_heads, head_dim, dtype, seed=0,
                  spare_blocks=3, width=None, name="custom-decode", shared_prefix_blocks=0) -> DecodeWorkload:
    """Small decode workload of any shape; used for edge cases."""
    rng = np.random.default_rng(seed)
    ctx = [int(c) for c in ctx]
    # a shared block must hold history of every sharer, never its new token
    assert all(c > shared_prefix_blocks * block_size for c in ctx) or shared_prefix_blocks == 0
    need = [num_blocks_for(c, block_size) for c in ctx]
    private = [max(n - shared_prefix_blocks, 0) for n in need]
    n_blocks = shared_prefix_blocks + sum(private) + spare_blocks
    free = [int(x) for x in rng.permutation(n_blocks)]
    prefix = take_blocks(free, shared_prefix_blocks)
    tables = []
    for n, p in zip(need, private):
        tables.append((prefix[:n] if n <= shared_prefix_blocks else prefix) + take_blocks(free, p))
    w = width if width is not None else max(max(need, default=1), 1)
    return _decode_from_tables(name, tables, ctx, block_size, n_blocks, num_q_heads, num_kv_heads,
                               head_dim, dtype, w, seed)


def _prefill_from_parts(name, num_cached, num_sched, tables, bs, n_blocks, hq, hkv, d, dtype, seed,
                        groups=(), note=""):
    num_cached = np.asarray(num_cached, dtype=np.int64)
    num_sched = np.asarray(num_sched, dtype=np.int64)
    slots: list[int] = []
    for t, c, s in zip(tables, num_cached, num_sched):
        slots.extend(slots_for_range(t, int(c), int(c + s), bs))
    pos, cuq, cuk, mq, mk = prefill_layout(num_cached, num_sched)
    return PrefillWorkload(name=name, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                           block_size=bs, num_blocks=n_blocks, num_cached=num_cached,
                           num_scheduled=num_sched, block_tables=pad_block_tables(tables),
                           slot_mapping=np.asarray(slots, dtype=np.int32), positions=pos,
                           cu_seqlens_q=cuq, cu_seqlens_k=cuk, max_seqlen_q=mq, max_seqlen_k=mk,
                           scale=1.0 / math.sqrt(d), seed=seed, shared_groups=list(groups), note=note)


def chunked_prefill(seed: int = 0, total_q: int = 16384, num_seqs: int = 24, group: int = 4,
                    block_size: int = 256, max_prefix_blocks: int = 32, num_q_heads: int = 32,
                    num_kv_heads: int = 8, head_dim: int = 128, dtype: str = "bf16") -> PrefillWorkload:
    """16384 packed query tokens over 24 sequences in 6 groups of 4. Each
    group shares a cached prefix of 256*U{0..32} tokens through identical
    block ids; the query lengths are a seeded composition of 16384 into 24
    positive parts; sequence 0 also has 1..255 private cached tokens so its
    chunk starts inside a block."""
    rng = np.random.default_rng(seed)
    bs = block_size
    n_groups = num_seqs // group
    prefix_blocks = [int(rng.integers(0, max_prefix_blocks, endpoint=True)) for _ in range(n_groups)]
    cuts = np.sort(rng.choice(np.arange(1, total_q), size=num_seqs - 1, replace=False))
    lq = np.diff(np.concatenate([[0], cuts, [total_q]])).astype(np.int64)
    extra = int(rng.integers(1, bs))  # private cached tokens of sequence 0
    cached = []
    for i in range(num_seqs):
        cached.append(prefix_blocks[i // group] * bs + (extra if i == 0 else 0))
    need_private = []
    for i in range(num_seqs):
        total = num_blocks_for(cached[i] + lq[i], bs)
        need_private.append(total - prefix_blocks[i // group])
    needed = sum(prefix_blocks) + sum(need_private)
    n_blocks = int(math.ceil(1.1 * needed))
    free = [int(x) for x in rng.permutation(n_blocks)]
    prefixes = [take_blocks(free, n) for n in prefix_blocks]
    tables = [prefixes[i // group] + take_blocks(free, need_private[i]) for i in range(num_seqs)]
    groups = [list(range(g * group, (g + 1) * group)) for g in range(n_groups)]
    return _prefill_from_parts("chunked-prefill", cached, lq, tables, bs, n_blocks, num_q_heads,
                               num_kv_heads, head_dim, dtype, seed, groups,
                               note=f"prefix blocks per group {prefix_blocks}, seq0 extra {extra}")


def custom_prefill(num_cached, num_scheduled, *, block_size, num_q_heads, num_kv_heads, head_dim,
                   dtype, seed=0, spare_blocks=3, name="custom-prefill",
                   shared_prefix_blocks=0) -> PrefillWorkload:
    """Small prefill workload of any shape. With ``shared_prefix_blocks`` > 0
    every sequence's first blocks are the same physical ids."""
    rng = np.random.default_rng(seed)
    num_cached = [int(c) for c in num_cached]
    num_scheduled = [int(s) for s in num_scheduled]
    # shared blocks must be wholly cached for every sharer
    assert all(c >= shared_prefix_blocks * block_size for c in num_cached)
    need = [num_blocks_for(c + s, block_size) for c, s in zip(num_cached, num_scheduled)]
    private = [max(n - shared_prefix_blocks, 0) for n in need]
    n_blocks = shared_prefix_blocks + sum(private) + spare_blocks
    free = [int(x) for x in rng.permutation(n_blocks)]
    prefix = take_blocks(free, shared_prefix_blocks)
    tables = [(prefix[:n] if n <= shared_prefix_blocks else prefix) + take_blocks(free, p)
              for n, p in zip(need, private)]
    return _prefill_from_parts(name, num_cached, num_scheduled, tables, block_size, n_blocks,
                               num_q_heads, num_kv_heads, head_dim, dtype, seed)


DECODE_CONFIGS = {
    "tiny-decode": tiny_decode,
    "qwen3-0.6b-decode": qwen3_0p6b_decode,
    "8b-decode-bs16": lambda seed=0: large_batch_decode(16, seed),
    "8b-decode-bs256": lambda seed=0: large_batch_decode(256, seed),
    "long-context-decode": long_context_decode,
}


def with_fp8_cache(w, k_scale: float = FP8_SCALE, v_scale: float = FP8_SCALE):
    """The same workload over E4M3 caches (bf16 queries and new rows)."""
    assert w.dtype == "bf16", "fp8 caches pair with bf16 queries"
    return dataclasses.replace(w, name=w.name + "-fp8", kv_dtype="fp8e4m3", k_scale=k_scale,
                               v_scale=v_scale)


DECODE_CONFIGS.update({
    "qwen3-0.6b-decode-fp8": lambda seed=0: with_fp8_cache(qwen3_0p6b_decode(seed)),
    "long-context-decode-fp8": lambda seed=0: with_fp8_cache(long_context_decode(seed)),
})

PREFILL_CONFIGS = {"chunked-prefill": chunked_prefill,
                   "chunked-prefill-fp8": lambda seed=0: with_fp8_cache(chunked_prefill(seed))}


# ---------------------------------------------------------------------------
# Tensor contents
# ---------------------------------------------------------------------------

def _readable_rows_decode(w: DecodeWorkload):
    """(block id, number of leading rows holding history) per sequence block."""
    bs = w.block_size
    out = {}
    for b in range(w.num_seqs):
        n = w.readable_positions(b)
        nb_tab = num_blocks_for(int(w.context_lens[b]), bs)
        for j in range(nb_tab):
            bid = int(w.block_tables[b, j])
            rows = min(max(n - j * bs, 0), bs)
            out[bid] = max(out.get(bid, 0), rows)
    return out


def _readable_rows_prefill(w: PrefillWorkload):
    bs = w.block_size
    out = {}
    for b in range(w.num_seqs):
        n = int(w.num_cached[b])
        nb_tab = num_blocks_for(int(w.num_cached[b] + w.num_scheduled[b]), bs)
        for j in range(nb_tab):
            bid = int(w.block_tables[b, j])
            rows = min(max(n - j * bs, 0), bs)
            out[bid] = max(out.get(bid, 0), rows)
    return out


def readable_rows(w) -> dict:
    """Map physical block id -> count of leading rows that hold cached K/V
    before the step. Every other row of the pool is poisoned with NaN."""
    return _readable_rows_decode(w) if isinstance(w, DecodeWorkload) else _readable_rows_prefill(w)


def make_host_tensors(w, seed: int | None = None) -> dict:
    """Host (numpy) tensors for small workloads.

    Returns ``k_cache``/``v_cache`` [N, bs, H_kv, D] in storage dtype (uint16
    bit patterns for bf16), ``qkv`` [T, (H_q + 2 H_kv) D] from which ``q``,
    ``k`` and ``v`` are row-strided views as a fused QKV projection would
    produce them."""
    rng = np.random.default_rng(w.seed * 7919 + 17 if seed is None else seed)
    h, hq, d, bs = w.num_kv_heads, w.num_q_heads, w.head_dim, w.block_size
    fp8 = w.cache_dtype == "fp8e4m3"
    nanv = FP8_NAN_CODE if fp8 else nan_value(w.dtype)
    k_cache = np.full((w.num_blocks, bs, h, d), nanv, dtype=storage_np_dtype(w.cache_dtype))
    v_cache = np.full_like(k_cache, nanv)
    for bid, rows in sorted(readable_rows(w).items()):
        if rows and fp8:
            k_cache[bid, :rows] = fp8_codes(rng, (rows, h, d), w.k_scale)
            v_cache[bid, :rows] = fp8_codes(rng, (rows, h, d), w.v_scale)
        elif rows:
            k_cache[bid, :rows] = randn_storage(rng, (rows, h, d), w.dtype)
            v_cache[bid, :rows] = randn_storage(rng, (rows, h, d), w.dtype)
    t = w.num_seqs if isinstance(w, DecodeWorkload) else w.total_q
    qkv = randn_storage(rng, (t, (hq + 2 * h) * d), w.dtype)
    q = qkv[:, : hq * d].reshape(t, hq, d)
    k = qkv[:, hq * d:(hq + h) * d].reshape(t, h, d)
    v = qkv[:, (hq + h) * d:].reshape(t, h, d)
    return {"k_cache": k_cache, "v_cache": v_cache, "qkv": qkv, "q": q, "k": k, "v": v}


def make_device_tensors(w, device="cuda", seed: int | None = None, chunk_blocks: int | None = None):
    """Device (torch) tensors for any workload, generated on the device with a
    seeded torch generator so multi-GB pools never pass through the host.

    Same layout as :func:`make_host_tensors`; bf16 tensors have dtype
    torch.bfloat16, fp32 ones torch.float32, fp8 caches torch.uint8."""
    import torch

    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    fp8 = w.cache_dtype == "fp8e4m3"
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 7919 + 17 if seed is None else seed)
    h, hq, d, bs = w.num_kv_heads, w.num_q_heads, w.head_dim, w.block_size
    n = w.num_blocks
    k_cache = torch.empty((n, bs, h, d), dtype=torch.uint8 if fp8 else tdt, device=device)
    v_cache = torch.empty_like(k_cache)
    row = bs * h * d
    step = chunk_blocks or max(1, (1 << 28) // row)
    for cache, sc in ((k_cache, w.k_scale), (v_cache, w.v_scale)):
        flat = cache.view(n, row)
        for s in range(0, n, step):
            e = min(n, s + step)
            x = torch.randn((e - s, row), generator=g, device=device, dtype=torch.float32)
            if fp8:
                flat[s:e].copy_((x / sc).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8))
            else:
                flat[s:e].copy_(x)
    # poison every row that holds no history
    rr = readable_rows(w)
    keep = np.zeros(n, dtype=bool)
    partial_ids, partial_rows = [], []
    for bid, rows in rr.items():
        if rows == bs:
            keep[bid] = True
        elif rows > 0:
            keep[bid] = True
            partial_ids.append(bid)
            partial_rows.append(rows)
    dead = torch.from_numpy(np.nonzero(~keep)[0]).to(device)
    nanv = int(FP8_NAN_CODE) if fp8 else float("nan")
    for cache in (k_cache, v_cache):
        if dead.numel():
            cache.index_fill_(0, dead, nanv)
        for bid, rows in zip(partial_ids, partial_rows):
            cache[bid, rows:] = nanv
    t = w.num_seqs if isinstance(w, DecodeWorkload) else w.total_q
    qkv = torch.randn((t, (hq + 2 * h) * d), generator=g, device=device, dtype=torch.float32).to(tdt)
    q = qkv[:, : hq * d].view(t, hq, d)
    k = qkv[:, hq * d:(hq + h) * d].view(t, h, d)
    v = qkv[:, (hq + h) * d:].view(t, h, d)
    return {"k_cache": k_cache, "v_cache": v_cache, "qkv": qkv, "q": q, "k": k, "v": v}
