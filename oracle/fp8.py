"""fp8 (E4M3) KV-cache storage for the oracle: value table, encoder, and the
quantising store.

TEST INFRASTRUCTURE (like the rest of ``oracle``): only the tests,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may use it.

The pages size a cache element by its data type and list fp8 at one byte per
element ("nano-vLLM Part 2: Block Tables, KV Cache, and the Path to the
GPU", section 1, the KV-cache shape with its dtype factor) but say nothing
about the format or how values get there. Readings taken here (each is also
listed in the design notes of the repository):

* format: the OCP 8-bit floating point E4M3 encoding ("E4M3FN"): sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent 0 holds the
  subnormals m/8 * 2^-6; exponent 15 with mantissa 7 is NaN; there is no
  infinity; the largest finite magnitude is 448.
* scaling: one fp32 scale per cache tensor (k_scale for K, v_scale for V).
  A stored code c stands for value(c) * scale.
* quantising a value x (held in the input's storage type) for the cache:
  the finite E4M3 value nearest to the real number y = |x| / scale (scale as
  the fp32 value the library receives), ties to the code with an even
  mantissa; magnitudes of 448 and beyond (infinities included) saturate to
  448; a NaN gives the NaN code. The code's sign bit is x's sign bit (so -0
  and a negative NaN keep it; the sign of a NaN quotient is left to no
  hardware). This is the plain reading of "store x / scale as E4M3": the
  exact quotient is rounded once, with no intermediate rounding of the
  quotient to some working precision.
"""
from __future__ import annotations

import numpy as np


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code, straight from the field definition."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


# fp64 value of each of the 256 codes
E4M3_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)

# non-negative finite codes (0x00 .. 0x7E) and their values, in increasing order
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = E4M3_VALUES[:0x7F]


def decode(codes) -> np.ndarray:
    """Codes (uint8 array) to fp64 values."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def encode_one(y: float) -> int:
    """Nearest E4M3 code to the real number y: ties go to the even mantissa,
    magnitudes past 448 saturate, NaN stays NaN with its sign."""
    neg = bool(np.signbit(y))
    if np.isnan(y):
        return 0xFF if neg else 0x7F
    a = abs(float(y))
    if a >= 448.0:
        code = 0x7E
    else:
        # brute force over the 127 non-negative finite values
        dist = np.abs(_POS_VALUES - a)
        best = dist.min()
        cands = _POS_CODES[dist == best]
        if len(cands) == 1:
            code = int(cands[0])
        else:  # exactly half-way between two neighbours: the even mantissa wins
            code = int([c for c in cands if c % 2 == 0][0])
    return code | (0x80 if neg else 0)


def encode(y) -> np.ndarray:
    """``encode_one`` over an array, as a sorted search: the two finite
    values that bracket |y| are found with ``np.searchsorted`` over the
    increasing non-negative values, the nearer one wins and a tie goes to
    the even code (neighbouring codes alternate parity). Returns uint8."""
    y = np.asarray(y, dtype=np.float64)
    neg = np.signbit(y)
    nan = np.isnan(y)
    a = np.where(nan, 0.0, np.minimum(np.abs(y), 448.0))   # 448 and beyond saturate
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, 0x7E)  # first value >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(nan, 0x7F, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize(x64: np.ndarray, scale: float) -> np.ndarray:
    """Codes for exact input values ``x64`` (widened from their storage type)
    under a per-tensor scale: the finite E4M3 value nearest the real quotient
    y = |x| / s with s = fp32(scale), ties to the even mantissa, 448 and
    beyond saturating, NaN giving the NaN code, with x's sign bit.

    No quotient is formed. With v_0 < v_1 < ... < v_126 = 448 the finite
    non-negative E4M3 values, y lies between v_lo and v_hi = the first value
    with v * s >= |x|, and the half-way point m = (v_lo + v_hi) / 2 decides:
    |x| < m * s picks lo, |x| > m * s picks hi, equality is a tie. Every v
    and m has at most 5 significant bits and s at most 24, so v * s and m * s
    are exact in fp64, as is |x|: each comparison is decided exactly."""
    s = float(np.float32(scale))
    x = np.asarray(x64, dtype=np.float64)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.abs(x))
    thresholds = _POS_VALUES * s                                        # v_k * s, exact
    hi = np.clip(np.searchsorted(thresholds, a, side="left"), 0, 0x7E)  # first v_k * s >= |x|
    lo = np.maximum(hi - 1, 0)
    mid_s = (_POS_VALUES[lo] + _POS_VALUES[hi]) / 2 * s                 # m * s, exact
    code = np.where(a < mid_s, lo, np.where(a > mid_s, hi, np.where(lo & 1, hi, lo)))
    code = np.where(a >= 448.0 * s, 0x7E, code)                         # y >= 448 saturates
    code = np.where(np.isnan(x), 0x7F, code)                            # NaN keeps a NaN code
    sign = np.where(np.signbit(x), 0x80, 0)
    return (code | sign).astype(np.uint8)


def dequantize(codes, scale: float) -> np.ndarray:
    """fp64 values of cache codes: value(code) * scale (exact in fp64: a
    4-bit significand times a 24-bit one)."""
    return decode(codes) * float(np.float32(scale))


def store_kvcache(key64, value64, k_cache, v_cache, slot_mapping, k_scale: float,
                  v_scale: float) -> None:
    """Quantising KV scatter, in place: for token t with slot s >= 0, the
    cache row (s // block_size, s % block_size) receives the codes of
    key[t] / k_scale and value[t] / v_scale; negative slots are skipped (the
    same slot rule as the plain store, "Inference Engine Inside nano-vLLM",
    "Attention in nano-vLLM").

    key64, value64: exact fp64 values [T, H_kv, D]; caches: uint8 codes
    [N, block_size, H_kv, D].
    """
    block_size = k_cache.shape[1]
    for t in range(len(slot_mapping)):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        block, offset = divmod(s, block_size)
        k_cache[block, offset] = quantize(key64[t], k_scale)
        v_cache[block, offset] = quantize(value64[t], v_scale)
