"""Test-side helpers: host/device conversion of storage dtypes and the parity
gates. No attention arithmetic lives here."""
from __future__ import annotations

import numpy as np

# Attention tolerances (max-abs against the fp64 oracle): fp32 inputs with
# fp32 accumulation, and bf16 inputs with fp32 accumulation.
TOL = {"f32": 1e-5, "bf16": 1.5e-2}


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_host(t, dtype: str) -> np.ndarray:
    """Device tensor -> numpy array in storage form (uint16 bits for bf16)."""
    import torch
    if dtype == "bf16":
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().contiguous().cpu().numpy()


def widen_host(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (via fp32), returned as fp64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def assert_attention_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """Max-abs gate against the fp64 oracle. For bf16 outputs whose reference
    magnitude is >= 4 the output rounding step alone (2^-9 * 2^floor(log2|o|)
    = 1.5625e-2) can exceed 1.5e-2; such elements must instead be within one
    bf16 ulp of the correctly rounded reference."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    tol = TOL[dtype]
    bad = err > tol
    if dtype == "bf16" and bad.any():
        big = np.abs(ref) >= 4.0
        if np.all(big[bad]):
            r = bf16_rne(ref[bad])
            ulp = np.ldexp(1.0, np.floor(np.log2(np.abs(r))).astype(int) - 7)
            assert np.all(np.abs(got[bad] - r) <= ulp), f"{what}: >1 ulp where |ref|>=4"
            return float(err[~bad].max(initial=0.0))
    assert not bad.any(), f"{what}: max abs err {err.max():.3e} > {tol} at {np.argwhere(bad)[:5].tolist()}"
    return float(err.max(initial=0.0))
