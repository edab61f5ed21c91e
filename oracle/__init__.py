"""fp64 CPU oracle for the paged-attention hot path (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this package; the library never imports it.
"""
from . import fp8  # noqa: F401
from .paged_attention import (  # noqa: F401
    decode,
    gather_history,
    prefill_varlen,
    softmax_attention,
    store_kvcache,
    widen,
    widen_kv,
)
