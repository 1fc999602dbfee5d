"""Float64 CPU oracle for paged-KV GQA decode (split-K) and MLA causal paged prefill.

TEST INFRASTRUCTURE ONLY. This package is imported, called or run only by
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``. The HIP library and its Python binding never import it, and it
imports nothing from them: the two sides share no code, only the seeded inputs.

Everything is plain numpy in float64 (library matmuls as single steps, no
blocking or fusion beyond what each definition states). Inputs are upcast
exactly (bf16 -> fp32 -> fp64) before any arithmetic.

Every function here is pinned by tests in ``tests/test_oracle.py`` against
values it does not compute itself (dense brute force through library
softmax / logsumexp / SDPA, closed forms, invariants, hand-worked fixtures).
"""
from .decode import (TOKEN_MAJOR, XPACKED, decode, decode_partials, gather_sequence,
                     partition_ranges, reduce_partials)
from .mla import mla_prefill

__all__ = ["TOKEN_MAJOR", "XPACKED", "decode", "decode_partials", "gather_sequence",
           "partition_ranges", "reduce_partials", "mla_prefill"]
