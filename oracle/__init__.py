"""CPU oracle for the paged KV cache with RoPE-at-insert injection.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (no headers, helpers, tables or constants); the two meet only in
the seeded input generators of ``workloads/``, which hold none of the method's
arithmetic.

Every function is a plain, slow statement of what the pages define, in numpy,
with float64 wherever the pages leave precision open.  Sources, cited by page
title and section:

* [InferScale]      "InferScale: GPU-Native KV Injection for Personalized LLM
                     Serving" -- background on RoPE and paged attention (§2),
                     pre-RoPE key capture and composition (§3, §3.3), the
                     per-fact storage cost, chunked RoPE / Theorem 1 (§5.1),
                     the bf16 fidelity test (§6, Table 7).
* [KV essay]        "LLM Inference: KV Caching" -- sections "First, what K and
                     V are", "What the cache costs", "Paged attention".
* [Inside engines]  "Inside LLM Inference Engines: KV Caching, PagedAttention,
                     and Continuous Batching" -- sections "The KV Cache:
                     Mathematical Formulation & Memory Footprint",
                     "PagedAttention: Virtual Memory for LLM Generation",
                     "Continuous Batching".
* [KV management]   "Latency Optimization › KV Cache Management" -- the KV-size
                     formula and the paged-allocation paragraphs.

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against printed values, closed forms, invariants or brute force (see
``tests/test_oracle_*.py``).  No function is "parity unpinned".
"""

from . import kv_size, numerics, layout, allocator, rope, inject, attention  # noqa: F401
