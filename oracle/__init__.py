"""CPU oracle for the quantized paged KV store and its decode attention.

TEST INFRASTRUCTURE ONLY. Plain, slow, float64 NumPy code written from the
pages' description of the method; it shares no code with the HIP library and
imports nothing from it. Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import it. The product path never
calls it.

Modules:
  formats    - E4M3FN / E5M2 / E2M1 / E8M0 value tables, RNE encoders
  quantize   - FP8 per-tensor, FP4 block-16 (E8M0), NVFP4 two-level quantizers
  paged      - byte layout of the paged cache, store and gather
  attention  - paged decode attention by definition
  accounting - bytes per token and capacity ratios

Parity status: every function is pinned by tests under ``tests/``
(test_oracle_*.py) against values the pages print, closed forms, library
routines or brute force; see each test's docstring.
"""
from . import accounting, attention, formats, paged, quantize  # noqa: F401
