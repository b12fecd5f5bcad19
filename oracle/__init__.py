"""Reference oracle for mask-aware attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct CPU (numpy float64) implementation of what the
compressed-mask attention path computes.  It materialises the full dense
visibility mask and evaluates softmax attention over every key, exactly as the
definitions read; it shares no code with the HIP library and never imports it.

Only the tests, the smoke check of the graft entry point and the CPU-baseline
leg of the benchmark may import this package.  The product path must never call
it (there is no CPU fallback).

Modules:
  masks      -- mask families -> dense visibility (the definitions)
  encode     -- dense visibility -> canonical interval / bitmap / list encodings,
                exact tile states, compact tile lists and the longest-first order
  attention  -- dense masked softmax attention in float64 (vectorised per row
                chunk), a per-row sampler, a pure-Python brute force for tiny
                shapes, attention over exactly the listed cells for the
                selected-key family, and the analytic gradient (dQ, dK, dV)

Every function in this package has a pin in tests/test_oracle_*.py (values the
pages fix, closed forms, invariants, library reductions, brute force); none is
"parity unpinned".
"""

from . import masks, encode, attention  # noqa: F401
