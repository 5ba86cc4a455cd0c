"""CPU oracle for head-wise adaptive KV-cache eviction.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 NumPy
statement of what the eviction path computes, written from the pages'
definitions.  It exists to check the HIP library; the library never imports,
links or calls it, and it shares no code with the library.  Only the test
suite, the package smoke check and the benchmark's CPU-baseline leg may use
it.

Modules
  scoring     observation-window scores: Ada-KV/SnapKV, LAVa, CriticalKV, LaProx
  allocation  Ada-KV budget allocation with the safeguard, per-head top-k,
              LAVa entropy layer budgets, CriticalKV two-stage selection,
              the model-wide top-k of LaProx, the floor-then-global reading
              of the safeguard, the StreamingLLM baseline, the LAVa
              online-prefill budget schedule
  cache       compaction into the retained cache and decode attention
  bounds      the pages' loss bounds and the renormalisation identity

Parity status: every function is pinned by tests/test_oracle_*.py against
closed forms, library routines or brute force, except where a docstring says
"parity unpinned".
"""
from . import scoring, allocation, cache, bounds  # noqa: F401
