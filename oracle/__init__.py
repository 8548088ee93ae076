"""CPU oracle for the mixed-batch paged attention step -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and `bench.py`'s CPU-baseline leg may import this package. The product
(the HIP library and its Python binding) never imports it and shares no code with it; if the HIP extension is
missing, the product fails loudly instead of falling back here.

Contents:
  attention  -- fp64 exact attention (definition), paged gather, append, explicit-mask brute force
  scheduler  -- FIFO / token-budget / page-allocation reference of the step metadata
  reference  -- workload-level expected rows and cache pages for the synthetic workloads

Every function is pinned by the `-m "not gpu"` tests against values the pages print, closed forms, brute force and
independent library routines (tests/test_oracle_pins.py, tests/test_oracle_mutants.py).
"""
from . import attention, scheduler, reference  # noqa: F401
