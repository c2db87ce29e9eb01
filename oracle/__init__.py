"""CPU oracle of the CSA/HCA compressed-attention hot path (fp64, numpy).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and
the bench's CPU-baseline leg may import or run anything in this package; the
library path never calls it and fails when its HIP build is missing.  It shares
no code with the HIP path: the two meet only at the seeded inputs of the
`workloads` package.

Modules
  codecs    storage roundings (fp32, bf16, OCP e4m3) from the formats' definitions
  method    the method's steps: compressor, visibility, lightning indexer, top-k,
            attention over entries plus the raw window, heads back to model width
  pipeline  a workload layer end to end (caches from streams, decode rows)

Parity status: every function is pinned by tests/test_oracle_*.py to closed
forms, invariants of the method, library routines or brute force; the pages
print no worked example, so no pin comes from printed values.
"""
from . import codecs, method, pipeline  # noqa: F401
