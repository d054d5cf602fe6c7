"""CPU oracle for the weightless linear -- test infrastructure, not product code.

A plain, slow fp64 implementation of what the path computes, written from the
pages' description of the theta bundle.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import it; the GPU library never
does, and the oracle shares no code with the library (its only common
dependency is the seeded input generator in ``synth``).

Modules:
  forward    -- the factored forward y = s*(W0 x) + U (V^T x), the explicit
                form with W_eff = diag(s) W0 + U V^T, stacked calls
  decompose  -- band-mean shared block, per-row scale, truncated-SVD delta,
                relative Frobenius error (the analytic decomposition)
  sizes      -- analytic theta-bundle and dense byte counts
  bf16       -- round-to-nearest-even to bfloat16, written independently of
                the library and of torch
  compare    -- the parity tolerance (max |d| and per-token-row relative L2)
  workload   -- the oracle's view of a synthetic workload's bundle

Parity pinning: every function here is pinned by a CPU test against something
other than itself (closed forms, the pages' printed numbers, brute force on
tiny inputs, mathematical identities); see tests/test_oracle_*.py.
"""
