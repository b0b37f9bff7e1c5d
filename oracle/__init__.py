"""fp64 CPU oracle for the gated linear-attention recurrence.

TEST INFRASTRUCTURE ONLY: imported by tests/, the package smoke check and
the benchmark's CPU-baseline leg, never by the HIP product path.

  gla_oracle  - numpy fp64 token-by-token recurrence (forward, decode step)
  c_oracle    - independent C fp64 recurrence with OpenMP (timed baseline)

Parity status: every function here is pinned by tests/test_oracle_pins.py
(closed forms, brute force, exact rationals, invariants) and by
tests/test_oracle_mutants.py (planted mistakes must fail a pin).
"""
