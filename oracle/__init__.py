"""CPU fp64 oracle for the multi-LoRA adapter execution unit.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  The product library never
imports, links or calls it, and this package imports nothing from the product.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(hand-worked examples, closed forms, exact rational arithmetic, library
special cases, invariants).  Nothing here is "parity unpinned".
"""
from .oracle import (  # noqa: F401
    BASE_ONLY, MODE_NONE, MODE_FUSED, MODE_SEPARATE,
    POLICY_AUTO, POLICY_FUSED, POLICY_SEPARATE,
    load, route, apply, to_f64,
)
