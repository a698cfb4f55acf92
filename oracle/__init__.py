"""CPU oracle for the LeapQuant decode path (test infrastructure only).

Importable only by the test suite, the smoke check and the benchmark's
CPU-baseline leg.  Nothing in the product package imports it.
"""
from . import leapquant_oracle  # noqa: F401
