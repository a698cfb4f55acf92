"""Seeded synthetic workloads for the LeapQuant decode path.

This package holds the five workload shapes and the seeded input generators.
It is the only code that both the CPU oracle's tests and the HIP path's
callers use; it contains none of the method's arithmetic (no recurrence, no
quantizer), only the drawing of random inputs.
"""
from .configs import HEADLINE, WORKLOADS, WorkloadConfig, get_workload
from .generators import initial_state, token_inputs, sample_states

__all__ = ["HEADLINE", "WORKLOADS", "WorkloadConfig", "get_workload", "initial_state",
           "token_inputs", "sample_states"]
