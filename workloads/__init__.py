"""Seeded synthetic workloads for the DFlash draft-and-accept path.

This package only describes shapes and draws seeded random inputs.  It holds
none of the method's arithmetic, so both the HIP path and the CPU oracle can
consume what it produces.
"""
from .configs import DFlashConfig, Workload, WORKLOADS, get_workload  # noqa: F401
