"""Seeded synthetic inputs (values and workload structure) shared by the oracle and HIP harnesses.

Holds no arithmetic of the method itself; see ``values`` and ``workloads``.
"""
from . import values, workloads  # noqa: F401
