"""Seeded synthetic inputs and workload shapes (no arithmetic of the method)."""
from . import gen, workloads  # noqa: F401
