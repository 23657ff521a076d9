"""Seeded synthetic inputs (generator and workloads) for the int4 routed-expert hot path."""
from . import gen, workloads  # noqa: F401
