"""Seeded synthetic inputs for the paged decode workloads (no method arithmetic)."""
from .synthetic import DecodeWorkload, workload  # noqa: F401
