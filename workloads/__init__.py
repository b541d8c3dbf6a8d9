"""Seeded synthetic inputs for the paged decode workloads (no method arithmetic)."""
from .synthetic import DecodeWorkload, workload, poison_unused  # noqa: F401
