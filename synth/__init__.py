"""Seeded synthetic workloads shared by the oracle-side tests and the benchmark."""
from .gen import WORKLOADS, Workload, make_inputs, random_case, rng_for, workload_inputs, prefill_slots  # noqa: F401
