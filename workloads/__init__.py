"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check."""
from .synth import WORKLOADS, Workload, calibration_queries, decode_queries, keys, round_to, scaled, values

__all__ = ["WORKLOADS", "Workload", "calibration_queries", "decode_queries", "keys", "round_to", "scaled", "values"]
