"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the benchmark."""
from .gen import CONFIGS, Workload, make, bf16_round, bf16_decode, decode, algorithmic_bytes

__all__ = ["CONFIGS", "Workload", "make", "bf16_round", "bf16_decode", "decode",
           "algorithmic_bytes"]
