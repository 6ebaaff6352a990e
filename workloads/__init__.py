"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke run."""
from .generators import (CONFIG_NAMES, Layer, Workload, f32_to_bf16_bits, make, normal_bf16_bits,
                         normal_f16, random_small, shell_coords, shell_workload, uniform_coords,
                         uniform_workload)

__all__ = ["CONFIG_NAMES", "Layer", "Workload", "f32_to_bf16_bits", "make", "normal_bf16_bits",
           "normal_f16", "random_small", "shell_coords", "shell_workload", "uniform_coords",
           "uniform_workload"]
