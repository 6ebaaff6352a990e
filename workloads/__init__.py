"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke run."""
from .generators import (CONFIG_NAMES, Layer, Workload, make, normal_f16, random_small,
                         shell_coords, shell_workload, uniform_coords, uniform_workload)

__all__ = ["CONFIG_NAMES", "Layer", "Workload", "make", "normal_f16", "random_small",
           "shell_coords", "shell_workload", "uniform_coords", "uniform_workload"]
